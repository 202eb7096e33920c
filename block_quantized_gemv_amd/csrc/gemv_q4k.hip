// q4_K x q8_0 GEMV kernels for gfx950.
//
// The decode-step matvec over block-quantized weights: the weight stream is
// read once, in 16-byte non-temporal loads, while the q8_0 activation sits
// in LDS.  Integer 4-way dot products (v_dot4_i32_i8) form the exact int32
// sum of each 32-value sub-block, the f16 d/dmin fixup is applied in f64
// and each row is reduced across its lanes with DPP/swizzle steps in a fixed
// order.  This is the MMVQ "dp4a x q8_0" decode kernel of '07 · R3 —
// Small-model per-token overhead' (§1) redesigned for wave64/CDNA4; that
// page describes it only by name.
//
// Lane work: a super-block (144 B = 16 B header + 128 B nibbles) is shared
// by 4 lanes; lane j takes nibble chunk j (32 bytes = sub-blocks 2j, 2j+1:
// low nibbles pair with q8_0 block 8sb+2j, high nibbles with 8sb+2j+1) plus
// the 16-byte header, which the 4 lanes read as one broadcast.
#include "common.hpp"
#include "launch.hpp"

namespace mq {

struct SBLoad {
    u32x4 hdr, qa, qb;
};

__device__ __forceinline__ void load_sb(const uint8_t* __restrict__ blk, int j, SBLoad& L) {
    L.hdr = __builtin_nontemporal_load((const u32x4*)blk);
    L.qa = __builtin_nontemporal_load((const u32x4*)(blk + 16 + 32 * j));
    L.qb = __builtin_nontemporal_load((const u32x4*)(blk + 32 + 32 * j));
}

// Scales and mins of sub-blocks 2j and 2j+1 from the header.  Bytes s[0..3]
// are hdr.y, s[4..7] hdr.z, s[8..11] hdr.w; sub-blocks j' < 4 keep sc and m
// in the low six bits of s[j'] and s[j'+4]; j' >= 4 take their low four bits
// from the nibbles of s[j'+4] and their top two from the top bits of s[j'-4]
// (scale) and s[j'] (min).  The two sub-blocks of a lane sit in one 16-bit
// half of each dword, so both are decoded at once.
struct SBScales {
    double d, dmin, m0, m1;
    int sc0, sc1;
};
__device__ __forceinline__ void decode_scales(const u32x4& hdr, int j, SBScales& s) {
    const int sh = (j & 1) * 16;
    const uint32_t a2 = (hdr.y >> sh) & 0xFFFFu;
    const uint32_t b2 = (hdr.z >> sh) & 0xFFFFu;
    const uint32_t c2 = (hdr.w >> sh) & 0xFFFFu;
    const uint32_t sc_lo = a2 & 0x3F3Fu, m_lo = b2 & 0x3F3Fu;
    const uint32_t sc_hi = (c2 & 0x0F0Fu) | ((a2 & 0xC0C0u) >> 2);
    const uint32_t m_hi = ((c2 >> 4) & 0x0F0Fu) | ((b2 & 0xC0C0u) >> 2);
    const uint32_t scp = j < 2 ? sc_lo : sc_hi, mp = j < 2 ? m_lo : m_hi;
    s.sc0 = (int)(scp & 0xFFu);
    s.sc1 = (int)(scp >> 8);
    s.m0 = (double)(int)(mp & 0xFFu);
    s.m1 = (double)(int)(mp >> 8);
    s.d = (double)f16_to_f32(hdr.x);
    s.dmin = (double)f16_to_f32(hdr.x >> 16);
}

// Exact int32 sums of one lane's two sub-blocks against the staged codes.
__device__ __forceinline__ void sb_isums(const SBLoad& L, const StagedPair& x, int& i0, int& i1) {
    const uint32_t q[8] = {L.qa.x, L.qa.y, L.qa.z, L.qa.w, L.qb.x, L.qb.y, L.qb.z, L.qb.w};
    int a = 0, b = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        a = dot4(q[k] & 0x0F0F0F0Fu, x.c[k], a);
        b = dot4((q[k] >> 4) & 0x0F0F0F0Fu, x.c[8 + k], b);
    }
    i0 = a;
    i1 = b;
}

// acc += d8_0*(d*sc0*i0 - dmin*m0*ysum_0) + d8_1*(d*sc1*i1 - dmin*m1*ysum_1).
// Each product is exact in f64 (sc*isum < 2^22, d8*ysum < 2^24 significant
// bits), so only the additions round.
__device__ __forceinline__ double sb_fixup(const SBScales& s, const StagedPair& x, int i0, int i1,
                                           double acc) {
    const double t = fma((double)(s.sc1 * i1), x.d1, (double)(s.sc0 * i0) * x.d0);
    const double u = fma(s.m1, x.ds1, s.m0 * x.ds0);
    acc = fma(s.d, t, acc);
    return fma(-s.dmin, u, acc);
}

// --------------------------------------------------------------------------
// Full staging: all ncols activation columns live in LDS; each wave walks its
// (tile, pass) items with the next item's loads in flight while the current
// one computes.
template <int NC, bool DUMP>
__global__ __launch_bounds__(256) void k_gemv_q4k(
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ xq, int64_t xq_col_bytes,
    float* __restrict__ y, int32_t* __restrict__ dump_isum, int32_t* __restrict__ dump_ysum,
    int M, int nsb, int log2s, int passes, int n_tiles) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int nb = nsb * 8;
    const int col_bytes = stage_bytes(nb);
#pragma unroll
    for (int c = 0; c < NC; ++c)
        stage_q8(xq + c * xq_col_bytes, 0, nb, lds + c * col_bytes, threadIdx.x, blockDim.x,
                 (DUMP && blockIdx.x == 0 && c == 0) ? dump_ysum : nullptr);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int S = 1 << log2s, R = 64 >> log2s, gpp = S >> 2;
    const int row_local = lane >> log2s, g = (lane & (S - 1)) >> 2, j = lane & 3;
    const int wave_stride = gridDim.x * (blockDim.x >> 6);
    int tile = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (tile >= n_tiles) return;

    int p = 0;
    SBLoad cur, nxt;
    int row = tile * R + row_local, sb = g;
    bool ok = row < M && sb < nsb;
    if (ok) load_sb(w + ((int64_t)row * nsb + sb) * kQ4KBytes, j, cur);
    double acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.0;

    while (true) {
        int ntile = tile, np = p + 1;
        if (np == passes) { np = 0; ntile = tile + wave_stride; }
        const bool more = ntile < n_tiles;
        const int nrow = ntile * R + row_local, nsbi = np * gpp + g;
        const bool nok = more && nrow < M && nsbi < nsb;
        if (nok) load_sb(w + ((int64_t)nrow * nsb + nsbi) * kQ4KBytes, j, nxt);

        if (ok) {
            SBScales s;
            decode_scales(cur.hdr, j, s);
            const int P = 4 * sb + j;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                StagedPair x;
                read_pair(lds + c * col_bytes, P, x, true);
                int i0, i1;
                sb_isums(cur, x, i0, i1);
                acc[c] = sb_fixup(s, x, i0, i1, acc[c]);
                if (DUMP) {
                    dump_isum[((int64_t)c * M + row) * nb + 2 * P] = i0;
                    dump_isum[((int64_t)c * M + row) * nb + 2 * P + 1] = i1;
                }
            }
        }
        if (p == passes - 1) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const double v = group_sum_f64(acc[c], log2s);
                if ((lane & (S - 1)) == 0 && row < M) y[(int64_t)row * NC + c] = (float)v;
                acc[c] = 0.0;
            }
        }
        if (!more) break;
        tile = ntile; p = np; row = nrow; sb = nsbi; ok = nok; cur = nxt;
    }
}

// --------------------------------------------------------------------------
// Split-k: workgroup column s covers super-blocks [16s, 16s+16) of every row
// (one staging group per activation column), one row per wave tile; the f64
// partial of each (split, row, column) goes to `part` and a second kernel
// sums the splits in order.
template <int NC>
__global__ __launch_bounds__(256) void k_gemv_q4k_splitk(
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ xq, int64_t xq_col_bytes,
    double* __restrict__ part, int M, int nsb) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int split = blockIdx.y;
    const int sb0 = 16 * split;
    const int nsb_s = min(16, nsb - sb0);
#pragma unroll
    for (int c = 0; c < NC; ++c)
        stage_q8(xq + c * xq_col_bytes, 8 * sb0, 8 * nsb_s, lds + c * kStageGroupBytes, threadIdx.x,
                 blockDim.x, nullptr);
    __syncthreads();

    const int lane = threadIdx.x & 63, g = lane >> 2, j = lane & 3;
    const int wave_stride = gridDim.x * (blockDim.x >> 6);
    int row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (row >= M) return;
    const bool active = g < nsb_s;
    SBLoad cur, nxt;
    if (active) load_sb(w + ((int64_t)row * nsb + sb0 + g) * kQ4KBytes, j, cur);
    while (true) {
        const int nrow = row + wave_stride;
        const bool more = nrow < M;
        if (more && active) load_sb(w + ((int64_t)nrow * nsb + sb0 + g) * kQ4KBytes, j, nxt);
        double acc[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] = 0.0;
        if (active) {
            SBScales s;
            decode_scales(cur.hdr, j, s);
            const int P = 4 * g + j;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                StagedPair x;
                read_pair(lds + c * kStageGroupBytes, P, x, true);
                int i0, i1;
                sb_isums(cur, x, i0, i1);
                acc[c] = sb_fixup(s, x, i0, i1, 0.0);
            }
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const double v = wave_sum_f64(acc[c]);
            if (lane == 0) part[((int64_t)split * M + row) * NC + c] = v;
        }
        if (!more) break;
        row = nrow;
        cur = nxt;
    }
}

__global__ void k_splitk_finalize(const double* __restrict__ part, float* __restrict__ y, int64_t n,
                                  int n_split) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    double v = 0.0;
    for (int s = 0; s < n_split; ++s) v += part[(int64_t)s * n + i];
    y[i] = (float)v;
}

// --------------------------------------------------------------------------
// Grouped GEMV for routed experts.  Without a combine, each wave work item
// is (slot, tile); with one, a wave computes a tile for every slot in slot
// order and forms sum_s combine[s]*y_s in f64.  Per slot the lane layout,
// arithmetic and reduction are those of k_gemv_q4k, so a slot's result
// equals the single GEMV on that expert.
template <bool COMBINE>
__global__ __launch_bounds__(256) void k_gemv_q4k_grouped(
    const uint8_t* __restrict__ w_all, int64_t expert_bytes, int n_experts,
    const int32_t* __restrict__ ids, int n_sel, const uint8_t* __restrict__ xq, int64_t xq_stride,
    float* __restrict__ y, const float* __restrict__ combine, float* __restrict__ y_out,
    const int64_t* __restrict__ out_row, int64_t out_rows, int M, int nsb, int log2s, int passes,
    int n_tiles) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int nb = nsb * 8;
    const int col_bytes = stage_bytes(nb);
    const int n_cols = xq_stride ? n_sel : 1;
    for (int c = 0; c < n_cols; ++c)
        stage_q8(xq + c * xq_stride, 0, nb, lds + c * col_bytes, threadIdx.x, blockDim.x, nullptr);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int S = 1 << log2s, R = 64 >> log2s, gpp = S >> 2;
    const int row_local = lane >> log2s, g = (lane & (S - 1)) >> 2, j = lane & 3;
    const int wave_stride = gridDim.x * (blockDim.x >> 6);
    const int n_items = COMBINE ? n_tiles : n_tiles * n_sel;
    float* yo = y_out;
    if (COMBINE && out_row) yo += (int64_t)(*out_row % out_rows) * M;

    for (int item = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); item < n_items;
         item += wave_stride) {
        const int tile = COMBINE ? item : item % n_tiles;
        const int s_begin = COMBINE ? 0 : item / n_tiles;
        const int s_end = COMBINE ? n_sel : s_begin + 1;
        const int row = tile * R + row_local;
        double comb = 0.0;
        for (int s = s_begin; s < s_end; ++s) {
            const int e = ids[s];
            const bool valid = e >= 0 && e < n_experts;
            const uint8_t* wb = w_all + (int64_t)(valid ? e : 0) * expert_bytes;
            const uint8_t* xs = lds + (xq_stride ? s : 0) * col_bytes;
            double acc = 0.0;
            for (int p = 0; p < passes; ++p) {
                const int sb = p * gpp + g;
                if (valid && row < M && sb < nsb) {
                    SBLoad L;
                    load_sb(wb + ((int64_t)row * nsb + sb) * kQ4KBytes, j, L);
                    SBScales sc;
                    decode_scales(L.hdr, j, sc);
                    StagedPair x;
                    read_pair(xs, 4 * sb + j, x, true);
                    int i0, i1;
                    sb_isums(L, x, i0, i1);
                    acc = sb_fixup(sc, x, i0, i1, acc);
                }
            }
            const double v = group_sum_f64(acc, log2s);
            const float ys = valid ? (float)v : __builtin_nanf("");
            if ((lane & (S - 1)) == 0 && row < M) {
                if (y) y[(int64_t)s * M + row] = ys;
                if (COMBINE) comb += (double)combine[s] * (double)ys;
            }
        }
        if (COMBINE && (lane & (S - 1)) == 0 && row < M) yo[row] = (float)comb;
    }
}

// --------------------------------------------------------------------------
// Host side.

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

static int ceil_log2(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

Q4KPlan plan_q4k(int64_t m, int nsb) {
    Q4KPlan p;
    p.log2s = ceil_log2(4 * nsb);
    if (p.log2s < 2) p.log2s = 2;
    if (p.log2s > 6) p.log2s = 6;
    p.rows_per_tile = 64 >> p.log2s;
    const int gpp = (1 << p.log2s) / 4;
    p.passes = (nsb + gpp - 1) / gpp;
    p.n_tiles = (int)((m + p.rows_per_tile - 1) / p.rows_per_tile);
    return p;
}

static int grid_for(int n_waves) {
    const int cap = device_cu_count() * 8;
    int g = (n_waves + 3) / 4;
    return g < cap ? (g > 0 ? g : 1) : cap;
}

template <int NC, bool DUMP>
static hipError_t launch_nc(const void* w, const void* xq, int64_t xq_col_bytes, float* y,
                            int32_t* dump_isum, int32_t* dump_ysum, int64_t m, int nsb,
                            hipStream_t stream) {
    const Q4KPlan p = plan_q4k(m, nsb);
    const int lds = NC * stage_bytes(nsb * 8);
    hipLaunchKernelGGL((k_gemv_q4k<NC, DUMP>), dim3(grid_for(p.n_tiles)), dim3(256), lds, stream,
                       (const uint8_t*)w, (const uint8_t*)xq, xq_col_bytes, y, dump_isum, dump_ysum,
                       (int)m, nsb, p.log2s, p.passes, p.n_tiles);
    return hipGetLastError();
}

hipError_t launch_gemv_q4k(const void* w, const void* xq, int64_t xq_col_bytes, float* y,
                           int32_t* dump_isum, int32_t* dump_ysum, int64_t m, int64_t k, int ncols,
                           hipStream_t stream) {
    const int nsb = (int)(k / 256);
    if (dump_isum) return launch_nc<1, true>(w, xq, xq_col_bytes, y, dump_isum, dump_ysum, m, nsb, stream);
    switch (ncols) {
        case 1: return launch_nc<1, false>(w, xq, xq_col_bytes, y, nullptr, nullptr, m, nsb, stream);
        case 2: return launch_nc<2, false>(w, xq, xq_col_bytes, y, nullptr, nullptr, m, nsb, stream);
        case 3: return launch_nc<3, false>(w, xq, xq_col_bytes, y, nullptr, nullptr, m, nsb, stream);
        case 4: return launch_nc<4, false>(w, xq, xq_col_bytes, y, nullptr, nullptr, m, nsb, stream);
        case 5: return launch_nc<5, false>(w, xq, xq_col_bytes, y, nullptr, nullptr, m, nsb, stream);
        case 6: return launch_nc<6, false>(w, xq, xq_col_bytes, y, nullptr, nullptr, m, nsb, stream);
        case 7: return launch_nc<7, false>(w, xq, xq_col_bytes, y, nullptr, nullptr, m, nsb, stream);
        case 8: return launch_nc<8, false>(w, xq, xq_col_bytes, y, nullptr, nullptr, m, nsb, stream);
        default: return hipErrorInvalidValue;
    }
}

int gemv_q4k_splitk_nsplit(int64_t k) { return (int)((k / 256 + 15) / 16); }

template <int NC>
static hipError_t launch_split_nc(const void* w, const void* xq, int64_t xq_col_bytes, float* y,
                                  double* part, int64_t m, int nsb, hipStream_t stream) {
    const int n_split = (nsb + 15) / 16;
    const int lds = NC * kStageGroupBytes;
    const int cap = device_cu_count() * 8;
    int gx = (int)((m + 3) / 4);
    const int per_split_cap = (cap + n_split - 1) / n_split;
    if (gx > per_split_cap) gx = per_split_cap;
    hipLaunchKernelGGL((k_gemv_q4k_splitk<NC>), dim3(gx, n_split), dim3(256), lds, stream,
                       (const uint8_t*)w, (const uint8_t*)xq, xq_col_bytes, part, (int)m, nsb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = m * NC;
    hipLaunchKernelGGL(k_splitk_finalize, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       (const double*)part, y, n, n_split);
    return hipGetLastError();
}

hipError_t launch_gemv_q4k_splitk(const void* w, const void* xq, int64_t xq_col_bytes, float* y,
                                  double* part, int64_t m, int64_t k, int ncols, hipStream_t stream) {
    const int nsb = (int)(k / 256);
    switch (ncols) {
        case 1: return launch_split_nc<1>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 2: return launch_split_nc<2>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 3: return launch_split_nc<3>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 4: return launch_split_nc<4>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 5: return launch_split_nc<5>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 6: return launch_split_nc<6>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 7: return launch_split_nc<7>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 8: return launch_split_nc<8>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_q4k_grouped(const void* w_all, int64_t expert_bytes, int n_experts,
                                   const int32_t* ids, int n_sel, const void* xq, int64_t xq_stride,
                                   float* y, const float* combine, float* y_out,
                                   const int64_t* out_row, int64_t out_rows, int64_t m, int64_t k,
                                   hipStream_t stream) {
    const int nsb = (int)(k / 256);
    const Q4KPlan p = plan_q4k(m, nsb);
    const int lds = (xq_stride ? n_sel : 1) * stage_bytes(nsb * 8);
    const int n_items = combine ? p.n_tiles : p.n_tiles * n_sel;
    if (combine)
        hipLaunchKernelGGL((k_gemv_q4k_grouped<true>), dim3(grid_for(n_items)), dim3(256), lds, stream,
                           (const uint8_t*)w_all, expert_bytes, n_experts, ids, n_sel,
                           (const uint8_t*)xq, xq_stride, y, combine, y_out, out_row, out_rows, (int)m,
                           nsb, p.log2s, p.passes, p.n_tiles);
    else
        hipLaunchKernelGGL((k_gemv_q4k_grouped<false>), dim3(grid_for(n_items)), dim3(256), lds, stream,
                           (const uint8_t*)w_all, expert_bytes, n_experts, ids, n_sel,
                           (const uint8_t*)xq, xq_stride, y, combine, y_out, out_row, out_rows, (int)m,
                           nsb, p.log2s, p.passes, p.n_tiles);
    return hipGetLastError();
}

}  // namespace mq
