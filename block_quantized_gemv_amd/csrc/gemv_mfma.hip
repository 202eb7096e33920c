// Batched q4_K x q8_0 GEMV on the matrix cores: y[r][c] = sum_k W[r][k] *
// X[c][k] for n <= 8 activation columns, the integer part of every
// sub-block's dot product by v_mfma_i32_16x16x64_i8.
//
// A lane group g = lane/16 of the weight operand loads 16 bytes per row:
// bytes 16g..16g+15 of the 64 bytes that hold chunks 2u and 2u+1 of a
// super-block's quants (u = 0, 1; a chunk is 32 bytes, its low nibbles are
// sub-block 2*chunk and its high nibbles sub-block 2*chunk+1, q4_K's
// layout), so that each load instruction moves 1 KB.  One MFMA (u, e) takes
// the e-nibbles (e = 0 low, 1 high) of those 16 bytes as its B operand (16
// columns j = the weight rows): lane groups 0 and 1 then hold sub-block
// 4u + e, groups 2 and 3 sub-block 4u + 2 + e.  Its A operand has 16 rows
// i = 8h + c: row i holds column c's codes of sub-block 4u + 2h + e in the
// lane groups that hold that sub-block's nibbles (g >> 1 == h) and zeros in
// the others.  So C[8h + c][j] is the exact int32 sum of sub-block
// 4u + 2h + e of row j against column c: the sub-blocks stay separate, as
// their scales differ, and all 16 output rows are used at n = 8.  The
// instruction pairs A's and B's bytes position by position within a lane
// group, so any split of k over the groups works if both operands use it.
//
// The output lane (g, j) holds C[4g + r][j], r = 0..3: weight row j and
// columns c = 4(g & 1) + r of sub-block 4u + 2(g >> 1) + e, and folds them
// into f64 accumulators as acc += isum * (d*sc * d8), every product exact
// (d, d8 are f16, sc six-bit, |isum| < 2^16), so each step rounds once.
// The mins' part, sum over sub-blocks s of (dmin*m_s) * (d8*ysum)_s, is
// itself a product of a (column x sub-block) and a (sub-block x row)
// matrix: one v_mfma_f64_16x16x4_f64 per four sub-blocks accumulates it for
// the tile (products exact: 17 and 24 significant bits).  That
// instruction's output lane (g, j) holds rows 4r + g; its A row i is given
// column 4((i % 4) & 1) + i/4, so that the lane's four rows are the same
// four columns its own accumulators hold (each column is computed twice,
// by lanes g and g + 2).  At the end of a row tile the two halves of a
// (row, column) pair, held by lanes l and l ^ 32, are added and the mins'
// part subtracted.  The sums are grouped differently from the vector
// kernels', so results agree with them to rounding, not bit for bit.
//
// Staging (per workgroup, for its k range of nb blocks, np = nb/2 pairs):
//   codes:  byte b*256 + c*32: the 32 codes of block b of column c, so that
//           an A operand's live lanes read 256 consecutive bytes per half;
//   scales: byte np*512 + P*256 + h*64 + c*8: d8 of block 2P+h of column c
//           (f64), and 128 bytes further d8*ysum.
// Columns c >= n hold zero codes and scales (they add zero).
//
// A wave owns 16-row tiles (strided across the CUs) and streams their
// super-blocks in k order, kMfmaDepth in flight; blockIdx.y splits k, each
// split leaving f64 partials that k_splitk_finalize sums in split order.
// The weights are read through a raw buffer descriptor sized to the matrix:
// a lane's byte offset is a per-lane constant plus the wave's cursor (one
// add per load), and the rows of the last tile past M lie beyond the
// descriptor's range, so the hardware returns zeros for them (they are
// never stored).  The whole offset is in the lane's offset register, which
// the range check covers; the matrix plus one tile must fit 32-bit offsets
// (mfma_rows_fit).
#include "common.hpp"
#include "launch.hpp"

namespace mq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int kMfmaPairBytes = 768;         // codes 512 + scales 256 per block pair
// After the staged blocks: zeros that the A operand's lane groups without
// live codes read (at offsets (4u + e) * 256, 16 bytes each).
constexpr int kMfmaZeroBytes = 1536;
__host__ __device__ constexpr int mfma_stage_bytes(int sb_per_split) {
    return sb_per_split * 4 * kMfmaPairBytes + kMfmaZeroBytes;
}
constexpr uint32_t kRawBufferWord3 = 0x00020000u;   // raw (untyped) buffer, 32-bit data format
constexpr int kMfmaMaxSbPerSplit = 16;      // 48 KiB of staging
#ifndef MQ_MFMA_DEPTH
#define MQ_MFMA_DEPTH 2
#endif
constexpr int kMfmaDepth = MQ_MFMA_DEPTH;   // items in flight per wave

// Writes block b (relative) of column c into the staging layout above.
__device__ __forceinline__ void stage_mfma_block(uint8_t* __restrict__ lds, int np, int c, int b, uint32_t dbits,
                                                 const uint32_t (&q)[8], bool real) {
    const int P = b >> 1, h = b & 1;
    double d = 0.0, ds = 0.0;
    if (real) {
        int s = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) s = dot4(q[i], 0x01010101u, s);
        d = (double)f16_to_f32(dbits);
        ds = d * (double)s;
    }
    uint8_t* cp = lds + b * 256 + c * 32;
    *(u32x4*)cp = real ? u32x4{q[0], q[1], q[2], q[3]} : u32x4{0u, 0u, 0u, 0u};
    *(u32x4*)(cp + 16) = real ? u32x4{q[4], q[5], q[6], q[7]} : u32x4{0u, 0u, 0u, 0u};
    uint8_t* scl = lds + np * 512 + P * 256 + h * 64 + c * 8;
    *(double*)scl = d;
    *(double*)(scl + 128) = ds;
}

// Stages blocks [b0, b0 + nb) of the n = NC columns (zeros for columns NC..7).
// Each thread first requests up to R of its blocks, then writes them, so
// that their loads are in flight together.
template <int NC, int R>
__device__ __forceinline__ void stage_mfma(const uint8_t* __restrict__ xq, int64_t col_stride, int b0, int nb,
                                           uint8_t* __restrict__ lds) {
    const int np = nb >> 1, T = blockDim.x, tid = threadIdx.x;
    const int real = NC * nb;
    for (int base = tid; base < real; base += R * T) {
        uint32_t q[R][8], dbits[R];
        int cc[R], bb[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // the column varies fastest, so that neighbouring threads write
            // neighbouring LDS words
            const int f = base + r * T;
            const bool in = f < real;
            const int b = in ? f / NC : 0;
            bb[r] = b;
            cc[r] = in ? f - b * NC : 0;
            dbits[r] = load_q8_block(xq + cc[r] * col_stride + (int64_t)(b0 + b) * kQ8Bytes, q[r]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (base + r * T < real) stage_mfma_block(lds, np, cc[r], bb[r], dbits[r], q[r], true);
    }
    if (NC < 8) {
        const uint32_t z[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        for (int f = tid; f < (8 - NC) * nb; f += T) {
            const int b = f / (8 - NC);
            stage_mfma_block(lds, np, NC + (f - b * (8 - NC)), b, 0u, z, false);
        }
    }
}

// Six-bit scale and min of sub-block s = 4*HI + j (j = 0..3) of a q4_K
// header (bytes 4..15 are the packed scales s[0..11], in hdr.y, hdr.z,
// hdr.w): s < 4 keeps them in the low six bits of s[s] and s[s+4]; s >= 4
// takes the nibbles of s[s+4] and the top two bits of s[s-4] (scale) and
// s[s] (min).  HI is compile-time; j may differ between lanes.
template <int HI>
__device__ __forceinline__ void scale_min_of(const u32x4& hdr, int j, uint32_t& sc, uint32_t& m) {
    const int sh = 8 * j;
    if constexpr (HI == 0) {
        sc = (hdr.y >> sh) & 63u;
        m = (hdr.z >> sh) & 63u;
    } else {
        const uint32_t lo = hdr.w >> sh;
        sc = (lo & 15u) | (((hdr.y >> sh) >> 2) & 48u);
        m = ((lo >> 4) & 15u) | (((hdr.z >> sh) >> 2) & 48u);
    }
}

// Items 0..n-1 through a ring of D register buffers: items 0..D-1 are
// fetched by the caller, then item i is used and item i + D fetched into
// its buffer, so that D items' loads are in flight while one computes.
// The fetches of full rounds are unconditional (past the end they re-read
// the last item, which the fetch must allow) so that the compiler can wait
// for exactly the buffer about to be used; the last, partial round only
// uses.
template <int D, class Buf, class Fetch, class Use>
__device__ __forceinline__ void stream_ring(int n, Buf (&buf)[D], Fetch&& fetch, Use&& use) {
    int i = 0;
    for (; i + D <= n; i += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            use(buf[u]);
            fetch(i + u + D, buf[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < D; ++u)
        if (i + u < n) use(buf[u]);
}

// One workgroup per CU and k split (so that every CU gets the same share):
// wave w of workgroup b owns row tiles b + GX*w, b + GX*(w + W), ... (GX
// workgroups per split, W waves each) and walks their super-blocks in k
// order with a cursor, kMfmaDepth items in flight.
template <int NC, int D>
__global__ __launch_bounds__(1024) void k_gemv_q4k_mfma(const uint8_t* __restrict__ w, const uint8_t* __restrict__ xq,
                                                        int64_t xq_col_bytes, float* __restrict__ y,
                                                        double* __restrict__ part, int M, int nsb, int sb_per_split,
                                                        int n_tiles) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int sb0 = (int)blockIdx.y * sb_per_split;
    const int nsb_s = min(sb_per_split, nsb - sb0);
    const int nb = 8 * nsb_s, np = nb >> 1;
    const int lane = threadIdx.x & 63, g = lane >> 4, i16 = lane & 15;
    const int GX = (int)gridDim.x, WPG = (int)(blockDim.x >> 6);
    const int t0 = (int)blockIdx.x + GX * wave_id();            // the wave's first tile
    const int stride = GX * WPG;
    const int my_tiles = t0 < n_tiles ? (n_tiles - 1 - t0) / stride + 1 : 0;
    const int n_items = my_tiles * nsb_s;
    const uint32_t row_bytes = (uint32_t)nsb * kQ4KBytes;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)w, (short)0, (int)((uint32_t)M * row_bytes), (int)kRawBufferWord3);

    // Items are (tile, super-block) in that order, walked by a wave-uniform
    // cursor (the item's byte offset, tile * 16 rows + super-block) that
    // stays on the last item past the end (its lines are re-read, nothing
    // is computed from them).
    struct Item {
        u32x4 hdr;
        u32x4 q[2];     // bytes 16g..16g+15 of chunks 2u, 2u+1 (64 bytes from 16 + 64u)
        int tile, sbl;
    };
    const uint32_t lane_hdr = (uint32_t)i16 * row_bytes, lane_q = lane_hdr + 16u + 16u * (uint32_t)g;
    const uint32_t tile_wrap = (uint32_t)stride * 16u * row_bytes - (uint32_t)(nsb_s - 1) * kQ4KBytes;
    int c_tile = t0, c_sb = 0, c_done = 0;
    uint32_t c_off = (uint32_t)t0 * 16u * row_bytes + (uint32_t)sb0 * kQ4KBytes;
    auto fetch = [&](int, Item& it) {
        it.tile = c_tile;
        it.sbl = c_sb;
        const uint32_t off = c_off;
        if (c_done < n_items && ++c_done < n_items) {
            if (++c_sb == nsb_s) {
                c_sb = 0;
                c_tile += stride;
                c_off += tile_wrap;
            } else {
                c_off += kQ4KBytes;
            }
        }
        it.hdr = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_hdr + off, 0, 0));
#pragma unroll
        for (int u = 0; u < 2; ++u)
            it.q[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_q + off + 64u * u, 0, 0));
    };

    Item ring[D];
#pragma unroll
    for (int u = 0; u < D; ++u) fetch(u, ring[u]);
    stage_mfma<NC, 2>(xq, xq_col_bytes, 8 * sb0, nb, lds);
    uint8_t* const zeros = lds + mfma_stage_bytes(sb_per_split) - kMfmaZeroBytes;
    for (int t = threadIdx.x; t < kMfmaZeroBytes / 16; t += blockDim.x) *(u32x4*)(zeros + 16 * t) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();

    const int h = g >> 1, cb = 4 * (g & 1);
    // A operand: row i16 = 8*ha + c takes, in lane group g, codes 16(g&1)..16(g&1)+15 of
    // block 4u + 2ha + e (of the item's super-block) of column c when g >> 1 == ha, else zeros
    // (lanes without live codes read the zeros, at the same offsets, whatever the item)
    const int ha = i16 >> 3;
    const bool a_live = (g >> 1) == ha;
    const uint8_t* xa = a_live ? lds + (2 * ha) * 256 + (i16 & 7) * 32 + 16 * (g & 1) : zeros;
    const int xa_step = a_live ? 8 * 256 : 0;                       // per super-block
    const uint8_t* xd = lds + np * 512 + h * 256 + cb * 8;           // its four columns' d8 (pair 2u + h, half e)
    // the mins' operand: column 4((i % 4) & 1) + i/4 of row i = i16, sub-blocks
    // g (pair g/2, half g%2) and 4 + g (two pairs further)
    const uint8_t* xm = lds + np * 512 + 128 + (g >> 1) * 256 + (g & 1) * 64 + (4 * ((i16 & 3) & 1) + (i16 >> 2)) * 8;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    v4d mins = {0.0, 0.0, 0.0, 0.0};
    stream_ring<D>(n_items, ring, fetch, [&](const Item& it) {
        const int P0 = 4 * it.sbl;
        const uint8_t* xi = xa + it.sbl * xa_step;
        // C[2u + e]: sub-block 4u + 2h + e of this lane's rows (h = g >> 1)
        v4i C[4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const u32x4 q = it.q[u];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t sh = 4 * e;
                const v4i wb = {(int)((q.x >> sh) & 0x0F0F0F0Fu), (int)((q.y >> sh) & 0x0F0F0F0Fu),
                                (int)((q.z >> sh) & 0x0F0F0F0Fu), (int)((q.w >> sh) & 0x0F0F0F0Fu)};
                const u32x4 x = *(const u32x4*)(xi + (4 * u + e) * 256);
                const v4i xv = {(int)x.x, (int)x.y, (int)x.z, (int)x.w};
                C[2 * u + e] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xv, wb, v4i{0, 0, 0, 0}, 0, 0, 0);
            }
        }
        // mins: row j = i16's (dmin * m_s) against (d8 * ysum)_s, s = g and 4 + g
        const double dmin = (double)f16_to_f32(it.hdr.x >> 16);
        {
            const uint32_t z = it.hdr.z >> (8 * g);
            const uint32_t m_lo = z & 63u;
            const uint32_t m_hi = ((it.hdr.w >> (8 * g)) >> 4 & 15u) | ((z >> 2) & 48u);
            const uint8_t* mp = xm + P0 * 256;
            mins = __builtin_amdgcn_mfma_f64_16x16x4f64(*(const double*)mp, dmin * (double)m_lo, mins, 0, 0, 0);
            mins = __builtin_amdgcn_mfma_f64_16x16x4f64(*(const double*)(mp + 512), dmin * (double)m_hi, mins, 0, 0, 0);
        }
        const double d = (double)f16_to_f32(it.hdr.x);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                uint32_t sc, m;
                if (u == 0) scale_min_of<0>(it.hdr, 2 * h + e, sc, m);
                else scale_min_of<1>(it.hdr, 2 * h + e, sc, m);
                (void)m;
                const double a1 = d * (double)sc;
                const uint8_t* dp = xd + (P0 + 2 * u) * 256 + e * 64;
                const f64x2 d01 = *(const f64x2*)dp;
                const f64x2 d23 = *(const f64x2*)(dp + 16);
                const v4i& Ct = C[2 * u + e];
                acc[0] = fma((double)Ct[0], a1 * d01.x, acc[0]);
                acc[1] = fma((double)Ct[1], a1 * d01.y, acc[1]);
                acc[2] = fma((double)Ct[2], a1 * d23.x, acc[2]);
                acc[3] = fma((double)Ct[3], a1 * d23.y, acc[3]);
            }
        }
        if (it.sbl != nsb_s - 1) return;
        // tile done: the two sub-block parities (lanes l and l ^ 32) added and
        // the mins' part subtracted; lanes g < 2 hold (row i16, columns cb..cb+3)
        const int row = it.tile * 16 + i16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const double tot = (acc[r] + __shfl_xor(acc[r], 32, 64)) - mins[r];
            acc[r] = 0.0;
            const int c = cb + r;
            if (g < 2 && c < NC && row < M) {
                if (part) part[((int64_t)blockIdx.y * M + row) * NC + c] = tot;
                else y[(int64_t)row * NC + c] = (float)tot;
            }
        }
        mins = v4d{0.0, 0.0, 0.0, 0.0};
    });
}

}  // namespace

// The split of k for m rows of nsb super-blocks: enough (tile, split) units
// for the GPU's waves, at most kMfmaMaxSbPerSplit super-blocks staged per
// workgroup; then about one workgroup per CU, split evenly among the k
// ranges, each with the waves its tiles need (at most 16; past that waves
// take several tiles).
MfmaPlan plan_gemv_q4k_mfma(int64_t m, int nsb) {
    MfmaPlan p;
    const int64_t tiles = (m + 15) / 16;
    const int64_t cus = device_cu_count();
    const int64_t target = cus * 8;
    int64_t ns = (nsb + kMfmaMaxSbPerSplit - 1) / kMfmaMaxSbPerSplit;
    const int64_t want = (target + tiles - 1) / tiles;
    if (want > ns) ns = want < nsb ? want : nsb;
    p.sb_per_split = (int)((nsb + ns - 1) / ns);
    p.n_split = (nsb + p.sb_per_split - 1) / p.sb_per_split;
    p.n_tiles = (int)tiles;
    p.lds = mfma_stage_bytes(p.sb_per_split);
    int64_t gx = cus / p.n_split;
    if (gx < 1) gx = 1;
    if (gx > tiles) gx = tiles;
    int64_t wpg = (tiles + gx - 1) / gx;
    if (wpg > 16) wpg = 16;
    p.grid_x = (int)gx;
    p.threads = (int)(64 * wpg);
    return p;
}

template <int NC>
static hipError_t launch_mfma_nc(const void* w, const void* xq, int64_t xq_col_bytes, float* y, double* part,
                                 int64_t m, int nsb, hipStream_t stream) {
    const MfmaPlan p = plan_gemv_q4k_mfma(m, nsb);
    if (p.n_split > 1 && !part) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_gemv_q4k_mfma<NC, kMfmaDepth>), dim3((unsigned)p.grid_x, (unsigned)p.n_split),
                       dim3((unsigned)p.threads), p.lds, stream, (const uint8_t*)w, (const uint8_t*)xq, xq_col_bytes,
                       y, p.n_split > 1 ? part : nullptr, (int)m, nsb, p.sb_per_split, p.n_tiles);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_split == 1) return e;
    return launch_splitk_finalize(part, y, m * NC, p.n_split, stream);
}

int64_t gemv_q4k_mfma_partial_bytes(int64_t m, int64_t k, int ncols) {
    const MfmaPlan p = plan_gemv_q4k_mfma(m, (int)(k / 256));
    return p.n_split > 1 ? (int64_t)p.n_split * m * ncols * (int64_t)sizeof(double) : 0;
}

bool mfma_rows_fit(int64_t m, int64_t k) { return (m + 16) * (k / 256) * kQ4KBytes <= (int64_t)0xFFFFFFFF; }

hipError_t launch_gemv_q4k_mfma(const void* w, const void* xq, int64_t xq_col_bytes, float* y, double* part,
                                int64_t m, int64_t k, int ncols, hipStream_t stream) {
    if (!mfma_rows_fit(m, k)) return hipErrorInvalidValue;
    const int nsb = (int)(k / 256);
    switch (ncols) {
        case 2: return launch_mfma_nc<2>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 3: return launch_mfma_nc<3>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 4: return launch_mfma_nc<4>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 5: return launch_mfma_nc<5>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 6: return launch_mfma_nc<6>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 7: return launch_mfma_nc<7>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 8: return launch_mfma_nc<8>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mq
