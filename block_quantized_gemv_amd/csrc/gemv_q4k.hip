// q4_K x q8_0 GEMV kernels for gfx950.
//
// The decode-step matvec over block-quantized weights: the weight stream is
// read once, in 16-byte loads, while the q8_0 activation sits in LDS.
// Integer 4-way dot products (v_dot4_i32_i8) form the exact int32 sum of
// each 32-value sub-block, the f16 d/dmin fixup is applied in f64 and each
// row is reduced across its lanes with DPP/swizzle steps in a fixed order.
// '07 · R3 — Small-model per-token overhead' (§1) credits this kind of
// decode kernel (MMVQ: 4-way integer dot products against activations
// re-quantized to q8_0) with a large q4_K decode gain but describes it only
// by name; this is a wave64/CDNA4 design of it.
//
// Lane work: a super-block (144 B = 16 B header + 128 B nibbles) is shared
// by 4 lanes; lane j takes nibble chunk j (32 bytes = sub-blocks 2j, 2j+1:
// low nibbles pair with q8_0 block 8sb+2j, high nibbles with 8sb+2j+1) plus
// the 16-byte header, which the 4 lanes read as one broadcast.  A row gets
// an aligned slot of S lanes (S/4 super-blocks per pass, `passes` passes);
// a wave holds 64/S rows (a tile).
//
// Streaming: each wave walks its (tile, pass) items with two register
// buffers in ping-pong, so the loads of the next item are in flight while
// the current one computes.  Loads are never skipped (lanes past the end
// read a clamped, in-bounds address and contribute zero; items past a
// wave's last one read the matrix's first bytes, one shared cache line),
// which lets the compiler wait only for the item it is about to use.
#include <hip/hip_ext.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "common.hpp"
#include "glue.hpp"
#include "launch.hpp"

namespace mq {

struct SBLoad {
    u32x4 hdr, qa, qb;
};

// blk: super-block start; jo = 32*j, the lane's nibble chunk.  Ordinary
// (temporal) loads: the three loads of a super-block touch the same cache
// lines at different times, and a non-temporal hint lets those lines leave
// the cache in between, which costs a second fetch from HBM (measured: 37%
// longer on the 37888x3584 matrix).
__device__ __forceinline__ void load_sb(const uint8_t* __restrict__ blk, int jo, SBLoad& L) {
    L.hdr = *(const u32x4*)blk;
    L.qa = *(const u32x4*)(blk + 16 + jo);
    L.qb = *(const u32x4*)(blk + 32 + jo);
}

// Scales and mins of sub-blocks 2j and 2j+1 from the header.  Bytes s[0..3]
// are hdr.y, s[4..7] hdr.z, s[8..11] hdr.w; sub-blocks j' < 4 keep sc and m
// in the low six bits of s[j'] and s[j'+4]; j' >= 4 take their low four bits
// from the nibbles of s[j'+4] and their top two from the top bits of s[j'-4]
// (scale) and s[j'] (min).  A lane's two sub-blocks sit in one 16-bit half
// of each dword (sh = 0 or 16), so both are decoded at once, and both obey
// the same rule, so the rule is a set of per-lane masks rather than a
// branch: mA = 0x3F3F or 0xC0C0, shA = 0 or 2, mC = 0 or 0x0F0F (see
// Lanes).  hx is the header's d/dmin dword, or 0 for an invalid item so
// that it adds exactly zero.
struct SBScales {
    double d, dmin, m0, m1;
    uint32_t scp;      // the two six-bit scales: sc0 | sc1 << 8
};
__device__ __forceinline__ void decode_scales(const u32x4& hdr, uint32_t hx, int sh, uint32_t mA, uint32_t shA,
                                              uint32_t mC, SBScales& s) {
    const uint32_t a2 = hdr.y >> sh, b2 = hdr.z >> sh, c2 = hdr.w >> sh;
    const uint32_t scp = ((a2 & mA) >> shA) | (c2 & mC);
    const uint32_t mp = ((b2 & mA) >> shA) | ((c2 >> 4) & mC);
    // An empty asm hides scp's range, so that the byte masks where the
    // scales are used survive and both products select 24-bit multiplies.
    uint32_t opaque = scp;
    asm("" : "+v"(opaque));
    s.scp = opaque;
    s.m0 = (double)(mp & 0xFFu);
    s.m1 = (double)(mp >> 8);
    s.d = (double)f16_to_f32(hx);
    s.dmin = (double)f16_to_f32(hx >> 16);
}

// Exact int32 sums of one lane's two sub-blocks against the staged codes.
// The high nibbles of two dwords come from one 64-bit shift: the bits the
// low dword takes from the high one land in its top nibble, which the mask
// clears.
__device__ __forceinline__ void sb_isums(const SBLoad& L, const StagedPair& x, int& i0, int& i1) {
    const uint32_t q[8] = {L.qa.x, L.qa.y, L.qa.z, L.qa.w, L.qb.x, L.qb.y, L.qb.z, L.qb.w};
    const uint64_t h0 = (((uint64_t)q[1] << 32) | q[0]) >> 4;
    int a = dot4_first(q[0] & 0x0F0F0F0Fu, x.c[0]);
    int b = dot4_first((uint32_t)h0 & 0x0F0F0F0Fu, x.c[8]);
    a = dot4(q[1] & 0x0F0F0F0Fu, x.c[1], a);
    b = dot4((uint32_t)(h0 >> 32) & 0x0F0F0F0Fu, x.c[9], b);
#pragma unroll
    for (int k = 2; k < 8; k += 2) {
        const uint64_t h = (((uint64_t)q[k + 1] << 32) | q[k]) >> 4;
        a = dot4(q[k] & 0x0F0F0F0Fu, x.c[k], a);
        b = dot4((uint32_t)h & 0x0F0F0F0Fu, x.c[8 + k], b);
        a = dot4(q[k + 1] & 0x0F0F0F0Fu, x.c[k + 1], a);
        b = dot4((uint32_t)(h >> 32) & 0x0F0F0F0Fu, x.c[9 + k], b);
    }
    i0 = a;
    i1 = b;
}

// acc + d8_0*(d*sc0*i0 - dmin*m0*ysum_0) + d8_1*(d*sc1*i1 - dmin*m1*ysum_1)
// in f64, as acc + d*t - dmin*u.  Every product is exact (sc*isum < 2^22 and
// d8*ysum < 2^24 significant bits against 53), so only the additions round.
// An invalid item has zero scales and a staged stand-in pair: t and u are
// then finite (six-bit scales and mins, exact integer sums, finite
// activation scales), so it adds exactly zero.  The scales are masked where
// they are used, so that both products select 24-bit multiplies.  Every
// column count uses this same sequence (measured: per-row products shared
// by the columns save time only at n = 8 and cost the one-column GEMV
// more), so a batched column equals the one-column GEMV bit for bit.
__device__ __forceinline__ double sb_accumulate(double acc, const SBScales& s, const StagedPair& x, int i0, int i1) {
    const int sc0 = (int)(s.scp & 0xFFu), sc1 = (int)((s.scp >> 8) & 0xFFu);
    const double t = fma((double)__mul24(sc1, i1), x.d1, (double)__mul24(sc0, i0) * x.d0);
    const double u = fma(s.m1, x.ds1, s.m0 * x.ds0);
    return fma(-s.dmin, u, fma(s.d, t, acc));
}

// Per-lane constants of the lane layout.
// A staged pair's LDS banks depend only on its index mod 16.  An invalid
// lane reads pair (P & pmask) instead of P, which is staged (pairs 0..15 are
// when the row has at least four super-blocks) and lies in the same banks
// whenever pmask = 15, so that the redirection adds no bank conflicts.
__device__ __forceinline__ int staged_pair_mask(int nsb) { return nsb >= 4 ? 15 : nsb >= 2 ? 7 : 3; }

struct Lanes {
    int lane, log2s, S, R, gpp, row_local, g, j, sh, pmask;
    uint32_t mA, shA, mC;       // the lane's scale-decode rule (decode_scales)
    int lds_lane, lds_inval;    // staging byte offsets: the lane's pair within a pass, and its stand-in
    __device__ Lanes(int log2s_, int nsb) {
        pmask = staged_pair_mask(nsb);
        lane = threadIdx.x & 63;
        log2s = log2s_;
        S = 1 << log2s;
        R = 64 >> log2s;
        gpp = S >> 2;
        row_local = lane >> log2s;
        g = (lane & (S - 1)) >> 2;
        j = lane & 3;
        sh = (j & 1) * 16;
        const bool low = j < 2;
        mA = low ? 0x3F3Fu : 0xC0C0u;
        shA = low ? 0u : 2u;
        mC = low ? 0u : 0x0F0Fu;
        lds_lane = (4 * g + j) * 16;
        lds_inval = ((4 * g + j) & pmask) * 16;
    }
};

// The staged pair that lane (g, j) needs in pass p: P = 4*(p*gpp + g) + j.
__device__ __forceinline__ int pair_of(const Lanes& ln, int p) { return 4 * (p * ln.gpp + ln.g) + ln.j; }

// Staging offset (group base plus slot) where pass p's pairs start.  Pass p
// covers pairs 4*gpp*p .. 4*gpp*p + 4*gpp - 1, which never cross a 64-pair
// group (4*gpp divides 64), so the lane's pair is lds_lane bytes further.
// Wave-uniform.
__device__ __forceinline__ int pass_lds_base(const Lanes& ln, int p) {
    const int P0 = 4 * ln.gpp * p;
    return (P0 >> 6) * kStageGroupBytes + (P0 & 63) * 16;
}

// The staged data of the pair at byte offset A (its group's base plus
// (P & 63)*16), as read_pair reads pair P.
__device__ __forceinline__ void read_pair_at(const uint8_t* __restrict__ lds, int A, StagedPair& sp) {
    const uint8_t* g = lds + A;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const u32x4 v = *(const u32x4*)(g + k * 1024);
        sp.c[4 * k + 0] = v.x; sp.c[4 * k + 1] = v.y; sp.c[4 * k + 2] = v.z; sp.c[4 * k + 3] = v.w;
    }
    sp.d0 = *(const double*)(g + 4096);
    sp.d1 = *(const double*)(g + 4096 + 8);
    sp.ds0 = *(const double*)(g + 5120);
    sp.ds1 = *(const double*)(g + 5120 + 8);
}

// One q4_K super-block item for NC activation columns: adds the lane's
// contribution to acc[] (nothing for an invalid item).  A: the LDS offset of
// the lane's staged pair, or, for an invalid item, of a staged stand-in
// (lds_inval: pair P & pmask, staged whenever the row has the super-blocks
// pmask implies, and in the same LDS banks), so that its terms are finite
// and, with zero scales, add exactly zero.  P is only for the dump.
template <int NC, bool DUMP>
__device__ __forceinline__ void sb_item_at(const SBLoad& L, const Lanes& ln, int A, int P, bool valid,
                                           const uint8_t* __restrict__ lds, int col_bytes, double (&acc)[NC],
                                           int32_t* __restrict__ dump, int64_t dump_row_off) {
    SBScales s;
    decode_scales(L.hdr, valid ? L.hdr.x : 0u, ln.sh, ln.mA, ln.shA, ln.mC, s);
    // With many columns they are double-buffered: column c+1's staged pair
    // is read before column c is computed, so its LDS latency overlaps that
    // work (with few columns the extra registers would cost occupancy).
    constexpr bool kPipe = NC >= 5;
    StagedPair xb[2];
    if (kPipe) read_pair_at(lds, A, xb[0]);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (kPipe && c + 1 < NC) read_pair_at(lds + (c + 1) * col_bytes, A, xb[(c + 1) & 1]);
        if (!kPipe) read_pair_at(lds + c * col_bytes, A, xb[c & 1]);
        const StagedPair& x = xb[c & 1];
        int i0, i1;
        sb_isums(L, x, i0, i1);
        acc[c] = sb_accumulate(acc[c], s, x, i0, i1);
        if (DUMP && valid) {
            dump[dump_row_off + 2 * P] = i0;
            dump[dump_row_off + 2 * P + 1] = i1;
        }
    }
}

// The same item addressed by its staged pair P.
template <int NC, bool DUMP>
__device__ __forceinline__ void sb_item(const SBLoad& L, const Lanes& ln, int P, bool valid,
                                        const uint8_t* __restrict__ lds, int col_bytes, double (&acc)[NC],
                                        int32_t* __restrict__ dump, int64_t dump_row_off) {
    const int A = valid ? (P >> 6) * kStageGroupBytes + (P & 63) * 16 : (P & ln.pmask) * 16;
    sb_item_at<NC, DUMP>(L, ln, A, P, valid, lds, col_bytes, acc, dump, dump_row_off);
}

// --------------------------------------------------------------------------
// q4_0 weights in the same geometry.  Eight 18-byte q4_0 blocks (f16 d, then
// 16 quant bytes: byte i holds weight i in its low nibble and weight 16+i in
// its high nibble; weight = d*(q - 8)) fill the same 144 bytes and 256
// weights as one q4_K super-block, so rows of k/256 such groups use the q4_K
// lane layout unchanged.  Lane j takes blocks 2j and 2j+1 (bytes 36j..36j+35,
// dword aligned), whose activation is staged pair 4*group + j as for q4_K.
// The first block's quants start 2 bytes into a dword and are realigned
// with v_alignbyte; the second block's are aligned.
struct Q40Load {
    u32x4 a, b;
    uint32_t c;
};

__device__ __forceinline__ void load_group(const uint8_t* __restrict__ grp, int j, Q40Load& L) {
    const uint8_t* p = grp + 36 * j;
    L.a = *(const u32x4_a4*)p;
    L.b = *(const u32x4_a4*)(p + 16);
    L.c = *(const uint32_t*)(p + 32);
}
__device__ __forceinline__ void load_group(const uint8_t* __restrict__ grp, int j, SBLoad& L) {
    load_sb(grp, 32 * j, L);
}

// The same loads at w + off: the base stays in SGPRs and the lane's
// offset is one 32-bit VGPR (the matrix must be smaller than 4 GiB; the
// launchers split larger ones by rows).
__device__ __forceinline__ void load_group_off(const uint8_t* __restrict__ w, uint32_t off, int j, SBLoad& L) {
    L.hdr = *(const u32x4*)(w + off);
    const uint32_t oq = off + 32u * (uint32_t)j;
    L.qa = *(const u32x4*)(w + oq + 16u);
    L.qb = *(const u32x4*)(w + oq + 32u);
}
__device__ __forceinline__ void load_group_off(const uint8_t* __restrict__ w, uint32_t off, int j, Q40Load& L) {
    const uint32_t o = off + 36u * (uint32_t)j;
    L.a = *(const u32x4_a4*)(w + o);
    L.b = *(const u32x4_a4*)(w + o + 16u);
    L.c = *(const uint32_t*)(w + o + 32u);
}

template <int FMT> struct GroupLoad { using type = SBLoad; };
template <> struct GroupLoad<kFmtQ4_0> { using type = Q40Load; };

template <int NC, bool DUMP>
__device__ __forceinline__ void group_item(const SBLoad& L, const Lanes& ln, int P, bool valid,
                                           const uint8_t* __restrict__ lds, int col_bytes, double (&acc)[NC],
                                           int32_t* __restrict__ dump, int64_t dump_row_off) {
    sb_item<NC, DUMP>(L, ln, P, valid, lds, col_bytes, acc, dump, dump_row_off);
}

// acc + d_a*(d8_0*isum_0 - 8*d8_0*ysum_0) + d_b*(d8_1*isum_1 - 8*d8_1*ysum_1)
// in f64: d8*isum has < 28 significant bits and 8*d8*ysum shares its scale,
// so each bracket is exact, and so is its product with the block's f16 d;
// only the two additions round.
template <int NC, bool DUMP>
__device__ __forceinline__ void group_item(const Q40Load& L, const Lanes& ln, int P, bool valid,
                                           const uint8_t* __restrict__ lds, int col_bytes, double (&acc)[NC],
                                           int32_t* __restrict__ dump, int64_t dump_row_off) {
    const uint32_t dw[9] = {L.a.x, L.a.y, L.a.z, L.a.w, L.b.x, L.b.y, L.b.z, L.b.w, L.c};
    uint32_t q0[4], q1[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        q0[k] = __builtin_amdgcn_alignbyte(dw[k + 1], dw[k], 2);
        q1[k] = dw[5 + k];
    }
    // zero scales for an invalid item, which reads a staged pair (finite
    // brackets), so that it adds zero
    const double da = valid ? (double)f16_to_f32(dw[0]) : 0.0;
    const double db = valid ? (double)f16_to_f32(dw[4] >> 16) : 0.0;
    P = valid ? P : (P & ln.pmask);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        StagedPair x;
        read_pair(lds + c * col_bytes, P, x, true);
        int i0 = 0, i1 = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            i0 = dot4(q0[k] & 0x0F0F0F0Fu, x.c[k], i0);
            i0 = dot4((q0[k] >> 4) & 0x0F0F0F0Fu, x.c[4 + k], i0);
            i1 = dot4(q1[k] & 0x0F0F0F0Fu, x.c[8 + k], i1);
            i1 = dot4((q1[k] >> 4) & 0x0F0F0F0Fu, x.c[12 + k], i1);
        }
        acc[c] = fma(da, fma(x.d0, (double)i0, -8.0 * x.ds0), fma(db, fma(x.d1, (double)i1, -8.0 * x.ds1), acc[c]));
        if (DUMP && valid) {
            dump[dump_row_off + 2 * P] = i0;
            dump[dump_row_off + 2 * P + 1] = i1;
        }
    }
}

// --------------------------------------------------------------------------
// Full staging: all NC activation columns live in LDS.  Wave w owns tiles
// w, w+W, w+2W, ... (W = waves in the grid); its items are (tile, pass) in
// that order.  Where the activation comes from (SRC):
//   kSrcQ8       q8_0 columns at xq, staged by 256-thread workgroups
//                (several per CU) after the first item is requested (the
//                debug dump, and 7 or 8 columns, where the early form would
//                spill registers);
//   kSrcQ8Early  one to six q8_0 columns at xq, requested before the
//                weights and staged by one workgroup per CU (up to 1024
//                threads, 768 from five columns on, for the registers);
//   kSrcNorm     Q8(RMSNorm(x)) of the f32 vector `nin` describes, formed
//                by one workgroup of up to 1024 threads per CU.
// The last two fetch two items before the prologue and give consecutive
// tiles to different workgroups, so that every CU gets the same share.
constexpr int kSrcQ8 = 0, kSrcQ8Early = 1, kSrcNorm = 2;

template <int FMT, int NC, bool DUMP, int SRC, bool ST = false>
__global__ __launch_bounds__(SRC == kSrcQ8 ? 256 : NC >= 5 ? 64 * kWavesQ8EarlyMax : 1024)
__attribute__((amdgpu_waves_per_eu(1, NC >= 5 ? 3 : 8))) void k_gemv_q4k(
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ xq, int64_t xq_col_bytes,
    float* __restrict__ y, int32_t* __restrict__ dump_isum, int32_t* __restrict__ dump_ysum,
    int M, int nsb, int log2s, int passes, int n_tiles, NormIn nin) {
    const SpanStamp<ST> span(nin.stamp);
    extern __shared__ __align__(16) uint8_t lds[];
    const Lanes ln(log2s, nsb);
    const int nb = nsb * 8;
    const int col_bytes = stage_bytes(nb);
    const int W = gridDim.x * (blockDim.x >> 6);
    constexpr bool kEarly = SRC != kSrcQ8;
    static_assert(SRC == kSrcQ8 || SRC == kSrcQ8Early || (NC == 1 && !DUMP), "the norm prologue takes one column");
    static_assert(SRC != kSrcQ8Early || !DUMP, "early staging has no dump");
    // The norm-prologue kernel keeps the wave index (and so its few items'
    // index arithmetic) in vector registers: measured faster there; the
    // others take it as a scalar and walk their items with a cursor.
    constexpr bool kCursor = SRC != kSrcNorm;
    const int wv = kCursor ? wave_id() : (int)(threadIdx.x >> 6);
    const int wave = kEarly ? wv * (int)gridDim.x + (int)blockIdx.x : blockIdx.x * (blockDim.x >> 6) + wv;
    const int my_tiles = wave < n_tiles ? (n_tiles - 1 - wave) / W + 1 : 0;
    const int n_items = my_tiles * passes;
    const int64_t row_bytes = (int64_t)nsb * kQ4KBytes;

    // Items past the wave's last one re-read that item's lines and are not
    // computed: those requests merge with the real ones in the cache,
    // whereas one fixed address for all waves would queue thousands of
    // requests on a single channel.
    struct Item {
        typename GroupLoad<FMT>::type L;
        bool valid;
        int row, pass;
    };
    // Item (tile t, pass p) reads the lane's super-block at byte offset
    // (t*R + row_local)*row_bytes + (p*gpp + g)*144: a wave-uniform part plus
    // the lane's constant lane_off.  stream_items fetches items in order, so
    // with kCursor a wave-uniform cursor (the tile's first row, the pass and
    // their offset) advances one item per fetch instead of dividing the
    // item index.  Past the wave's last item the fetch stays on it.
    const uint32_t lane_off = (uint32_t)ln.row_local * (uint32_t)row_bytes + (uint32_t)(ln.g * kQ4KBytes);
    int c_row0 = wave * ln.R, c_pass = 0, c_done = 0;
    uint32_t c_off = (uint32_t)c_row0 * (uint32_t)row_bytes;
    const uint32_t pass_bytes = (uint32_t)(ln.gpp * kQ4KBytes);
    const uint32_t wrap_bytes = (uint32_t)(W * ln.R) * (uint32_t)row_bytes - (uint32_t)passes * pass_bytes;
    auto fetch = [&](int i, Item& it) {
        int row0;
        uint32_t off;
        bool past;
        if constexpr (kCursor) {
            past = c_done >= n_items;
            it.pass = c_pass;
            row0 = c_row0;
            off = c_off;
            if (!past && ++c_done < n_items) {
                c_off += pass_bytes;
                if (++c_pass == passes) {
                    c_pass = 0;
                    c_row0 += W * ln.R;
                    c_off += wrap_bytes;
                }
            }
        } else {
            past = i >= n_items;
            const int ii = past ? (n_items > 0 ? n_items - 1 : 0) : i;
            it.pass = ii % passes;
            row0 = (wave + (ii / passes) * W) * ln.R;
            off = (uint32_t)row0 * (uint32_t)row_bytes + (uint32_t)it.pass * pass_bytes;
        }
        it.row = past ? M : row0 + ln.row_local;
        const bool inb = n_items > 0 && ln.row_local < M - row0 && ln.g < nsb - it.pass * ln.gpp;
        it.valid = inb && !past;
        load_group_off(w, inb ? off + lane_off : 0u, ln.j, it.L);
    };

    // Early sources: the activation is requested first, then items 0 and
    // 1, whose weight loads are in flight while the prologue stages it.
    float4 xr[kNormRegChunks];
    Q8Regs qr;
    const float* xin = nullptr;
    if constexpr (SRC == kSrcNorm) {
        xin = norm_row(nin, nsb * 256);
        norm_load(xin, nsb * 256, xr);
    }
    if constexpr (SRC == kSrcQ8Early) {
        if constexpr (NC == 1) stage_q8_load(xq, nb, qr);
        else stage_q8_load_cols(xq, xq_col_bytes, nb, NC, qr);
    }
    Item A, B;
    fetch(0, A);
    if constexpr (kEarly) fetch(1, B);
    if constexpr (SRC == kSrcNorm) {
        __shared__ double sh[16];
        stage_norm_input(nin, xin, nsb * 256, xr, lds, sh);
    } else if constexpr (SRC == kSrcQ8Early) {
        if constexpr (NC == 1) stage_q8_store(xq, nb, qr, lds);
        else stage_q8_store_cols(xq, xq_col_bytes, nb, NC, qr, lds, col_bytes);
    } else {
        stage_q8_cols<4>(xq, xq_col_bytes, 0, nb, NC, lds, col_bytes, (DUMP && blockIdx.x == 0) ? dump_ysum : nullptr);
    }
    __syncthreads();

    double acc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = 0.0;
    stream_items<kEarly>(n_items, A, B, fetch, [&](const Item& it) {
        if constexpr (FMT == kFmtQ4K) {
            const int a = it.valid ? pass_lds_base(ln, it.pass) + ln.lds_lane : ln.lds_inval;
            sb_item_at<NC, DUMP>(it.L, ln, a, pair_of(ln, it.pass), it.valid, lds, col_bytes, acc, dump_isum,
                                 (int64_t)it.row * nb);
        } else {
            group_item<NC, DUMP>(it.L, ln, pair_of(ln, it.pass), it.valid, lds, col_bytes, acc, dump_isum,
                                 (int64_t)it.row * nb);
        }
        if (it.pass != passes - 1) return;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const double v = group_sum_f64(acc[c], ln.log2s);
            if ((ln.lane & (ln.S - 1)) == 0 && it.row < M) y[(int64_t)it.row * NC + c] = (float)v;
            acc[c] = 0.0;
        }
    });
}

// --------------------------------------------------------------------------
// Split-k: workgroup column s covers super-blocks [16s, 16s+16) of every row
// (one staging group per activation column), rows in slots of 64 lanes; the
// f64 partial of each (split, row, column) goes to `part` and a second kernel
// sums the splits in order.
template <int FMT, int NC>
__global__ __launch_bounds__(256) void k_gemv_q4k_splitk(
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ xq, int64_t xq_col_bytes,
    double* __restrict__ part, int M, int nsb) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int split = blockIdx.y;
    const int sb0 = 16 * split;
    const int nsb_s = min(16, nsb - sb0);
    const Lanes ln(6, nsb_s);
    const int W = gridDim.x * (blockDim.x >> 6);
    const int wave = blockIdx.x * (blockDim.x >> 6) + wave_id();
    const int n_items = wave < M ? (M - 1 - wave) / W + 1 : 0;
    const int64_t row_bytes = (int64_t)nsb * kQ4KBytes;
    const bool lane_ok = ln.g < nsb_s;

    auto where = [&](int i, const uint8_t*& p, int& row) {
        if (i >= n_items) { p = w; row = 0; return; }
        row = wave + i * W;
        p = w + row * row_bytes + (lane_ok ? (sb0 + ln.g) * kQ4KBytes : 0);
    };
    typename GroupLoad<FMT>::type A, B;
    const uint8_t* pa;
    int ra = 0;
    if (n_items > 0) {
        where(0, pa, ra);
        load_group(pa, ln.j, A);
    }
    stage_q8_cols<4>(xq, xq_col_bytes, 8 * sb0, 8 * nsb_s, NC, lds, kStageGroupBytes, nullptr);
    __syncthreads();

    auto item = [&](const typename GroupLoad<FMT>::type& L, int row) {
        double acc[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[c] = 0.0;
        group_item<NC, false>(L, ln, pair_of(ln, 0), lane_ok, lds, kStageGroupBytes, acc, nullptr, 0);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const double v = wave_sum_f64(acc[c]);
            if (ln.lane == 0) part[((int64_t)split * M + row) * NC + c] = v;
        }
    };
    for (int i = 0; i < n_items; i += 2) {
        const uint8_t* pb;
        int rb;
        where(i + 1, pb, rb);
        load_group(pb, ln.j, B);
        item(A, ra);
        where(i + 2, pa, ra);
        load_group(pa, ln.j, A);
        if (i + 1 < n_items) item(B, rb);
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
// Grouped GEMV for routed experts.  Without a combine, the wave work items
// are (slot, tile, pass); with one, a wave owns a tile and walks (slot, pass)
// in slot order, forming sum_s combine[s]*y_s in f64 at the end of each
// slot.  Per slot the lane layout, arithmetic and reduction are those of
// k_gemv_q4k with the same layout, so a slot's result equals the single GEMV
// on that expert.
template <bool COMBINE>
__global__ __launch_bounds__(256) void k_gemv_q4k_grouped(
    const uint8_t* __restrict__ w_all, int64_t expert_bytes, int n_experts,
    const int32_t* __restrict__ ids, int n_sel, const uint8_t* __restrict__ xq, int64_t xq_stride,
    float* __restrict__ y, const float* __restrict__ combine, float* __restrict__ y_out,
    const int64_t* __restrict__ out_row, int64_t out_rows, int M, int nsb, int log2s, int passes,
    int n_tiles, int64_t* __restrict__ inc_step) {
    extern __shared__ __align__(16) uint8_t lds[];
    if (inc_step && blockIdx.x == 0 && threadIdx.x == 0) *inc_step += 1;
    const Lanes ln(log2s, nsb);
    const int nb = nsb * 8;
    const int col_bytes = stage_bytes(nb);
    const int n_cols = xq_stride ? n_sel : 1;
    const int W = gridDim.x * (blockDim.x >> 6);
    const int wave = blockIdx.x * (blockDim.x >> 6) + wave_id();
    // COMBINE: units are tiles, each of n_sel*passes items; else units are
    // (slot, tile) pairs of `passes` items.
    const int n_units = COMBINE ? n_tiles : n_tiles * n_sel;
    const int per_unit = COMBINE ? n_sel * passes : passes;
    const int my_units = wave < n_units ? (n_units - 1 - wave) / W + 1 : 0;
    const int n_items = my_units * per_unit;
    const int64_t row_bytes = (int64_t)nsb * kQ4KBytes;
    float* yo = y_out;

    struct Meta {
        int row, pass, slot;
        bool valid, slot_ok;
    };
    auto where = [&](int i, const uint8_t*& p, Meta& m) {
        if (i >= n_items) { p = w_all; m = Meta{M, 0, 0, false, false}; return; }
        const int u = wave + (i / per_unit) * W;
        const int r = i % per_unit;
        const int tile = COMBINE ? u : u % n_tiles;
        m.slot = COMBINE ? r / passes : u / n_tiles;
        m.pass = r % passes;
        m.row = tile * ln.R + ln.row_local;
        const int sb = m.pass * ln.gpp + ln.g;
        const int e = ids[m.slot];
        m.slot_ok = e >= 0 && e < n_experts;
        m.valid = m.slot_ok && m.row < M && sb < nsb;
        p = m.valid ? w_all + e * expert_bytes + m.row * row_bytes + sb * kQ4KBytes : w_all;
    };

    SBLoad A, B;
    const uint8_t* pa;
    Meta ma{0, 0, 0, false, false};
    if (n_items > 0) {
        where(0, pa, ma);
        load_sb(pa, 32 * ln.j, A);
    }
    for (int c = 0; c < n_cols; ++c)
        stage_q8(xq + c * xq_stride, 0, nb, lds + c * col_bytes, threadIdx.x, blockDim.x, nullptr);
    __syncthreads();
    if (n_items == 0) return;
    if (COMBINE && out_row) yo += (int64_t)(*out_row % out_rows) * M;

    double acc[1] = {0.0};
    double comb = 0.0;
    auto item = [&](const SBLoad& L, const Meta& m) {
        const uint8_t* xs = lds + (xq_stride ? m.slot : 0) * col_bytes;
        sb_item<1, false>(L, ln, pair_of(ln, m.pass), m.valid, xs, col_bytes, acc, nullptr, 0);
        if (m.pass != passes - 1) return;
        const double v = group_sum_f64(acc[0], ln.log2s);
        acc[0] = 0.0;
        const float ys = m.slot_ok ? (float)v : __builtin_nanf("");
        const bool writer = (ln.lane & (ln.S - 1)) == 0 && m.row < M;
        if (writer && y) y[(int64_t)m.slot * M + m.row] = ys;
        if (COMBINE) {
            comb += (double)combine[m.slot] * (double)ys;
            if (m.slot == n_sel - 1) {
                if (writer) yo[m.row] = (float)comb;
                comb = 0.0;
            }
        }
    };
    for (int i = 0; i < n_items; i += 2) {
        const uint8_t* pb;
        Meta mb;
        where(i + 1, pb, mb);
        load_sb(pb, 32 * ln.j, B);
        item(A, ma);
        where(i + 2, pa, ma);
        load_sb(pa, 32 * ln.j, A);
        if (i + 1 < n_items) item(B, mb);
    }
}


// --------------------------------------------------------------------------
// Gate/up GEMV with the SwiGLU stand-in fused.  Workgroup u owns outputs
// [32u, 32u+32): gate rows 32u..32u+31 and up rows inter+32u..+31, so it can
// finish whole q8_0 blocks itself.  Rows use 16-lane slots (4 rows a tile);
// with WV waves, wave q takes gate rows 32u + (32/WV)q .. +32/WV-1 and the
// matching up rows, 8/WV tiles of each.  The per-row arithmetic and
// reduction are those of k_gemv_q4k with 16-lane slots, so gate and up
// values are the ones the plain GEMV would write.  With NORM the input is
// Q8(RMSNorm(x)) formed in the prologue (8 waves, so that fewer
// workgroups repeat it); otherwise xq (4 waves).
template <int FMT, bool NORM, bool ST = false>
__global__ __launch_bounds__(NORM ? 512 : 256) void k_gemv_q4k_swiglu(
    const uint8_t* __restrict__ w, const uint8_t* __restrict__ xq, float* __restrict__ gu_out,
    uint8_t* __restrict__ g_q8, int inter, int nsb, NormIn nin, double* __restrict__ part,
    unsigned* __restrict__ cnt) {
    const SpanStamp<ST> span(nin.stamp);
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ float gu_s[64];
    __shared__ double gu_d[64];
    constexpr int WV = NORM ? 8 : 4;        // waves per workgroup
    constexpr int TPH = 8 / WV;             // tiles per half (gate or up) per wave
    const Lanes ln(4, nsb);
    const int nb = nsb * 8;
    // The last NS output blocks are split along K into two halves (their
    // first and last passes), run by workgroups 0 .. 2*NS-1 so that they
    // start first; the other blocks follow, one workgroup each.  A half
    // leaves its f64 row sums in `part`; the second half to finish adds the
    // two (addition commutes, so the order of arrival does not matter) and
    // writes the block.  NS = gridDim.x - inter/32.
    const int nblk = inter / 32, NS = (int)gridDim.x - nblk;
    const bool half = (int)blockIdx.x < 2 * NS;
    const int hs = (int)blockIdx.x & 1;                     // which half
    const int u = half ? nblk - NS + (int)blockIdx.x / 2 : (int)blockIdx.x - 2 * NS;
    const int passes_all = (nsb + 3) / 4;
    const int p0 = half && hs ? passes_all / 2 : 0;
    const int passes = half ? (hs ? passes_all - passes_all / 2 : passes_all / 2) : passes_all;
    const int n_items = 2 * TPH * passes;
    const int q = wave_id();
    const int64_t row_bytes = (int64_t)nsb * kQ4KBytes;

    // item i: tile st = i / passes (st / TPH: 0 gate, 1 up; st % TPH: which
    // tile of the half), pass i % passes
    auto local_of = [&](int st) { return (32 / WV) * q + 4 * (st % TPH) + ln.row_local; };
    auto row_of = [&](int st) { return (st / TPH) * inter + 32 * u + local_of(st); };
    // Items past the last re-read the last item's lines (see k_gemv_q4k)
    // and are not computed.
    struct Item {
        typename GroupLoad<FMT>::type L;
        bool valid;
        int st, pass;
    };
    // An in-order cursor over (st, pass), as in k_gemv_q4k.
    const uint32_t lane_off = (uint32_t)ln.row_local * (uint32_t)row_bytes + (uint32_t)(ln.g * kQ4KBytes);
    int c_st = 0, c_pass = 0, c_done = 0;
    auto fetch = [&](int, Item& it) {
        const bool past = c_done >= n_items;
        it.st = c_st;
        it.pass = p0 + c_pass;
        const bool inb = ln.g < nsb - it.pass * ln.gpp;
        it.valid = inb && !past;
        const int row0 = row_of(it.st) - ln.row_local;
        const uint32_t off = (uint32_t)row0 * (uint32_t)row_bytes + (uint32_t)(it.pass * ln.gpp * kQ4KBytes);
        load_group_off(w, inb ? off + lane_off : 0u, ln.j, it.L);
        if (!past && ++c_done < n_items && ++c_pass == passes) {
            c_pass = 0;
            ++c_st;
        }
    };

    float4 xr[kNormRegChunks];
    const float* xin = nullptr;
    if constexpr (NORM) {
        xin = norm_row(nin, nsb * 256);
        norm_load(xin, nsb * 256, xr);
    }
    Item A, B;
    fetch(0, A);
    if constexpr (NORM) fetch(1, B);
    if constexpr (NORM) {
        __shared__ double sh[16];
        stage_norm_input(nin, xin, nsb * 256, xr, lds, sh);
    } else {
        stage_q8(xq, 0, nb, lds, threadIdx.x, blockDim.x, nullptr);
    }
    __syncthreads();

    double acc[1] = {0.0};
    stream_items<NORM>(n_items, A, B, fetch, [&](const Item& it) {
        if constexpr (FMT == kFmtQ4K) {
            const int a = it.valid ? pass_lds_base(ln, it.pass) + ln.lds_lane : ln.lds_inval;
            sb_item_at<1, false>(it.L, ln, a, 0, it.valid, lds, 0, acc, nullptr, 0);
        } else {
            group_item<1, false>(it.L, ln, pair_of(ln, it.pass), it.valid, lds, 0, acc, nullptr, 0);
        }
        if (it.pass != p0 + passes - 1) return;
        const double v = group_sum_f64(acc[0], 4);
        acc[0] = 0.0;
        if ((ln.lane & 15) == 0) {
            const int r = (it.st / TPH) * 32 + local_of(it.st);
            if (half) {
                gu_d[r] = v;
            } else {
                gu_s[r] = (float)v;
                if (gu_out) gu_out[row_of(it.st)] = (float)v;
            }
        }
    });
    __syncthreads();
    if (q != 0) return;
    const int i = ln.lane;
    if (half) {
        // Row sums of this half to `part`, then the block's counter; the
        // second arrival reads the other half's sums.  The sums are stored
        // and read with agent-scope accesses, which go through the L2 to the
        // device's coherence point, so ordering needs only the wait for the
        // stores' completion before the counter moves, and the reads are
        // issued after the counter's value has returned.  Agent-scope fences
        // would instead write back and invalidate the whole L2 of the XCD,
        // once per half: that cost more than the split saves.
        const int sblk = u - (nblk - NS);
        double* mine = part + (int64_t)(2 * sblk + hs) * 64;
        const double* other = part + (int64_t)(2 * sblk + (hs ^ 1)) * 64;
        const double own = gu_d[i];
        __hip_atomic_store(mine + i, own, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        unsigned prev = 0;
        if (i == 0) prev = __hip_atomic_fetch_add(cnt + sblk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prev = __builtin_amdgcn_readfirstlane(prev);
        if (prev == 0) return;                  // the other half finishes the block
        asm volatile("" ::: "memory");
        const float v = (float)(own + __hip_atomic_load(other + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        gu_s[i] = v;
        if (gu_out) gu_out[(i / 32) * inter + 32 * u + (i & 31)] = v;
        if (i == 0) __hip_atomic_store(cnt + sblk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const float a = i < 32 ? swiglu_value(gu_s[i], gu_s[32 + i]) : 0.0f;
    quantize_lane(a, g_q8 + (int64_t)u * kQ8Bytes, i & 31, i < 32);
}

// --------------------------------------------------------------------------
// Grouped GEMV with the weighted combine, slots in parallel: wave s of a
// workgroup computes slot s (expert ids[s], activation column s) for the
// workgroup's tiles [tpw*g, tpw*g + tpw) over all passes, keeping each row's
// result in LDS; after a barrier the workgroup forms y_out[r] =
// sum_s combine[s]*y_s[r] in f64 in slot order (the order of
// k_gemv_q4k_grouped<true>, so the results are the same).  n_sel waves.
__global__ __launch_bounds__(1024) void k_gemv_q4k_grouped_combine(
    const uint8_t* __restrict__ w_all, int64_t expert_bytes, int n_experts,
    const int32_t* __restrict__ ids, int n_sel, const uint8_t* __restrict__ xq, int64_t xq_stride,
    const float* __restrict__ combine, float* __restrict__ y_out, const int64_t* __restrict__ out_row,
    int64_t out_rows, int M, int nsb, int log2s, int passes, int n_tiles, int tpw,
    int64_t* __restrict__ inc_step, const int32_t* __restrict__ ids_table, int32_t* __restrict__ ids_next) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ float res[16 * 64];          // [slot][tile in the workgroup][row in the tile]
    // The first wave of workgroup 0 advances the token counter (out_rows
    // tokens) and, with ids_next, hands the next token's routing ids to the
    // next gate/up kernel, which then need not wait for the counter to read
    // them.  The counter is read first, the ids once it has arrived, and
    // both are stored at the end, so no wait lands before the weights.
    const bool counter = inc_step && blockIdx.x == 0 && threadIdx.x < 64;
    const bool hand = counter && ids_next && (int)threadIdx.x < n_sel;
    int64_t next = 0;
    if (counter && (threadIdx.x == 0 || hand)) next = *inc_step + 1;
    const Lanes ln(log2s, nsb);
    const int nb = nsb * 8;
    const int col_bytes = stage_bytes(nb);
    const int slot = wave_id();
    const int t0 = (int)blockIdx.x * tpw;
    const int n_items = tpw * passes;
    const int64_t row_bytes = (int64_t)nsb * kQ4KBytes;
    const int e = ids[slot];
    const bool slot_ok = e >= 0 && e < n_experts;

    // Items past the last re-read the last item's lines and are not computed.
    struct Item {
        SBLoad L;
        bool valid;
        int k, row, pass;
    };
    auto fetch = [&](int i, Item& it) {
        const bool past = i >= n_items;
        const int ii = past ? n_items - 1 : i;
        it.k = ii / passes;
        it.pass = ii % passes;
        it.row = (t0 + it.k) * ln.R + ln.row_local;
        const int sb = it.pass * ln.gpp + ln.g;
        const bool inb = slot_ok && it.row < M && sb < nsb;
        it.valid = inb && !past;
        load_sb(inb ? w_all + e * expert_bytes + (int64_t)it.row * row_bytes + sb * kQ4KBytes : w_all,
                32 * ln.j, it.L);
    };

    // Contiguous slot columns (the expert chain's) are staged as one vector,
    // slot s's pairs starting at s*nb/2: their loads go out together with the
    // ids, before the weights, and both weight items are requested before
    // the staging stores.  Otherwise each column is staged on its own after
    // the first item is requested.
    const bool contig = xq_stride == (int64_t)nb * kQ8Bytes;
    Item A, B;
    if (contig) {
        Q8Regs qr;
        stage_q8_load(xq, n_sel * nb, qr);
        fetch(0, A);
        fetch(1, B);
        stage_q8_store(xq, n_sel * nb, qr, lds);
    } else {
        fetch(0, A);
        for (int c = 0; c < n_sel; ++c)
            stage_q8(xq + c * xq_stride, 0, nb, lds + c * col_bytes, threadIdx.x, blockDim.x, nullptr);
    }
    int32_t next_id = 0;
    if (hand) next_id = ids_table[(int64_t)((uint64_t)next % (uint64_t)out_rows) * n_sel + threadIdx.x];
    __syncthreads();

    double acc[1] = {0.0};
    const uint8_t* xs = contig ? lds : lds + slot * col_bytes;
    const int pbase = contig ? slot * (nb / 2) : 0;
    auto use = [&](const Item& it) {
        // lanes past the row's last super-block read pair 0 (their result is dropped)
        const int P = it.valid ? pbase + pair_of(ln, it.pass) : 0;
        sb_item<1, false>(it.L, ln, P, it.valid, xs, col_bytes, acc, nullptr, 0);
        if (it.pass != passes - 1) return;
        const double v = group_sum_f64(acc[0], ln.log2s);
        acc[0] = 0.0;
        if ((ln.lane & (ln.S - 1)) == 0) res[(slot * tpw + it.k) * ln.R + ln.row_local] = slot_ok ? (float)v : __builtin_nanf("");
    };
    if (contig)
        stream_items<true>(n_items, A, B, fetch, use);
    else
        stream_items<false>(n_items, A, B, fetch, use);
    __syncthreads();
    float* yo = y_out + (out_row ? (int64_t)(*out_row % out_rows) * M : 0);
    for (int i = threadIdx.x; i < tpw * ln.R; i += blockDim.x) {
        const int row = t0 * ln.R + i;
        if (row >= M) continue;
        double comb = 0.0;
        for (int s2 = 0; s2 < n_sel; ++s2) comb += (double)combine[s2] * (double)res[s2 * tpw * ln.R + i];
        yo[row] = (float)comb;
    }
    if (counter && threadIdx.x == 0) *inc_step = next;
    if (hand) ids_next[threadIdx.x] = next_id;
}

// --------------------------------------------------------------------------
// Routed-expert gate/up with the SwiGLU epilogue, for the token t = *step mod
// n_tokens.  Workgroup (block b = blockIdx.x, slot s = blockIdx.y) computes
// gate rows 32b..32b+31 and up rows inter+32b..+31 of expert
// ids_table[t][s] against Q8(x_table[t]), quantized in its prologue, and
// writes block b of slot s of g = Q8(silu(gate)*up) (slot stride k_pad/32
// blocks); blocks at or past inter/32 (the padding up to k_pad) and slots
// whose expert id is out of range get zero blocks.  Workgroup (0, 0) also
// writes cur = t, the token's ids and combine = softmax(logits_table[t])
// (f64, slot order, rounded to f32).  Rows and arithmetic as in
// k_gemv_q4k_swiglu<true> (8 waves, 16-lane slots).
__global__ __launch_bounds__(512) void k_moe_gate_up(
    const uint8_t* __restrict__ w_all, int64_t expert_bytes, int n_experts, int inter, int nsb,
    const int64_t* __restrict__ step, int n_tokens, const int32_t* __restrict__ ids_table,
    const float* __restrict__ logits_table, const float* __restrict__ x_table, int n_sel, int64_t k_pad,
    int64_t* __restrict__ cur, int32_t* __restrict__ ids_out, float* __restrict__ combine_out,
    uint8_t* __restrict__ g_q8, float* __restrict__ gu_out, const int32_t* __restrict__ ids_next,
    int n_split, double* __restrict__ part, unsigned* __restrict__ cnt) {
    extern __shared__ __align__(16) uint8_t lds[];
    __shared__ float gu_s[64];
    __shared__ double gu_d[64];
    const Lanes ln(4, nsb);
    const int q = wave_id();
    // One workgroup per (slot, output block), in a 1-D grid.  As in
    // k_gemv_q4k_swiglu, the last n_split working blocks (slot-major) run as
    // two halves along K, workgroups 0 .. 2*n_split-1, which hand over
    // through part/cnt; the other blocks, padding included, follow.
    const int nbw = inter / 32, nbp = (int)(k_pad / 32), working = n_sel * nbw;
    const int idx = blockIdx.x;
    const bool half = idx < 2 * n_split;
    const int hs = idx & 1;
    int slot, b;
    if (half) {
        const int lin = working - n_split + idx / 2;
        slot = lin / nbw;
        b = lin - slot * nbw;
    } else {
        const int f = idx - 2 * n_split;
        if (f < working - n_split) {
            slot = f / nbw;
            b = f - slot * nbw;
        } else {
            const int pz = f - (working - n_split), npad = nbp - nbw;
            slot = pz / npad;
            b = nbw + (pz - slot * npad);
        }
    }
    const int passes_all = (nsb + 3) / 4;
    const int p0 = half && hs ? passes_all / 2 : 0;
    const int passes = half ? (hs ? passes_all - passes_all / 2 : passes_all / 2) : passes_all;
    const int64_t t = (int64_t)((uint64_t)*step % (uint64_t)n_tokens);
    // ids_next, when given, already holds token t's ids (see the down kernel)
    const int e = ids_next ? ids_next[slot] : ids_table[t * n_sel + slot];
    const bool e_ok = e >= 0 && e < n_experts;
    const bool work = e_ok && b < inter / 32;
    const int n_items = work ? 2 * passes : 0;
    const int64_t row_bytes = (int64_t)nsb * kQ4KBytes;
    const uint8_t* w = w_all + (e_ok ? (int64_t)e * expert_bytes : 0);
    const int local = 4 * q + ln.row_local;     // row within the gate or up half of the block
    auto row_of = [&](int st) { return st * inter + 32 * b + local; };

    // Items past the last re-read the last item's lines and are not computed.
    struct Item {
        SBLoad L;
        bool valid;
        int st, pass;
    };
    auto fetch = [&](int i, Item& it) {
        const bool past = i >= n_items;
        const int ii = past ? (n_items > 0 ? n_items - 1 : 0) : i;
        it.st = ii / passes;
        it.pass = p0 + ii % passes;
        const int sb = it.pass * ln.gpp + ln.g;
        const bool inb = n_items > 0 && sb < nsb;
        it.valid = inb && !past;
        load_sb(inb ? w + (int64_t)row_of(it.st) * row_bytes + sb * kQ4KBytes : w_all, 32 * ln.j, it.L);
    };

    const float* x = x_table + t * (int64_t)(nsb * 256);
    float4 xr[kNormRegChunks];
    if (work) norm_load(x, nsb * 256, xr);
    Item A, B;
    fetch(0, A);
    fetch(1, B);
    if (work) stage_scaled_q8(x, nsb * 256, xr, 1.0f, false, lds, nullptr);
    if (b == 0 && slot == 0 && q == 0) {
        // combine = softmax of the router logits, in slot order like a
        // sequential loop: lane i holds logit i, every lane adds the
        // exponentials in slot order
        const int i = ln.lane;
        const double l = i < n_sel ? (double)logits_table[t * n_sel + i] : -INFINITY;
        double mx = l;
        for (int j = 0; j < n_sel; ++j) mx = fmax(mx, __shfl(l, j));
        const double ex = exp(l - mx);
        double sum = 0.0;
        for (int j = 0; j < n_sel; ++j) sum += __shfl(ex, j);
        if (i < n_sel) {
            combine_out[i] = (float)(ex / sum);
            ids_out[i] = ids_next ? ids_next[i] : ids_table[t * n_sel + i];
        }
        if (i == 0) *cur = t;
    }
    __syncthreads();

    double acc[1] = {0.0};
    stream_items<true>(n_items, A, B, fetch, [&](const Item& it) {
        group_item<1, false>(it.L, ln, pair_of(ln, it.pass), it.valid, lds, 0, acc, nullptr, 0);
        if (it.pass != p0 + passes - 1) return;
        const double v = group_sum_f64(acc[0], 4);
        acc[0] = 0.0;
        if ((ln.lane & 15) == 0) {
            if (half) {
                gu_d[it.st * 32 + local] = v;
            } else {
                gu_s[it.st * 32 + local] = (float)v;
                if (gu_out) gu_out[(int64_t)slot * 2 * inter + row_of(it.st)] = (float)v;
            }
        }
    });
    __syncthreads();
    if (q != 0) return;
    const int i = ln.lane;
    if (half) {
        // The hand-over of k_gemv_q4k_swiglu.  A half whose expert id is out
        // of range has no items; its sums are zero, and so is the block.
        const int sblk = idx / 2;
        double* mine = part + (int64_t)(2 * sblk + hs) * 64;
        const double* other = part + (int64_t)(2 * sblk + (hs ^ 1)) * 64;
        const double own = work ? gu_d[i] : 0.0;
        __hip_atomic_store(mine + i, own, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        unsigned prev = 0;
        if (i == 0) prev = __hip_atomic_fetch_add(cnt + sblk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prev = __builtin_amdgcn_readfirstlane(prev);
        if (prev == 0) return;
        asm volatile("" ::: "memory");
        const float v = (float)(own + __hip_atomic_load(other + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        gu_s[i] = v;
        if (gu_out && work) gu_out[(int64_t)slot * 2 * inter + (i / 32) * inter + 32 * b + (i & 31)] = v;
        if (i == 0) __hip_atomic_store(cnt + sblk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const float a = work && i < 32 ? swiglu_value(gu_s[i], gu_s[32 + i]) : 0.0f;
    quantize_lane(a, g_q8 + ((int64_t)slot * (k_pad / 32) + b) * kQ8Bytes, i & 31, i < 32);
}

// --------------------------------------------------------------------------
// Host side.

struct LaunchEvents {
    std::vector<hipEvent_t> starts, stops;
    size_t next = 0;
};
static thread_local LaunchEvents t_events;

void set_next_launch_events(const hipEvent_t* starts, const hipEvent_t* stops, int n) {
    t_events.starts.assign(starts, starts + n);
    t_events.stops.assign(stops, stops + n);
    t_events.next = 0;
}

bool take_next_launch_events(hipEvent_t* start, hipEvent_t* stop) {
    if (t_events.next >= t_events.starts.size()) return false;
    *start = t_events.starts[t_events.next];
    *stop = t_events.stops[t_events.next];
    ++t_events.next;
    return true;
}

// Launch through hipExtLaunchKernelGGL when a measurement hook is armed.
// The stream is drained first: a dispatch queued behind a running kernel
// would otherwise take its start timestamp before it can begin executing.
#define MQ_LAUNCH(kernel, grid, block, lds, stream, ...)                                         \
    do {                                                                                        \
        hipEvent_t ev0_, ev1_;                                                                  \
        if (take_next_launch_events(&ev0_, &ev1_)) {                                            \
            (void)hipStreamSynchronize(stream);                                                 \
            hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ev0_, ev1_, 0, __VA_ARGS__); \
        } else {                                                                                \
            hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                  \
        }                                                                                       \
    } while (0)

// Both caches below are filled on first use and may be read and filled by
// several host threads at once: the CU count per device is an atomic, the
// occupancy table sits behind a mutex.
int device_cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Resident workgroups of `threads` threads per CU for kernel fn with `lds`
// bytes of dynamic LDS on the current device (occupancy query, cached).
int blocks_per_cu(const void* fn, int threads, int lds) {
    struct Entry { int dev; const void* fn; int threads, lds, n; };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    (void)hipGetDevice(&dev);
    {
        std::lock_guard<std::mutex> lock(mu);
        for (const Entry& e : cache)
            if (e.dev == dev && e.fn == fn && e.threads == threads && e.lds == lds) return e.n;
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, lds) != hipSuccess || n <= 0) n = 2;
    std::lock_guard<std::mutex> lock(mu);
    cache.push_back(Entry{dev, fn, threads, lds, n});
    return n;
}

static int ceil_log2(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

// Lane layout for m rows of nsb super-blocks, `mult` independent copies
// (grouped slots): prefer enough tiles to give every CU ~16 waves, then few
// idle lanes, then the narrowest slot (cheapest row reduction).
Q4KPlan plan_q4k_mult(int64_t m, int nsb, int mult) {
    const int64_t target = (int64_t)device_cu_count() * 16;
    Q4KPlan best{6, 1, 1, 1};
    double best_score = -1.0;
    const int lo = nsb < 4 ? ceil_log2(4 * nsb) : 4;
    for (int l = (lo < 2 ? 2 : lo); l <= 6; ++l) {
        const int gpp = (1 << l) / 4;
        const int passes = (nsb + gpp - 1) / gpp;
        const double used = (double)nsb / (passes * gpp);
        const int64_t tiles = (m + (64 >> l) - 1) / (64 >> l);
        const double work = (double)(tiles * mult < target ? tiles * mult : target);
        const double score = work * used;
        if (score > best_score * 1.0001) {
            best_score = score;
            best = Q4KPlan{l, 64 >> l, passes, (int)tiles};
        }
    }
    return best;
}

Q4KPlan plan_q4k(int64_t m, int nsb) { return plan_q4k_mult(m, nsb, 1); }

// Waves to launch for `units` equal work units: all resident at once and
// every wave with the same number of units (or one fewer).
static int balanced_grid(int64_t units, const void* fn, int lds) {
    const int64_t wmax = (int64_t)device_cu_count() * blocks_per_cu(fn, 256, lds) * 4;
    const int64_t k = (units + wmax - 1) / wmax;
    const int64_t waves = (units + k - 1) / k;
    const int64_t grid = (waves + 3) / 4;
    return (int)(grid > 0 ? grid : 1);
}

template <int FMT, int NC, bool DUMP>
static hipError_t launch_nc(const void* w, const void* xq, int64_t xq_col_bytes, float* y,
                            int32_t* dump_isum, int32_t* dump_ysum, int64_t m, int nsb,
                            hipStream_t stream) {
    const Q4KPlan p = plan_q4k(m, nsb);
    const int lds = NC * stage_bytes(nsb * 8);
    const void* fn = (const void*)k_gemv_q4k<FMT, NC, DUMP, kSrcQ8>;
    MQ_LAUNCH((k_gemv_q4k<FMT, NC, DUMP, kSrcQ8>), dim3(balanced_grid(p.n_tiles, fn, lds)), dim3(256), lds,
              stream, (const uint8_t*)w, (const uint8_t*)xq, xq_col_bytes, y, dump_isum, dump_ysum, (int)m, nsb,
              p.log2s, p.passes, p.n_tiles, NormIn{});
    return hipGetLastError();
}

// Grid of a GEMV whose workgroups each stage the activation in a prologue
// of `prologue` per-thread steps: at most one workgroup per CU, so the
// prologue is repeated about once per CU, and enough waves (up to 16) that
// every thread takes at most one step when possible (a prologue is bound by
// each wave's instruction latency, not by the CU's issue rate).  Waves loop
// over `units` equal work units.
void prologue_grid(int64_t units, int64_t prologue, int* grid, int* threads, int max_waves) {
    const int64_t cus = device_cu_count();
    const int64_t g = units < cus ? units : cus;
    const int64_t for_units = (units + g - 1) / g;
    const int64_t for_chunks = (prologue + 63) / 64;
    int64_t wpg = for_units > for_chunks ? for_units : for_chunks;
    if (wpg > max_waves) wpg = max_waves;
    if (wpg < 1) wpg = 1;
    *grid = (int)(g > 0 ? g : 1);
    *threads = (int)(64 * wpg);
}

// One q8_0 column with early staging (see k_gemv_q4k).
template <int FMT>
static hipError_t launch_q8_early(const void* w, const void* xq, float* y, int64_t m, int nsb,
                                  hipStream_t stream, uint64_t* stamp = nullptr) {
    const Q4KPlan p = plan_q4k(m, nsb);
    const int lds = stage_bytes(nsb * 8);
    // waves per CU for about kItemsPerWave items each, within [7, 12]
    const int64_t per_cu = (int64_t)device_cu_count() * kItemsPerWave;
    const int64_t want = ((int64_t)p.n_tiles * p.passes + per_cu - 1) / per_cu;
    const int cap = (int)(want < kWavesQ8EarlyMin ? kWavesQ8EarlyMin : want > kWavesQ8EarlyMax ? kWavesQ8EarlyMax : want);
    int grid = 1, threads = 64;
    prologue_grid(p.n_tiles, (nsb * 8 + kStageRegBlocks - 1) / kStageRegBlocks, &grid, &threads, cap);
    if (stamp) {
        MQ_LAUNCH((k_gemv_q4k<FMT, 1, false, kSrcQ8Early, true>), dim3(grid), dim3(threads), lds, stream,
                  (const uint8_t*)w, (const uint8_t*)xq, (int64_t)0, y, (int32_t*)nullptr, (int32_t*)nullptr,
                  (int)m, nsb, p.log2s, p.passes, p.n_tiles, NormIn{nullptr, nullptr, 0, 0.0f, nullptr, nullptr, 0, stamp});
    } else {
        MQ_LAUNCH((k_gemv_q4k<FMT, 1, false, kSrcQ8Early>), dim3(grid), dim3(threads), lds, stream,
                  (const uint8_t*)w, (const uint8_t*)xq, (int64_t)0, y, (int32_t*)nullptr, (int32_t*)nullptr,
                  (int)m, nsb, p.log2s, p.passes, p.n_tiles, NormIn{});
    }
    return hipGetLastError();
}

hipError_t launch_gemv_q4k_q8_stamped(const void* w, const void* xq, float* y, int64_t m, int64_t k,
                                      hipStream_t stream, int fmt, uint64_t* stamp) {
    if (m > max_rows_per_launch(k)) return hipErrorInvalidValue;
    const int nsb = (int)(k / 256);
    return fmt == kFmtQ4_0 ? launch_q8_early<kFmtQ4_0>(w, xq, y, m, nsb, stream, stamp)
                           : launch_q8_early<kFmtQ4K>(w, xq, y, m, nsb, stream, stamp);
}

template <int FMT>
static hipError_t launch_norm(const void* w, const NormIn& nin, float* y, int64_t m, int64_t k,
                              hipStream_t stream) {
    const int nsb = (int)(k / 256);
    const Q4KPlan p = plan_q4k(m, nsb);
    const int lds = stage_bytes(nsb * 8);
    int grid = 1, threads = 64;
    prologue_grid(p.n_tiles, k / 4, &grid, &threads, kWavesNorm);
    if (nin.stamp) {
        MQ_LAUNCH((k_gemv_q4k<FMT, 1, false, kSrcNorm, true>), dim3(grid), dim3(threads), lds, stream,
                  (const uint8_t*)w, (const uint8_t*)nullptr, (int64_t)0, y, (int32_t*)nullptr, (int32_t*)nullptr,
                  (int)m, nsb, p.log2s, p.passes, p.n_tiles, nin);
    } else {
        MQ_LAUNCH((k_gemv_q4k<FMT, 1, false, kSrcNorm>), dim3(grid), dim3(threads), lds, stream,
                  (const uint8_t*)w, (const uint8_t*)nullptr, (int64_t)0, y, (int32_t*)nullptr, (int32_t*)nullptr,
                  (int)m, nsb, p.log2s, p.passes, p.n_tiles, nin);
    }
    return hipGetLastError();
}

hipError_t launch_gemv_q4k_norm(const void* w, const NormIn& nin, float* y, int64_t m, int64_t k,
                                hipStream_t stream, int fmt) {
    return fmt == kFmtQ4_0 ? launch_norm<kFmtQ4_0>(w, nin, y, m, k, stream)
                           : launch_norm<kFmtQ4K>(w, nin, y, m, k, stream);
}

// NC q8_0 columns with early staging: the one-column GEMV's launch shape
// (one workgroup per CU, interleaved tiles, waves for about kItemsPerWave
// items each), the columns' first blocks requested before the weights and
// staged side by side (NC * stage_bytes <= kMaxStageLds, checked by the
// caller).
template <int FMT, int NC>
static hipError_t launch_q8_early_nc(const void* w, const void* xq, int64_t xq_col_bytes, float* y, int64_t m,
                                     int nsb, hipStream_t stream) {
    const Q4KPlan p = plan_q4k(m, nsb);
    const int lds = NC * stage_bytes(nsb * 8);
    const int64_t per_cu = (int64_t)device_cu_count() * kItemsPerWave;
    const int64_t want = ((int64_t)p.n_tiles * p.passes + per_cu - 1) / per_cu;
    const int cap = (int)(want < kWavesQ8EarlyMin ? kWavesQ8EarlyMin : want > kWavesQ8EarlyMax ? kWavesQ8EarlyMax : want);
    int grid = 1, threads = 64;
    prologue_grid(p.n_tiles, (NC * nsb * 8 + kStageRegBlocks - 1) / kStageRegBlocks, &grid, &threads, cap);
    MQ_LAUNCH((k_gemv_q4k<FMT, NC, false, kSrcQ8Early>), dim3(grid), dim3(threads), lds, stream, (const uint8_t*)w,
              (const uint8_t*)xq, xq_col_bytes, y, (int32_t*)nullptr, (int32_t*)nullptr, (int)m, nsb, p.log2s,
              p.passes, p.n_tiles, NormIn{});
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_fmt(const void* w, const void* xq, int64_t xq_col_bytes, float* y, int32_t* dump_isum,
                             int32_t* dump_ysum, int64_t m, int nsb, int ncols, hipStream_t stream) {
    if (dump_isum) return launch_nc<FMT, 1, true>(w, xq, xq_col_bytes, y, dump_isum, dump_ysum, m, nsb, stream);
    switch (ncols) {
        case 1: return launch_q8_early<FMT>(w, xq, y, m, nsb, stream);
        case 2: return launch_q8_early_nc<FMT, 2>(w, xq, xq_col_bytes, y, m, nsb, stream);
        case 3: return launch_q8_early_nc<FMT, 3>(w, xq, xq_col_bytes, y, m, nsb, stream);
        case 4: return launch_q8_early_nc<FMT, 4>(w, xq, xq_col_bytes, y, m, nsb, stream);
        case 5: return launch_q8_early_nc<FMT, 5>(w, xq, xq_col_bytes, y, m, nsb, stream);
        case 6: return launch_q8_early_nc<FMT, 6>(w, xq, xq_col_bytes, y, m, nsb, stream);
        case 7: return launch_nc<FMT, 7, false>(w, xq, xq_col_bytes, y, nullptr, nullptr, m, nsb, stream);
        case 8: return launch_nc<FMT, 8, false>(w, xq, xq_col_bytes, y, nullptr, nullptr, m, nsb, stream);
        default: return hipErrorInvalidValue;
    }
}

int64_t max_rows_per_launch(int64_t k) { return (((int64_t)1 << 32) - 1) / ((k / 256) * kQ4KBytes); }

hipError_t launch_gemv_q4k(const void* w, const void* xq, int64_t xq_col_bytes, float* y,
                           int32_t* dump_isum, int32_t* dump_ysum, int64_t m, int64_t k, int ncols,
                           hipStream_t stream, int fmt) {
    const int nsb = (int)(k / 256);
    // the kernels address the matrix with 32-bit offsets: row blocks under 4 GiB
    const int64_t step = max_rows_per_launch(k), row_bytes = (int64_t)nsb * kQ4KBytes;
    for (int64_t r0 = 0; r0 < m; r0 += step) {
        const int64_t mr = m - r0 < step ? m - r0 : step;
        const uint8_t* wr = (const uint8_t*)w + r0 * row_bytes;
        float* yr = y + r0 * ncols;
        int32_t* ir = dump_isum ? dump_isum + r0 * (k / 32) : nullptr;
        const hipError_t e =
            fmt == kFmtQ4_0 ? launch_fmt<kFmtQ4_0>(wr, xq, xq_col_bytes, yr, ir, dump_ysum, mr, nsb, ncols, stream)
                            : launch_fmt<kFmtQ4K>(wr, xq, xq_col_bytes, yr, ir, dump_ysum, mr, nsb, ncols, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

int gemv_q4k_splitk_nsplit(int64_t k) { return (int)((k / 256 + 15) / 16); }

template <int FMT, int NC>
static hipError_t launch_split_nc(const void* w, const void* xq, int64_t xq_col_bytes, float* y,
                                  double* part, int64_t m, int nsb, hipStream_t stream) {
    const int n_split = (nsb + 15) / 16;
    const int lds = NC * kStageGroupBytes;
    const void* fn = (const void*)k_gemv_q4k_splitk<FMT, NC>;
    const int64_t wmax = (int64_t)device_cu_count() * blocks_per_cu(fn, 256, lds) * 4 / n_split;
    const int64_t k = (m + (wmax > 0 ? wmax : 1) - 1) / (wmax > 0 ? wmax : 1);
    const int64_t waves = (m + k - 1) / k;
    const int gx = (int)((waves + 3) / 4);
    MQ_LAUNCH((k_gemv_q4k_splitk<FMT, NC>), dim3(gx, n_split), dim3(256), lds, stream,
                       (const uint8_t*)w, (const uint8_t*)xq, xq_col_bytes, part, (int)m, nsb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_splitk_finalize(part, y, m * NC, n_split, stream);
}

hipError_t launch_splitk_finalize(const double* part, float* y, int64_t n, int n_split, hipStream_t stream) {
    hipLaunchKernelGGL(k_splitk_finalize, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, part, y, n,
                       n_split);
    return hipGetLastError();
}

template <int FMT>
static hipError_t launch_split_fmt(const void* w, const void* xq, int64_t xq_col_bytes, float* y, double* part,
                                   int64_t m, int nsb, int ncols, hipStream_t stream) {
    switch (ncols) {
        case 1: return launch_split_nc<FMT, 1>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 2: return launch_split_nc<FMT, 2>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 3: return launch_split_nc<FMT, 3>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 4: return launch_split_nc<FMT, 4>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 5: return launch_split_nc<FMT, 5>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 6: return launch_split_nc<FMT, 6>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 7: return launch_split_nc<FMT, 7>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        case 8: return launch_split_nc<FMT, 8>(w, xq, xq_col_bytes, y, part, m, nsb, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_q4k_splitk(const void* w, const void* xq, int64_t xq_col_bytes, float* y,
                                  double* part, int64_t m, int64_t k, int ncols, hipStream_t stream, int fmt) {
    const int nsb = (int)(k / 256);
    return fmt == kFmtQ4_0 ? launch_split_fmt<kFmtQ4_0>(w, xq, xq_col_bytes, y, part, m, nsb, ncols, stream)
                           : launch_split_fmt<kFmtQ4K>(w, xq, xq_col_bytes, y, part, m, nsb, ncols, stream);
}

template <int FMT>
static hipError_t launch_swiglu(const void* w, const void* xq, const NormIn* nin, float* gu_out, void* g_q8,
                                int64_t inter, int64_t k, hipStream_t stream, double* part, unsigned* cnt,
                                int n_split) {
    const int nsb = (int)(k / 256);
    const int lds = stage_bytes(nsb * 8);
    const unsigned nblk = (unsigned)(inter / 32);
    if (nin) {
        // halves need two passes or more; the hand-over space is the caller's
        const bool ok = part && cnt && n_split > 0 && n_split <= (int)nblk && (nsb + 3) / 4 >= 2;
        const int ns = ok ? n_split : 0;
        if (nin->stamp)
            MQ_LAUNCH((k_gemv_q4k_swiglu<FMT, true, true>), dim3(nblk + (unsigned)ns), dim3(512), lds, stream,
                      (const uint8_t*)w, (const uint8_t*)nullptr, gu_out, (uint8_t*)g_q8, (int)inter, nsb, *nin, part,
                      cnt);
        else
            MQ_LAUNCH((k_gemv_q4k_swiglu<FMT, true>), dim3(nblk + (unsigned)ns), dim3(512), lds, stream,
                      (const uint8_t*)w, (const uint8_t*)nullptr, gu_out, (uint8_t*)g_q8, (int)inter, nsb, *nin, part,
                      cnt);
    } else {
        MQ_LAUNCH((k_gemv_q4k_swiglu<FMT, false>), dim3(nblk), dim3(256), lds, stream,
                  (const uint8_t*)w, (const uint8_t*)xq, gu_out, (uint8_t*)g_q8, (int)inter, nsb, NormIn{},
                  (double*)nullptr, (unsigned*)nullptr);
    }
    return hipGetLastError();
}

// Blocks to split in two K-halves: those beyond a multiple of the CU count,
// or, when even the doubled count leaves CUs idle (a small gate/up such as
// one tensor-parallel rank's share), every block.  K must take at least two
// passes.
int swiglu_split_blocks(int64_t inter, int64_t k) {
    const int64_t nblk = inter / 32, cus = device_cu_count();
    const int64_t passes = (k / 256 + 3) / 4;
    if (passes < 2) return 0;
    if (nblk <= cus) return 2 * nblk <= cus ? (int)nblk : 0;
    return (int)(nblk % cus);
}

hipError_t launch_gemv_q4k_swiglu(const void* w, const void* xq, const NormIn* nin, float* gu_out, void* g_q8,
                                  int64_t inter, int64_t k, hipStream_t stream, int fmt, double* part, unsigned* cnt,
                                  int n_split) {
    return fmt == kFmtQ4_0 ? launch_swiglu<kFmtQ4_0>(w, xq, nin, gu_out, g_q8, inter, k, stream, part, cnt, n_split)
                           : launch_swiglu<kFmtQ4K>(w, xq, nin, gu_out, g_q8, inter, k, stream, part, cnt, n_split);
}

hipError_t launch_gemv_q4k_grouped(const void* w_all, int64_t expert_bytes, int n_experts,
                                   const int32_t* ids, int n_sel, const void* xq, int64_t xq_stride,
                                   float* y, const float* combine, float* y_out,
                                   const int64_t* out_row, int64_t out_rows, int64_t m, int64_t k,
                                   int64_t* inc_step, hipStream_t stream, const int32_t* ids_table,
                                   int32_t* ids_next) {
    const int nsb = (int)(k / 256);
    const Q4KPlan p = plan_q4k_mult(m, nsb, combine ? 1 : n_sel);
    const int lds = (xq_stride ? n_sel : 1) * stage_bytes(nsb * 8);
    const int64_t units = combine ? p.n_tiles : (int64_t)p.n_tiles * n_sel;
    if (combine && !y && xq_stride) {
        // contiguous slot columns are staged as one vector (see the kernel)
        const int lds_c = xq_stride == (int64_t)nsb * 8 * kQ8Bytes ? stage_bytes(n_sel * nsb * 8) : lds;
        // slots in parallel: about two workgroups per CU, tiles split evenly
        const int64_t want = 2 * (int64_t)device_cu_count();
        int tpw = (int)((p.n_tiles + want - 1) / want);
        if (tpw * p.rows_per_tile > 64) tpw = 64 / p.rows_per_tile;
        if (tpw < 1) tpw = 1;
        const int grid = (p.n_tiles + tpw - 1) / tpw;
        MQ_LAUNCH(k_gemv_q4k_grouped_combine, dim3(grid), dim3(64 * n_sel), lds_c, stream, (const uint8_t*)w_all,
                  expert_bytes, n_experts, ids, n_sel, (const uint8_t*)xq, xq_stride, combine, y_out, out_row,
                  out_rows, (int)m, nsb, p.log2s, p.passes, p.n_tiles, tpw, inc_step, ids_table, ids_next);
    } else if (combine) {
        const void* fn = (const void*)k_gemv_q4k_grouped<true>;
        MQ_LAUNCH((k_gemv_q4k_grouped<true>), dim3(balanced_grid(units, fn, lds)), dim3(256), lds, stream,
                           (const uint8_t*)w_all, expert_bytes, n_experts, ids, n_sel,
                           (const uint8_t*)xq, xq_stride, y, combine, y_out, out_row, out_rows, (int)m,
                           nsb, p.log2s, p.passes, p.n_tiles, inc_step);
    } else {
        const void* fn = (const void*)k_gemv_q4k_grouped<false>;
        MQ_LAUNCH((k_gemv_q4k_grouped<false>), dim3(balanced_grid(units, fn, lds)), dim3(256), lds, stream,
                           (const uint8_t*)w_all, expert_bytes, n_experts, ids, n_sel,
                           (const uint8_t*)xq, xq_stride, y, combine, y_out, out_row, out_rows, (int)m,
                           nsb, p.log2s, p.passes, p.n_tiles, inc_step);
    }
    return hipGetLastError();
}

hipError_t launch_moe_gate_up(const void* w_all, int64_t expert_bytes, int n_experts, int64_t inter, int64_t k,
                              const int64_t* step, int n_tokens, const int32_t* ids_table,
                              const float* logits_table, const float* x_table, int n_sel, int64_t k_pad,
                              int64_t* cur, int32_t* ids_out, float* combine_out, void* g_q8, float* gu_out,
                              hipStream_t stream, const int32_t* ids_next, double* part, unsigned* cnt,
                              int n_split) {
    const int nsb = (int)(k / 256);
    const int lds = stage_bytes(nsb * 8);
    const bool ok = part && cnt && n_split > 0 && n_split <= n_sel * (int)(inter / 32) && (nsb + 3) / 4 >= 2;
    const int ns = ok ? n_split : 0;
    MQ_LAUNCH(k_moe_gate_up, dim3((unsigned)((k_pad / 32) * n_sel + ns)), dim3(512), lds, stream,
              (const uint8_t*)w_all, expert_bytes, n_experts, (int)inter, nsb, step, n_tokens, ids_table,
              logits_table, x_table, n_sel, k_pad, cur, ids_out, combine_out, (uint8_t*)g_q8, gu_out, ids_next,
              ns, part, cnt);
    return hipGetLastError();
}

int moe_split_blocks(int n_sel, int64_t inter, int64_t k) {
    const int64_t working = (int64_t)n_sel * (inter / 32), cus = device_cu_count();
    const int64_t passes = (k / 256 + 3) / 4;
    if (passes < 2 || working <= cus) return 0;
    return (int)(working % cus);
}

__global__ void k_moe_prime(const int64_t* __restrict__ step, int n_tokens, const int32_t* __restrict__ ids_table,
                            int n_sel, int32_t* __restrict__ ids_next) {
    const int i = threadIdx.x;
    if (i < n_sel) ids_next[i] = ids_table[(int64_t)((uint64_t)*step % (uint64_t)n_tokens) * n_sel + i];
}

hipError_t launch_moe_prime(const int64_t* step, int n_tokens, const int32_t* ids_table, int n_sel,
                            int32_t* ids_next, hipStream_t stream) {
    hipLaunchKernelGGL(k_moe_prime, dim3(1), dim3(64), 0, stream, step, n_tokens, ids_table, n_sel, ids_next);
    return hipGetLastError();
}

}  // namespace mq
