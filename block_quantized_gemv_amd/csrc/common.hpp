// Device-side building blocks shared by the libmq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

constexpr int kWave = 64;
constexpr int kQ4KBytes = 144;     // q4_K super-block: 256 weights
constexpr int kQ8Bytes = 34;       // q8_0 block: 32 values

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef u32x4 u32x4_a4 __attribute__((aligned(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- f16 ----
// Hardware conversions: v_cvt_f32_f16 is exact; v_cvt_f16_f32 rounds to
// nearest even under the default MODE register, subnormals included.
__device__ __forceinline__ float f16_to_f32(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// The wave's index in its workgroup as a wave-uniform (scalar) value: the
// compiler cannot tell that threadIdx.x / 64 is the same on every lane, and
// index arithmetic derived from it would otherwise run on the vector ALUs.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Kernel span stamps, compiled only into the instantiations that take them
// (ON).  Each wave reads the real-time counter (100 MHz) when it starts and
// again at its end, and lane 0 stores the pair [start, end] to its own slot
// p[2*slot], p[2*slot+1], slot = workgroup * kStampWaves + wave: one plain
// 16-byte store that nothing waits for, so the kernel's tail is the one it
// has without stamps.  A launch overwrites the slots of the launch before
// it (the grid is the same every step).  The host takes the minimum start
// and the maximum end over the slots: the time from the kernel's first wave
// start to its last wave end (the end is the wave's last instruction; its
// stores drain after it).  Workgroups from kStampSlots on are not stamped.
// The production instantiations carry none of this.
constexpr int kStampSlots = 1024, kStampWaves = 16;
template <bool ON>
struct SpanStamp {
    __device__ explicit SpanStamp(uint64_t*) {}
};
template <>
struct SpanStamp<true> {
    unsigned long long t0;
    unsigned long long* p;
    __device__ explicit SpanStamp(uint64_t* q)
        : t0((unsigned long long)__builtin_amdgcn_s_memrealtime()), p((unsigned long long*)q) {}
    __device__ ~SpanStamp() {
        if (!p || (threadIdx.x & 63) != 0) return;
        const unsigned long long t1 = (unsigned long long)__builtin_amdgcn_s_memrealtime();
        if (blockIdx.x >= (unsigned)kStampSlots) return;
        const unsigned slot = blockIdx.x * kStampWaves + (threadIdx.x >> 6);
        *(ulonglong2*)(p + 2 * slot) = make_ulonglong2(t0, t1);
    }
};

__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);   // v_dot4_i32_i8
}
// The first dot of a chain: the clamped form takes its zero accumulator as
// an inline constant (the unclamped one becomes a move plus the accumulating
// v_dot4c).  A q4 x q8 sum of 4 products stays far inside int32, so the
// clamp never acts.
__device__ __forceinline__ int dot4_first(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, 0, true);
}

// ------------------------------------------------------ wave reductions ----
// All-reduce steps over aligned lane groups.  Every step adds a lane's value
// to its partner's (IEEE addition is commutative), so all lanes of a group
// end with the same bits and the order of additions is fixed: the sum is
// deterministic and tree-shaped, which is also the more accurate schedule
// ('Part 4 · Lecture 08 — Graph-Resident Decode', §8).  The DPP patterns
// used here read lanes of the same row, all active, so the moves need no
// fallback value (bound_ctrl set, no zeroing move before each).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, true);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double swizzle_xor16_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    // ds_swizzle bit mode: and_mask 0x1F, or_mask 0, xor_mask 0x10
    const int lo = __builtin_amdgcn_ds_swizzle((int)(uint32_t)b, 0x401F);
    const int hi = __builtin_amdgcn_ds_swizzle((int)(uint32_t)(b >> 32), 0x401F);
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over aligned groups of 2^log2s lanes (log2s in 2..6).  Afterwards every
// lane of a group holds the group's sum (for log2s == 6: the wave's sum).
// Must be called with all 64 lanes active.
__device__ __forceinline__ double group_sum_f64(double v, int log2s) {
    v += dpp_f64<0xB1>(v);                        // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp_f64<0x4E>(v);                        // quad_perm [2,3,0,1]: lane ^ 2
    if (log2s >= 3) v += dpp_f64<0x141>(v);       // row_half_mirror: quads of each 8
    if (log2s >= 4) v += dpp_f64<0x140>(v);       // row_mirror: halves of each 16
    if (log2s >= 5) v += swizzle_xor16_f64(v);    // rows of each 32
    if (log2s >= 6) v = readlane_f64(v, 0) + readlane_f64(v, 32);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) { return group_sum_f64(v, 6); }

// ------------------------------------------------ q8_0 activation staging ----
// A q8_0 vector is restaged once per workgroup into LDS in an aligned,
// lane-friendly layout.  Blocks are taken in pairs (P = block/2, 64 values);
// pairs are grouped 64 at a time, one pair per lane of a wave:
//
//   group G = P / 64 occupies kStageGroupBytes at G * kStageGroupBytes:
//     [0, 4096)      codes: 16-byte chunk k (0..3) of pair L = P % 64 at (k*64 + L)*16
//                    (chunks 0,1 = block 2P, chunks 2,3 = block 2P+1)
//     [4096, 5120)   (double)d of blocks 2P, 2P+1 at 4096 + L*16
//     [5120, 6144)   (double)d * sum(codes) of blocks 2P, 2P+1 at 5120 + L*16
//
// A wave whose lane L reads pair 64*G + L reads 1 KB contiguously per chunk,
// so the 16-byte LDS reads are free of bank conflicts; lanes that read the
// same pair get a broadcast.
constexpr int kStageGroupBytes = 6144;

__host__ __device__ constexpr int stage_groups(int nblocks) { return (nblocks / 2 + 63) / 64; }
__host__ __device__ constexpr int stage_bytes(int nblocks) { return stage_groups(nblocks) * kStageGroupBytes; }

// Reads block b of a q8_0 vector.  The 34-byte block starts 2-byte aligned;
// the nine aligned dwords read here are the ones that contain the block's
// bytes, so every dword holds at least one byte of the block and lies in its
// page.  Returns the f16 scale bits and the 32 codes as 8 dwords.
__device__ __forceinline__ uint32_t load_q8_block(const uint8_t* blk, uint32_t (&q)[8]) {
    const uint32_t shift = (uint32_t)((uintptr_t)blk & 3u);      // 0 or 2
    const uint32_t* p = (const uint32_t*)(blk - shift);
    uint32_t w[9];
#pragma unroll
    for (int i = 0; i < 9; ++i) w[i] = p[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = shift ? w[i + 1] : __builtin_amdgcn_alignbyte(w[i + 1], w[i], 2);
    return shift ? (w[0] >> 16) : (w[0] & 0xFFFFu);
}

// Writes block b (relative index) of a staged vector: codes, (double)d and
// d * (sum of codes).  Returns the code sum.
__device__ __forceinline__ int stage_q8_block(int b, uint32_t dbits, const uint32_t (&q)[8],
                                              uint8_t* __restrict__ lds) {
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s = dot4(q[i], 0x01010101u, s);
    const double d = (double)f16_to_f32(dbits);
    const int P = b >> 1, half = b & 1, G = P >> 6, L = P & 63;
    uint8_t* g = lds + G * kStageGroupBytes;
    *(u32x4*)(g + ((2 * half + 0) * 64 + L) * 16) = u32x4{q[0], q[1], q[2], q[3]};
    *(u32x4*)(g + ((2 * half + 1) * 64 + L) * 16) = u32x4{q[4], q[5], q[6], q[7]};
    *(double*)(g + 4096 + L * 16 + half * 8) = d;
    *(double*)(g + 5120 + L * 16 + half * 8) = d * (double)s;
    return s;
}

// Stage blocks [b0, b0 + nb) of the vector at xq into the layout above at
// lds (relative block index starts at 0).  Optionally records the int32
// code sums (for the debug dump).
__device__ __forceinline__ void stage_q8(const uint8_t* __restrict__ xq, int b0, int nb,
                                         uint8_t* __restrict__ lds, int tid, int nthreads,
                                         int32_t* __restrict__ ysum_out) {
    for (int b = tid; b < nb; b += nthreads) {
        uint32_t q[8];
        const uint32_t dbits = load_q8_block(xq + (int64_t)(b0 + b) * kQ8Bytes, q);
        const int s = stage_q8_block(b, dbits, q, lds);
        if (ysum_out) ysum_out[b0 + b] = s;
    }
}

// Stage blocks [b0, b0 + nb) of ncols columns (column c at xq + c*col_stride)
// into lds + c*col_bytes, relative block index from 0.  The workgroup's
// blocks are taken as one flat list; each thread first requests up to R of
// them into registers and only then writes them, so the columns' loads are
// in flight together instead of one column after another.  ysum_out, if
// set, receives column 0's code sums at b0 + b.
template <int R>
__device__ __forceinline__ void stage_q8_cols(const uint8_t* __restrict__ xq, int64_t col_stride, int b0, int nb,
                                              int ncols, uint8_t* __restrict__ lds, int col_bytes,
                                              int32_t* __restrict__ ysum_out) {
    const int total = nb * ncols, T = blockDim.x, tid = threadIdx.x;
    uint32_t q[R][8], d[R];
    int cc[R], bb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int f = tid + r * T;
        const bool in = f < total;
        const int c = in ? f / nb : 0;
        cc[r] = c;
        bb[r] = in ? f - c * nb : 0;
        d[r] = load_q8_block(xq + c * col_stride + (int64_t)(b0 + bb[r]) * kQ8Bytes, q[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (tid + r * T < total) {
            const int s = stage_q8_block(bb[r], d[r], q[r], lds + cc[r] * col_bytes);
            if (ysum_out && cc[r] == 0) ysum_out[b0 + bb[r]] = s;
        }
    }
    for (int f = tid + R * T; f < total; f += T) {
        const int c = f / nb, b = f - c * nb;
        uint32_t qq[8];
        const uint32_t dd = load_q8_block(xq + c * col_stride + (int64_t)(b0 + b) * kQ8Bytes, qq);
        const int s = stage_q8_block(b, dd, qq, lds + c * col_bytes);
        if (ysum_out && c == 0) ysum_out[b0 + b] = s;
    }
}

// Staging in two steps, so that a kernel can request its activation before
// its first weights: stage_q8_load reads the thread's first kStageRegBlocks
// blocks (b = tid + r*blockDim.x) into registers, stage_q8_store writes
// them, and any further blocks, into lds.
constexpr int kStageRegBlocks = 2;
struct Q8Regs {
    uint32_t q[kStageRegBlocks][8];
    uint32_t d[kStageRegBlocks];
};
__device__ __forceinline__ void stage_q8_load(const uint8_t* __restrict__ xq, int nb, Q8Regs& r) {
#pragma unroll
    for (int k = 0; k < kStageRegBlocks; ++k) {
        const int b = (int)threadIdx.x + k * (int)blockDim.x;
        r.d[k] = load_q8_block(xq + (int64_t)(b < nb ? b : 0) * kQ8Bytes, r.q[k]);
    }
}
__device__ __forceinline__ void stage_q8_store(const uint8_t* __restrict__ xq, int nb, const Q8Regs& r,
                                               uint8_t* __restrict__ lds) {
#pragma unroll
    for (int k = 0; k < kStageRegBlocks; ++k) {
        const int b = (int)threadIdx.x + k * (int)blockDim.x;
        if (b < nb) stage_q8_block(b, r.d[k], r.q[k], lds);
    }
    for (int b = (int)threadIdx.x + kStageRegBlocks * (int)blockDim.x; b < nb; b += (int)blockDim.x) {
        uint32_t q[8];
        const uint32_t dbits = load_q8_block(xq + (int64_t)b * kQ8Bytes, q);
        stage_q8_block(b, dbits, q, lds);
    }
}
// The same two steps for ncols columns (column c at xq + c*col_stride,
// staged at lds + c*col_bytes), their blocks taken as one flat list
// f = c*nb + b, so that the columns' first blocks are requested together.
__device__ __forceinline__ void stage_q8_load_cols(const uint8_t* __restrict__ xq, int64_t col_stride, int nb,
                                                   int ncols, Q8Regs& r) {
    const int total = nb * ncols;
#pragma unroll
    for (int k = 0; k < kStageRegBlocks; ++k) {
        const int f = (int)threadIdx.x + k * (int)blockDim.x;
        const int c = f < total ? f / nb : 0, b = f < total ? f - c * nb : 0;
        r.d[k] = load_q8_block(xq + c * col_stride + (int64_t)b * kQ8Bytes, r.q[k]);
    }
}
__device__ __forceinline__ void stage_q8_store_cols(const uint8_t* __restrict__ xq, int64_t col_stride, int nb,
                                                    int ncols, const Q8Regs& r, uint8_t* __restrict__ lds,
                                                    int col_bytes) {
    const int total = nb * ncols;
#pragma unroll
    for (int k = 0; k < kStageRegBlocks; ++k) {
        const int f = (int)threadIdx.x + k * (int)blockDim.x;
        if (f < total) {
            const int c = f / nb;
            stage_q8_block(f - c * nb, r.d[k], r.q[k], lds + c * col_bytes);
        }
    }
    for (int f = (int)threadIdx.x + kStageRegBlocks * (int)blockDim.x; f < total; f += (int)blockDim.x) {
        const int c = f / nb, b = f - c * nb;
        uint32_t q[8];
        const uint32_t dbits = load_q8_block(xq + c * col_stride + (int64_t)b * kQ8Bytes, q);
        stage_q8_block(b, dbits, q, lds + c * col_bytes);
    }
}

// The staged data of pair P: codes of blocks 2P (c[0..7]) and 2P+1 (c[8..15]),
// their scales and scale*code-sums.
struct StagedPair {
    uint32_t c[16];
    double d0, d1, ds0, ds1;
};
__device__ __forceinline__ void read_pair(const uint8_t* __restrict__ lds, int P, StagedPair& sp,
                                          bool need_sums) {
    const uint8_t* g = lds + (P >> 6) * kStageGroupBytes;
    const int L = P & 63;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const u32x4 v = *(const u32x4*)(g + (k * 64 + L) * 16);
        sp.c[4 * k + 0] = v.x; sp.c[4 * k + 1] = v.y; sp.c[4 * k + 2] = v.z; sp.c[4 * k + 3] = v.w;
    }
    sp.d0 = *(const double*)(g + 4096 + L * 16);
    sp.d1 = *(const double*)(g + 4096 + L * 16 + 8);
    if (need_sums) {
        sp.ds0 = *(const double*)(g + 5120 + L * 16);
        sp.ds1 = *(const double*)(g + 5120 + L * 16 + 8);
    } else {
        sp.ds0 = sp.ds1 = 0.0;
    }
}

// ------------------------------------------------------- item streaming ----
// A wave streams its work items 0..n-1 through two register buffers A and B
// (a ping-pong): `fetch(i, buf)` issues item i's loads into buf (for i >= n
// it must load in-bounds lines and mark the item invalid), `use(buf)`
// computes the item held in buf.  The loads of one item are in flight while
// the other computes, and the compiler only has to wait for the buffer it
// is about to use.
//
// EARLY: the caller fetched items 0 and 1 before its prologue (whose own
// loads were issued first), and the last round is peeled so that nothing
// is fetched past the end.  Otherwise the caller fetched item 0 before its
// prologue (whose loads then complete right behind it) and item i+1 is
// fetched at the top of each round.  Memory returns in order per wave, so a
// prologue that loads after the early fetches waits for them as well.
template <bool EARLY, class Buf, class Fetch, class Use>
__device__ __forceinline__ void stream_items(int n, Buf& A, Buf& B, Fetch&& fetch, Use&& use) {
    if constexpr (EARLY) {
        int i = 0;
        for (; i + 3 < n; i += 2) {
            use(A);
            fetch(i + 2, A);
            use(B);
            fetch(i + 3, B);
        }
        if (i < n) {
            use(A);
            const bool more = i + 2 < n;
            if (more) fetch(i + 2, A);
            if (i + 1 < n) use(B);
            if (more) use(A);
        }
    } else {
        for (int i = 0; i < n; i += 2) {
            fetch(i + 1, B);
            use(A);
            fetch(i + 2, A);
            if (i + 1 < n) use(B);
        }
    }
}

}  // namespace mq
