// Device-side glue shared by the standalone glue kernels and the fused
// tails/epilogues of the GEMV kernels: q8_0 quantization of one value per
// lane, and RMSNorm over a vector by one workgroup.
//
// Quantization decides integers from floats, so it runs in f32 with only
// exactly specified operations: a max over magnitudes (order-independent,
// 'Part 4 · Lecture 08 — Graph-Resident Decode', §8), an IEEE f32 divide,
// f16 round-to-nearest-even of the scale and roundf.  The SwiGLU stand-in
// is computed in f64 and rounded to f32 once; RMSNorm forms its scale in
// f64, rounds it to f32 once and multiplies each value by it in f32.
#pragma once

#include <math.h>

#include "common.hpp"

namespace mq {

// (as dpp_f64: same-row patterns with every lane active)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Max over each aligned group of 32 lanes (all 64 lanes must be active).
__device__ __forceinline__ float half_wave_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));      // lane ^ 1
    v = fmaxf(v, dpp_f32<0x4E>(v));      // lane ^ 2
    v = fmaxf(v, dpp_f32<0x141>(v));     // quads of each 8
    v = fmaxf(v, dpp_f32<0x140>(v));     // halves of each 16
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F)));
    return v;
}

// The lane's value v belongs to the q8_0 block starting at `out` (34 bytes);
// i = the lane's index inside the block.  The lanes of one block are the 32
// consecutive lanes of a half-wave, and all 64 lanes call this together.
__device__ __forceinline__ void quantize_lane(float v, uint8_t* __restrict__ out, int i, bool write) {
#pragma clang fp contract(off)
    const float amax = half_wave_max(fabsf(v));
    const float d32 = amax / 127.0f;
    const uint32_t dbits = f32_to_f16(d32);
    const float d = f16_to_f32(dbits);
    int q = 0;
    if (d != 0.0f) {
        const float r = roundf(v / d);
        q = r > 127.0f ? 127 : (r < -127.0f ? -127 : (int)r);
    }
    if (write) {
        if (i == 0) *(uint16_t*)out = (uint16_t)dbits;
        out[2 + i] = (uint8_t)(int8_t)q;
    }
}

// Sum over the workgroup (at most 16 waves) in a fixed order: a DPP/swizzle
// tree inside each wave, then a 16-lane tree over the wave sums (zeros past
// the last wave), which every lane forms from LDS after one barrier.  Every
// workgroup of the same size that sums the same per-thread values gets the
// same bits.  sh (16 doubles) must not be written again by the caller.
__device__ __forceinline__ double block_sum_f64(double v, double* sh) {
    v = wave_sum_f64(v);
    const int nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    const int l = threadIdx.x & 15;
    return group_sum_f64(l < nw ? sh[l] : 0.0, 4);
}

// The RMSNorm scale 1/sqrt(mean(x^2) + eps) of k values, formed in f64 and
// rounded to f32 once; the squares are summed in f64 by the workgroup in the
// order above (thread t takes elements t, t+B, t+2B, ...).
__device__ __forceinline__ float rms_scale(const float* __restrict__ x, int k, float eps, double* sh) {
#pragma clang fp contract(off)
    double ss = 0.0;
#pragma unroll 16
    for (int i = threadIdx.x; i < k; i += blockDim.x) {
        const double v = x[i];
        ss += v * v;
    }
    ss = block_sum_f64(ss, sh);
    return (float)(1.0 / sqrt(ss / (double)k + (double)eps));
}

// Outputs [first, first + count) of Q8(RMSNorm(x)) by one workgroup, one
// value per lane per round (blockDim.x must be a multiple of 64); each
// normalized value is the f32 product x * scale.
__device__ __forceinline__ void rmsnorm_quantize_range(const float* __restrict__ x, float scale, int k,
                                                       uint8_t* __restrict__ xq, int first, int count) {
#pragma clang fp contract(off)
    for (int base = first; base < first + count; base += blockDim.x) {
        const int idx = base + threadIdx.x;
        const bool in = idx < first + count && idx < k;
        const float v = in ? x[idx] * scale : 0.0f;
        quantize_lane(v, xq + (int64_t)(idx >> 5) * kQ8Bytes, idx & 31, in);
    }
}

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// The f32 input of a GEMV whose q8_0 activation is Q8(RMSNorm(x)), formed in
// the GEMV's own prologue.  With sel_step, x is a table and row
// (*sel_step mod n_inputs) is used; q8_copy, if set, receives the q8_0
// vector from workgroup 0; inc_step, if set, is advanced by one by thread 0
// of workgroup 0 after it has staged its input (the kernel must not also
// read it through sel_step); exact forces the division path of
// stage_rmsnorm_q8 everywhere (same results; a test hook).
struct NormIn {
    const float* x;
    const int64_t* sel_step;
    int n_inputs;
    float eps;
    uint8_t* q8_copy;
    int64_t* inc_step;
    int exact;          // take the division path for every value (test hook)
    uint64_t* stamp;    // kernel span stamps (SpanStamp), or null
};

// ------------------------------------------- RMSNorm -> q8_0 in a prologue ----
//
// Each normalized value n = x * scale is one f32 multiply.  Its q8_0 code
// needs the correctly rounded f32 quotient n/d, and the block scale amax/127
// another; as division sequences they cost more than the GEMV's own
// arithmetic, so both are formed as products with a reciprocal and a
// product is accepted only when it provably gives the same result:
//
// * The scale RN_f32(amax/127) from t = amax * RN_f64(1/127), which is
//   within 4 f64 ulps of the f64 quotient (f64 carries more than 2*24+2
//   bits, so rounding the quotient to f64 before f32 changes nothing).
//   Read as integers, f64 patterns of one sign are ordered like their
//   values, and rounding to f32 maps every pattern strictly between two
//   consecutive f32 midpoints (patterns whose low 29 bits are 2^28) to the
//   same f32.  So RN_f32(t) is the quotient's when t's low 29 bits are more
//   than 16 away from 2^28 and t is at least 2^-125 (the f32 normal range,
//   where those patterns are the midpoints).
// * A code roundf(RN_f32(n/d)) comes from the f32 product y = n * (1/d)
//   (see code_checked): unless y lies within |y|*2^-21 of a half-integer,
//   the code is y rounded to the nearest integer.
//
// When any lane of a wave meets a doubtful case the wave redoes the whole
// chunk with the divisions themselves.

// RN_f32(t), flagging t near an f32 midpoint.  The caller rules out the
// f32 subnormal range separately.
__device__ __forceinline__ float f32_checked(double t, bool& bad) {
    const uint32_t lo = (uint32_t)__builtin_bit_cast(uint64_t, t);
    bad |= ((lo & 0x1FFFFFFFu) - (0x10000000u - 16u)) <= 32u;
    return (float)t;
}

// clamp(roundf(RN_f32(n/d)), -127, 127) from y = n * r in f32, r within an
// f32 ulp of 1/d: y is within 1.6*2^-23 of n/d relative, and RN_f32 moves
// the quotient by at most 2^-24 relative, so both lie strictly on the same
// side of every half-integer unless y lies within |y|*2^-21 of one
// (flagged; exact half-integers are flagged too).  Off those, rounding to
// nearest-even and half away from zero agree.  The test needs |y - rint(y)|
// > 0.5 - |y|*2^-21; the subtraction is exact and the threshold's rounding
// (at most 2^-26) is covered for |y| >= 1/4, below which no half-integer
// is near.  y must be finite.
__device__ __forceinline__ int code_checked(float y, bool& bad) {
    const float r = rintf(y);
    bad |= fabsf(y - r) > fmaf(fabsf(y), -0x1p-21f, 0.5f);
    return (int)__builtin_amdgcn_fmed3f(r, -127.0f, 127.0f);
}

// 1/d in f32 to within an ulp: hardware estimate and a Newton step.
__device__ __forceinline__ float recip_f32(float d) {
    const float r = __builtin_amdgcn_rcpf(d);
    return fmaf(r, fmaf(-d, r, 1.0f), r);
}

// One 4-value chunk of a q8_0 block: the block is 8 aligned lanes of the
// wave (chunks 8b..8b+7), all 64 lanes active.  Gives the 4 codes (packed),
// the f16 scale bits and the block's code sum (all 8 lanes get it).
struct ChunkQ8 {
    uint32_t packed, dbits;
    int ysum;
};

__device__ __forceinline__ int code_of(float n, float d) {
    const float rq = roundf(n / d);
    return rq > 127.0f ? 127 : (rq < -127.0f ? -127 : (int)rq);
}

__device__ __forceinline__ int block8_sum(int s) {
    s += dpp_i32<0xB1>(s);
    s += dpp_i32<0x4E>(s);
    s += dpp_i32<0x141>(s);
    return s;
}

__device__ __forceinline__ float block8_max(float a) {
    a = fmaxf(a, dpp_f32<0xB1>(a));      // lane ^ 1
    a = fmaxf(a, dpp_f32<0x4E>(a));      // lane ^ 2
    a = fmaxf(a, dpp_f32<0x141>(a));     // the other quad of the 8
    return a;
}

__device__ __forceinline__ uint32_t pack4(const int (&q)[4]) {
    return ((uint32_t)q[0] & 0xFFu) | (((uint32_t)q[1] & 0xFFu) << 8) | (((uint32_t)q[2] & 0xFFu) << 16) |
           ((uint32_t)q[3] << 24);
}

// The reference arithmetic: divisions as written.
__device__ __forceinline__ ChunkQ8 chunk_exact(const float4& v, float scale) {
#pragma clang fp contract(off)
    const float n[4] = {v.x * scale, v.y * scale, v.z * scale, v.w * scale};
    const float amax = block8_max(fmaxf(fmaxf(fabsf(n[0]), fabsf(n[1])), fmaxf(fabsf(n[2]), fabsf(n[3]))));
    const float d32 = amax / 127.0f;
    ChunkQ8 o;
    o.dbits = f32_to_f16(d32);
    const float d = f16_to_f32(o.dbits);
    int q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = d != 0.0f ? code_of(n[i], d) : 0;
    o.packed = pack4(q);
    o.ysum = block8_sum(q[0] + q[1] + q[2] + q[3]);
    return o;
}

// The same values through reciprocal products; `bad` is set where they
// might differ (then chunk_exact is used).
__device__ __forceinline__ ChunkQ8 chunk_fast(const float4& v, float scale, bool& bad) {
#pragma clang fp contract(off)
    const float n[4] = {v.x * scale, v.y * scale, v.z * scale, v.w * scale};
    const float amax = block8_max(fmaxf(fmaxf(fabsf(n[0]), fabsf(n[1])), fmaxf(fabsf(n[2]), fabsf(n[3]))));
    const double d64 = (double)amax * (1.0 / 127.0);
    bad |= d64 != 0.0 && d64 < 0x1p-125;
    float d32 = f32_checked(d64, bad);
    // The scale is rounded to f32 and then to f16, as the reference does;
    // the empty asm keeps the compiler from fusing the two conversions into
    // one f64 -> f16 rounding, which differs in double-rounding cases.
    asm volatile("" : "+v"(d32));
    ChunkQ8 o;
    o.dbits = f32_to_f16(d32);
    const float d = f16_to_f32(o.dbits);
    // d == 0 only when the block is all zeros: r = 0 gives codes 0.
    const float rd = d == 0.0f ? 0.0f : recip_f32(d);
    int q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = code_checked(n[i] * rd, bad);
    o.packed = pack4(q);
    o.ysum = block8_sum(dot4(o.packed, 0x01010101u, 0));
    return o;
}

// Chunks of the f32 input held in registers through the prologue.
constexpr int kNormRegChunks = 2;

// Q8(RMSNorm(x)) of k values (k % 32 == 0, x 16-byte aligned), computed by
// the whole workgroup (blockDim.x % 64 == 0) and written to lds in the
// layout of stage_q8.  Thread t owns the 4-value chunks t, t+T, ... (T =
// blockDim.x); xr holds its first kNormRegChunks of them (loaded by
// norm_load).  It sums their squares in order, the workgroup adds the
// per-thread sums in the fixed order of block_sum_f64, and each value is
// x/sqrt(mean + eps) in f64 rounded to f32; a q8_0 block is 8 consecutive
// chunks, i.e. 8 aligned lanes, and its amax, f16 scale and codes follow
// quantize_lane (stage_scaled_q8).  With `exact` every chunk takes the
// division path (a test hook: the results are the same).  The caller
// synchronizes the workgroup before reading lds.
__device__ __forceinline__ void norm_load(const float* __restrict__ x, int k, float4 (&xr)[kNormRegChunks]) {
    const float4* x4 = (const float4*)x;
#pragma unroll
    for (int r = 0; r < kNormRegChunks; ++r) {
        const int c = r * (int)blockDim.x + (int)threadIdx.x;
        xr[r] = c < (k >> 2) ? x4[c] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
}

// RN_f32(1/sqrt(ss/k + eps)) with the f64 operations of the definition
// (each correctly rounded) replaced by a reciprocal and a reciprocal square
// root refined by Newton steps.  Each step squares the relative error, so
// three steps from any hardware estimate better than 2^-8 reach the f64
// rounding level; the result t is then within a few f64 ulps of the exactly
// computed chain's value, and RN_f32(t) is that chain's f32 unless t lies
// within 16 f64 ulps of an f32 midpoint (f32_checked), where the chain
// itself is evaluated.  The reciprocal of k does not depend on ss and
// overlaps the sum's reduction.  exact forces the chain (a test hook).
__device__ __forceinline__ float rms_scale_of(double ss, int k, float eps, bool exact) {
#pragma clang fp contract(off)
    const double kd = (double)k;
    double rk = __builtin_amdgcn_rcp(kd);
#pragma unroll
    for (int i = 0; i < 3; ++i) rk = fma(rk, fma(-kd, rk, 1.0), rk);
    const double v = ss * rk + (double)eps;
    double y = __builtin_amdgcn_rsq(v);
#pragma unroll
    for (int i = 0; i < 3; ++i) y = fma(0.5 * y, fma(-v * y, y, 1.0), y);
    bool bad = exact;
    const float f = f32_checked(y, bad);
    if (!bad) return f;
    return (float)(1.0 / sqrt(ss / kd + (double)eps));
}

// Q8(x * scale) of k values (k % 32 == 0) into lds in the layout of
// stage_q8: each value is the f32 product x * scale (x itself when scale
// is 1), then quantized as described above; q8_copy, if set, also
// receives the q8_0 vector.  xr: the thread's first chunks (norm_load).
__device__ __forceinline__ void stage_scaled_q8(const float* __restrict__ x, int k,
                                                const float4 (&xr)[kNormRegChunks], float scale, bool exact,
                                                uint8_t* __restrict__ lds, uint8_t* __restrict__ q8_copy) {
#pragma clang fp contract(off)
    const int nch = k >> 2;
    const int T = blockDim.x;
    const float4* x4 = (const float4*)x;
    const int rounds = (nch + T - 1) / T;
    for (int r = 0; r < rounds; ++r) {
        const int c = r * T + (int)threadIdx.x;
        const bool in = c < nch;      // whole 8-lane groups are in or out
        const float4 v = r < kNormRegChunks ? xr[r] : (in ? x4[c] : make_float4(0.0f, 0.0f, 0.0f, 0.0f));
        bool bad = exact;
        ChunkQ8 o = chunk_fast(v, scale, bad);
        if (__builtin_amdgcn_ballot_w64(bad) != 0) o = chunk_exact(v, scale);   // wave-uniform
        if (in) {
            const int b = c >> 3, cb = c & 7;
            const int P = b >> 1, half = b & 1, L = P & 63;
            uint8_t* g = lds + (P >> 6) * kStageGroupBytes;
            *(uint32_t*)(g + ((2 * half + (cb >> 2)) * 64 + L) * 16 + (cb & 3) * 4) = o.packed;
            if (cb == 0) {
                const double d = (double)f16_to_f32(o.dbits);
                *(double*)(g + 4096 + L * 16 + half * 8) = d;
                *(double*)(g + 5120 + L * 16 + half * 8) = d * (double)o.ysum;
            }
            if (q8_copy) {
                uint8_t* blk = q8_copy + (int64_t)b * kQ8Bytes;
                if (cb == 0) *(uint16_t*)blk = (uint16_t)o.dbits;
                *(uint16_t*)(blk + 2 + 4 * cb) = (uint16_t)(o.packed & 0xFFFFu);
                *(uint16_t*)(blk + 4 + 4 * cb) = (uint16_t)(o.packed >> 16);
            }
        }
    }
}

__device__ __forceinline__ void stage_rmsnorm_q8(const float* __restrict__ x, int k, float eps,
                                                 const float4 (&xr)[kNormRegChunks], bool exact,
                                                 uint8_t* __restrict__ lds, double* sh,
                                                 uint8_t* __restrict__ q8_copy) {
#pragma clang fp contract(off)
    const int nch = k >> 2;
    const int T = blockDim.x;
    const float4* x4 = (const float4*)x;
    const int rounds = (nch + T - 1) / T;
    double ss = 0.0;
    for (int r = 0; r < rounds; ++r) {
        const int c = r * T + (int)threadIdx.x;
        const float4 v = r < kNormRegChunks ? xr[r] : (c < nch ? x4[c] : make_float4(0.0f, 0.0f, 0.0f, 0.0f));
        ss += (double)v.x * (double)v.x;
        ss += (double)v.y * (double)v.y;
        ss += (double)v.z * (double)v.z;
        ss += (double)v.w * (double)v.w;
    }
    ss = block_sum_f64(ss, sh);
    stage_scaled_q8(x, k, xr, rms_scale_of(ss, k, eps, exact), exact, lds, q8_copy);
}

// The input row of a GEMV fed by a NormIn.
// The step counter is read through the constant address space: no kernel
// that selects a row with it also writes it, so the load may always go
// through the scalar unit (the compiler cannot prove that on its own once
// a side-effecting instruction, such as a clock read, precedes it).
__device__ __forceinline__ const float* norm_row(const NormIn& in, int k) {
    typedef const __attribute__((address_space(4))) int64_t const_i64;
    const float* x = in.x;
    if (in.sel_step) x += (int64_t)((uint64_t)*(const_i64*)(uintptr_t)in.sel_step % (uint64_t)in.n_inputs) * k;
    return x;
}

// Prologue of a GEMV fed by a NormIn (x = norm_row, xr from norm_load):
// stages Q8(RMSNorm(x)) into lds and advances the step counter if asked.
__device__ __forceinline__ void stage_norm_input(const NormIn& in, const float* x, int k,
                                                 const float4 (&xr)[kNormRegChunks], uint8_t* __restrict__ lds,
                                                 double* sh) {
    stage_rmsnorm_q8(x, k, in.eps, xr, in.exact != 0, lds, sh, blockIdx.x == 0 ? in.q8_copy : nullptr);
    if (in.inc_step && blockIdx.x == 0 && threadIdx.x == 0) *in.inc_step += 1;
}

// The glue stand-in between gate/up and down: silu(g)*u in f64, rounded to f32.
__device__ __forceinline__ float swiglu_value(float gate, float up) {
#pragma clang fp contract(off)
    const double g = gate;
    return (float)(g / (1.0 + exp(-g)) * (double)up);
}

}  // namespace mq
