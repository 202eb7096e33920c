// Device-side glue shared by the standalone glue kernels and the fused
// tails/epilogues of the GEMV kernels: q8_0 quantization of one value per
// lane, and RMSNorm over a vector by one workgroup.
//
// Quantization decides integers from floats, so it runs in f32 with only
// exactly specified operations: a max over magnitudes (order-independent,
// 'Part 4 · Lecture 08 — Graph-Resident Decode', §8), an IEEE f32 divide,
// f16 round-to-nearest-even of the scale and roundf.  The glue itself is
// computed in f64 and rounded to f32 once, then quantized.
#pragma once

#include <math.h>

#include "common.hpp"

namespace mq {

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
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

// Sum over the workgroup in a fixed order: DPP/swizzle inside each wave, then
// the wave sums in wave order.  Every workgroup of the same size that sums
// the same per-thread values gets the same bits.
__device__ __forceinline__ double block_sum_f64(double v, double* sh) {
    v = wave_sum_f64(v);
    const int nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    double t = 0.0;
    for (int i = 0; i < nw; ++i) t += sh[i];
    __syncthreads();
    return t;
}

// sqrt(mean(x^2) + eps) of k values in f64, summed by the workgroup in the
// order above (thread t takes elements t, t+B, t+2B, ...).
__device__ __forceinline__ double rms_denom(const float* __restrict__ x, int k, float eps, double* sh) {
#pragma clang fp contract(off)
    double ss = 0.0;
#pragma unroll 16
    for (int i = threadIdx.x; i < k; i += blockDim.x) {
        const double v = x[i];
        ss += v * v;
    }
    ss = block_sum_f64(ss, sh);
    return sqrt(ss / (double)k + (double)eps);
}

// Outputs [first, first + count) of Q8(RMSNorm(x)) by one workgroup, one
// value per lane per round (blockDim.x must be a multiple of 64).
__device__ __forceinline__ void rmsnorm_quantize_range(const float* __restrict__ x, double denom, int k,
                                                       uint8_t* __restrict__ xq, int first, int count) {
#pragma clang fp contract(off)
    for (int base = first; base < first + count; base += blockDim.x) {
        const int idx = base + threadIdx.x;
        const bool in = idx < first + count && idx < k;
        const float v = in ? (float)((double)x[idx] / denom) : 0.0f;
        quantize_lane(v, xq + (int64_t)(idx >> 5) * kQ8Bytes, idx & 31, in);
    }
}

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// The f32 input of a GEMV whose q8_0 activation is Q8(RMSNorm(x)), formed in
// the GEMV's own prologue.  With sel_step, x is a table and row
// (*sel_step mod n_inputs) is used; q8_copy, if set, receives the q8_0
// vector from workgroup 0; inc_step, if set, is advanced by one by thread 0
// of workgroup 0 after it has staged its input (the kernel must not also
// read it through sel_step).
struct NormIn {
    const float* x;
    const int64_t* sel_step;
    int n_inputs;
    float eps;
    uint8_t* q8_copy;
    int64_t* inc_step;
};

// Q8(RMSNorm(x)) of k values (k % 32 == 0, x 16-byte aligned), computed by
// the whole workgroup (blockDim.x % 64 == 0) and written to lds in the
// layout of stage_q8.  Thread t owns the 4-value chunks t, t+T, ... (T =
// blockDim.x): it sums their squares in order, the workgroup adds the
// per-thread sums in the fixed order of block_sum_f64, and each value is
// divided by sqrt(mean + eps) in f64 and rounded to f32 once.  A q8_0
// block is then 8 consecutive chunks, i.e. 8 aligned lanes: its amax, f16
// scale and codes are formed with exactly the operations of quantize_lane.
// The caller synchronizes the workgroup before reading lds.
__device__ __forceinline__ void stage_rmsnorm_q8(const float* __restrict__ x, int k, float eps,
                                                 uint8_t* __restrict__ lds, double* sh,
                                                 uint8_t* __restrict__ q8_copy) {
#pragma clang fp contract(off)
    const int nch = k >> 2;
    const int T = blockDim.x;
    const float4* x4 = (const float4*)x;
    double ss = 0.0;
    for (int c = threadIdx.x; c < nch; c += T) {
        const float4 v = x4[c];
        ss += (double)v.x * (double)v.x;
        ss += (double)v.y * (double)v.y;
        ss += (double)v.z * (double)v.z;
        ss += (double)v.w * (double)v.w;
    }
    ss = block_sum_f64(ss, sh);
    const double denom = sqrt(ss / (double)k + (double)eps);
    const int rounds = (nch + T - 1) / T;
    for (int r = 0; r < rounds; ++r) {
        const int c = r * T + (int)threadIdx.x;
        const bool in = c < nch;      // whole 8-lane groups are in or out
        const float4 v = in ? x4[c] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        const float n[4] = {(float)((double)v.x / denom), (float)((double)v.y / denom),
                            (float)((double)v.z / denom), (float)((double)v.w / denom)};
        float amax = fmaxf(fmaxf(fabsf(n[0]), fabsf(n[1])), fmaxf(fabsf(n[2]), fabsf(n[3])));
        amax = fmaxf(amax, dpp_f32<0xB1>(amax));     // lane ^ 1
        amax = fmaxf(amax, dpp_f32<0x4E>(amax));     // lane ^ 2
        amax = fmaxf(amax, dpp_f32<0x141>(amax));    // the other quad of the 8
        const float d32 = amax / 127.0f;
        const uint32_t dbits = f32_to_f16(d32);
        const float d = f16_to_f32(dbits);
        uint32_t packed = 0;
        int s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int q = 0;
            if (d != 0.0f) {
                const float rq = roundf(n[i] / d);
                q = rq > 127.0f ? 127 : (rq < -127.0f ? -127 : (int)rq);
            }
            packed |= ((uint32_t)q & 0xFFu) << (8 * i);
            s += q;
        }
        s += dpp_i32<0xB1>(s);
        s += dpp_i32<0x4E>(s);
        s += dpp_i32<0x141>(s);
        if (in) {
            const int b = c >> 3, cb = c & 7;
            const int P = b >> 1, half = b & 1, L = P & 63;
            uint8_t* g = lds + (P >> 6) * kStageGroupBytes;
            *(uint32_t*)(g + ((2 * half + (cb >> 2)) * 64 + L) * 16 + (cb & 3) * 4) = packed;
            if (cb == 0) {
                *(double*)(g + 4096 + L * 16 + half * 8) = (double)d;
                *(double*)(g + 5120 + L * 16 + half * 8) = (double)d * (double)s;
            }
            if (q8_copy) {
                uint8_t* blk = q8_copy + (int64_t)b * kQ8Bytes;
                if (cb == 0) *(uint16_t*)blk = (uint16_t)dbits;
                *(uint16_t*)(blk + 2 + 4 * cb) = (uint16_t)(packed & 0xFFFFu);
                *(uint16_t*)(blk + 4 + 4 * cb) = (uint16_t)(packed >> 16);
            }
        }
    }
}

// Prologue of a GEMV fed by a NormIn: selects the input row, stages
// Q8(RMSNorm(x)) into lds and advances the step counter if asked.
__device__ __forceinline__ void stage_norm_input(const NormIn& in, int k, uint8_t* __restrict__ lds,
                                                 double* sh) {
    const float* x = in.x;
    if (in.sel_step) x += (int64_t)((uint64_t)*in.sel_step % (uint64_t)in.n_inputs) * k;
    stage_rmsnorm_q8(x, k, in.eps, lds, sh, blockIdx.x == 0 ? in.q8_copy : nullptr);
    if (in.inc_step && blockIdx.x == 0 && threadIdx.x == 0) *in.inc_step += 1;
}

// The glue stand-in between gate/up and down: silu(g)*u in f64, rounded to f32.
__device__ __forceinline__ float swiglu_value(float gate, float up) {
#pragma clang fp contract(off)
    const double g = gate;
    return (float)(g / (1.0 + exp(-g)) * (double)up);
}

}  // namespace mq
