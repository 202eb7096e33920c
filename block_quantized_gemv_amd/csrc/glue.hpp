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

// The glue stand-in between gate/up and down: silu(g)*u in f64, rounded to f32.
__device__ __forceinline__ float swiglu_value(float gate, float up) {
#pragma clang fp contract(off)
    const double g = gate;
    return (float)(g / (1.0 + exp(-g)) * (double)up);
}

}  // namespace mq
