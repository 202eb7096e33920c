// q8_0 quantization and the elementwise glue of the decode step, fused with
// quantization of their outputs.
//
// Quantization decides integers from floats, so it runs in f32 with only
// exactly specified operations: a max over magnitudes (order-independent,
// 'Part 4 · Lecture 08 — Graph-Resident Decode', §8), an IEEE f32 divide,
// f16 round-to-nearest-even of the scale and roundf.  The glue itself is
// computed in f64 and rounded to f32 once, then quantized.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

#pragma clang fp contract(off)

namespace mq {

// One q8_0 block from 32 f32 values: returns the f16 scale bits and codes.
__device__ __forceinline__ void quantize_block(const float (&v)[32], uint8_t* __restrict__ out) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float d32 = amax / 127.0f;
    const uint32_t dbits = f32_to_f16(d32);
    const float d = f16_to_f32(dbits);
    uint16_t* o = (uint16_t*)out;                  // q8_0 blocks are 2-byte aligned
    o[0] = (uint16_t)dbits;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        int q[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int qi = 0;
            if (d != 0.0f) {
                const float r = roundf(v[2 * i + h] / d);
                qi = r > 127.0f ? 127 : (r < -127.0f ? -127 : (int)r);
            }
            q[h] = qi;
        }
        o[1 + i] = (uint16_t)((q[0] & 0xFF) | ((q[1] & 0xFF) << 8));
    }
}

__device__ __forceinline__ void zero_block(uint8_t* __restrict__ out) {
    uint16_t* o = (uint16_t*)out;
#pragma unroll
    for (int i = 0; i < 17; ++i) o[i] = 0;
}

__global__ __launch_bounds__(256) void k_quantize_q8_0(const float* __restrict__ x,
                                                      uint8_t* __restrict__ xq, int64_t nblocks) {
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = x[32 * b + i];
    quantize_block(v, xq + b * kQ8Bytes);
}

// Sum of a per-thread f64 value over the workgroup, fixed order: DPP/swizzle
// inside each wave, then the wave sums added in wave order by one thread.
__device__ double block_sum_f64(double v, double* sh) {
    v = wave_sum_f64(v);
    const int nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int i = 0; i < nw; ++i) t += sh[i];
        sh[16] = t;
    }
    __syncthreads();
    return sh[16];
}

// One workgroup: RMSNorm over k values (unit gain), then quantize.
__global__ __launch_bounds__(1024) void k_rmsnorm_quantize(const float* __restrict__ x,
                                                          uint8_t* __restrict__ xq, int k, float eps,
                                                          int64_t* __restrict__ step, int n_inputs) {
    __shared__ double sh[17];
    __shared__ int64_t row_sh;
    if (step) {
        if (threadIdx.x == 0) {
            const int64_t s = *step;
            row_sh = (int64_t)((uint64_t)s % (uint64_t)n_inputs);
            *step = s + 1;
        }
        __syncthreads();
        x += row_sh * k;
    }
    double ss = 0.0;
    for (int i = threadIdx.x; i < k; i += blockDim.x) ss += (double)x[i] * (double)x[i];
    ss = block_sum_f64(ss, sh);
    const double denom = sqrt(ss / (double)k + (double)eps);
    for (int b = threadIdx.x; b < k / 32; b += blockDim.x) {
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = (float)((double)x[32 * b + i] / denom);
        quantize_block(v, xq + (int64_t)b * kQ8Bytes);
    }
}

// Per column: y_i = silu(gate_i)*up_i on [gate | up], quantized; blocks past
// inter/32 are zero blocks.
__global__ __launch_bounds__(256) void k_swiglu_quantize(const float* __restrict__ gu,
                                                        uint8_t* __restrict__ xq, int64_t inter,
                                                        int n_cols, int64_t nbp) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)n_cols * nbp) return;
    const int64_t c = idx / nbp, b = idx % nbp;
    uint8_t* out = xq + idx * kQ8Bytes;
    if (b >= inter / 32) {
        zero_block(out);
        return;
    }
    const float* g = gu + c * 2 * inter + 32 * b;
    const float* u = g + inter;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const double gd = g[i];
        v[i] = (float)(gd / (1.0 + exp(-gd)) * (double)u[i]);
    }
    quantize_block(v, out);
}

__global__ __launch_bounds__(256) void k_moe_prep(int64_t* __restrict__ step, int64_t* __restrict__ cur,
                                                 int n_tokens, const int32_t* __restrict__ ids_table,
                                                 const float* __restrict__ logits_table,
                                                 const float* __restrict__ x_table, int n_sel, int hidden,
                                                 int32_t* __restrict__ ids_out,
                                                 float* __restrict__ combine_out,
                                                 uint8_t* __restrict__ xq_out) {
    __shared__ int64_t t_sh;
    if (threadIdx.x == 0) {
        const int64_t s = *step;
        const int64_t t = (int64_t)((uint64_t)s % (uint64_t)n_tokens);
        t_sh = t;
        *cur = t;
        *step = s + 1;
        // softmax of the n_sel router logits, f64, in slot order
        const float* lg = logits_table + t * n_sel;
        double mx = -INFINITY;
        for (int i = 0; i < n_sel; ++i) mx = fmax(mx, (double)lg[i]);
        double sum = 0.0;
        for (int i = 0; i < n_sel; ++i) sum += exp((double)lg[i] - mx);
        for (int i = 0; i < n_sel; ++i) combine_out[i] = (float)(exp((double)lg[i] - mx) / sum);
    }
    __syncthreads();
    const int64_t t = t_sh;
    if (threadIdx.x < n_sel) ids_out[threadIdx.x] = ids_table[t * n_sel + threadIdx.x];
    const float* x = x_table + t * hidden;
    for (int b = threadIdx.x; b < hidden / 32; b += blockDim.x) {
        float v[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = x[32 * b + i];
        quantize_block(v, xq_out + (int64_t)b * kQ8Bytes);
    }
}

__global__ void k_set_i64(int64_t* p, int64_t v) { *p = v; }

// ------------------------------------------------------------------ host ----

hipError_t launch_quantize_q8_0(const float* x, void* xq, int64_t k, int n_cols, hipStream_t stream) {
    const int64_t nblocks = (k / 32) * n_cols;
    hipLaunchKernelGGL(k_quantize_q8_0, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, stream, x,
                       (uint8_t*)xq, nblocks);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_quantize(const float* x, void* xq, int64_t k, float eps, int64_t* step,
                                   int n_inputs, hipStream_t stream) {
    hipLaunchKernelGGL(k_rmsnorm_quantize, dim3(1), dim3(1024), 0, stream, x, (uint8_t*)xq, (int)k, eps,
                       step, n_inputs);
    return hipGetLastError();
}

hipError_t launch_swiglu_quantize(const float* gu, void* xq, int64_t inter, int n_cols, int64_t k_pad,
                                  hipStream_t stream) {
    const int64_t nbp = k_pad / 32;
    const int64_t n = nbp * n_cols;
    hipLaunchKernelGGL(k_swiglu_quantize, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, gu,
                       (uint8_t*)xq, inter, n_cols, nbp);
    return hipGetLastError();
}

hipError_t launch_moe_prep(int64_t* step, int64_t* cur, int n_tokens, const int32_t* ids_table,
                           const float* logits_table, const float* x_table, int n_sel, int64_t hidden,
                           int32_t* ids_out, float* combine_out, void* xq_out, hipStream_t stream) {
    hipLaunchKernelGGL(k_moe_prep, dim3(1), dim3(256), 0, stream, step, cur, n_tokens, ids_table,
                       logits_table, x_table, n_sel, (int)hidden, ids_out, combine_out, (uint8_t*)xq_out);
    return hipGetLastError();
}

hipError_t launch_set_i64(int64_t* p, int64_t v, hipStream_t stream) {
    hipLaunchKernelGGL(k_set_i64, dim3(1), dim3(1), 0, stream, p, v);
    return hipGetLastError();
}

}  // namespace mq
