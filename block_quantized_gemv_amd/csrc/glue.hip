// Standalone glue kernels: q8_0 quantization, RMSNorm and SwiGLU fused with
// quantization of their outputs, and a counter setter.  One value per lane; the arithmetic lives in glue.hpp and
// is shared with the fused tails of the GEMV kernels, so both produce the
// same bytes.
#include "common.hpp"
#include "glue.hpp"
#include "launch.hpp"

#pragma clang fp contract(off)

namespace mq {

// x: n_cols rows of k values; one lane per value.
__global__ __launch_bounds__(256) void k_quantize_q8_0(const float* __restrict__ x,
                                                      uint8_t* __restrict__ xq, int64_t n) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool in = idx < n;
    const float v = in ? x[idx] : 0.0f;
    quantize_lane(v, xq + (idx >> 5) * kQ8Bytes, (int)(idx & 31), in);
}

// RMSNorm over k values (unit gain), quantized; every workgroup computes
// the (identical) sum of squares and handles 256 outputs.  With sel_step the
// input is row (step % n_inputs) of x; inc_step, when given, is advanced by
// one by a single thread (it must not be read by this kernel).
__global__ __launch_bounds__(256) void k_rmsnorm_quantize(const float* __restrict__ x,
                                                         uint8_t* __restrict__ xq, int k, float eps,
                                                         const int64_t* __restrict__ sel_step, int n_inputs,
                                                         int64_t* __restrict__ inc_step) {
    __shared__ double sh[16];
    if (sel_step) x += (int64_t)((uint64_t)*sel_step % (uint64_t)n_inputs) * k;
    const float scale = rms_scale(x, k, eps, sh);
    rmsnorm_quantize_range(x, scale, k, xq, blockIdx.x * blockDim.x, blockDim.x);
    if (inc_step && blockIdx.x == 0 && threadIdx.x == 0) *inc_step += 1;
}

// Per column c: y_i = silu(gate_i)*up_i on [gate | up], quantized; lanes past
// inter form zero blocks (d = 0, q = 0).
__global__ __launch_bounds__(256) void k_swiglu_quantize(const float* __restrict__ gu,
                                                        uint8_t* __restrict__ xq, int64_t inter,
                                                        int n_cols, int64_t k_pad) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool in = idx < (int64_t)n_cols * k_pad;
    const int64_t c = idx / k_pad, i = idx % k_pad;
    float v = 0.0f;
    if (in && i < inter) v = swiglu_value(gu[c * 2 * inter + i], gu[c * 2 * inter + inter + i]);
    quantize_lane(v, xq + (idx >> 5) * kQ8Bytes, (int)(idx & 31), in);
}

__global__ void k_set_i64(int64_t* p, int64_t v) { *p = v; }

__global__ void k_zero_u32(uint32_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// ------------------------------------------------------------------ host ----

hipError_t launch_quantize_q8_0(const float* x, void* xq, int64_t k, int n_cols, hipStream_t stream) {
    const int64_t n = k * n_cols;
    hipLaunchKernelGGL(k_quantize_q8_0, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, x,
                       (uint8_t*)xq, n);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_quantize(const float* x, void* xq, int64_t k, float eps, const int64_t* sel_step,
                                   int n_inputs, int64_t* inc_step, hipStream_t stream) {
    hipLaunchKernelGGL(k_rmsnorm_quantize, dim3((unsigned)((k + 255) / 256)), dim3(256), 0, stream, x,
                       (uint8_t*)xq, (int)k, eps, sel_step, n_inputs, inc_step);
    return hipGetLastError();
}

hipError_t launch_swiglu_quantize(const float* gu, void* xq, int64_t inter, int n_cols, int64_t k_pad,
                                  hipStream_t stream) {
    const int64_t n = k_pad * n_cols;
    hipLaunchKernelGGL(k_swiglu_quantize, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, gu,
                       (uint8_t*)xq, inter, n_cols, k_pad);
    return hipGetLastError();
}

hipError_t launch_set_i64(int64_t* p, int64_t v, hipStream_t stream) {
    hipLaunchKernelGGL(k_set_i64, dim3(1), dim3(1), 0, stream, p, v);
    return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

}  // namespace mq
