// Streaming-read probe: the rate a plain read of a large buffer reaches on
// this GPU, measured in the same run as the GEMVs so that their bandwidth can
// be stated as a fraction of it as well as of the data-sheet peak.  Every
// 16-byte chunk is read once: each workgroup reads one contiguous range,
// its lanes side by side with four independent 16-byte loads in flight per
// lane (of 90 plain-read variants timed on MI355X, grid-stride or
// contiguous, 4 or 8 loads in flight, temporal or non-temporal, 256 to 4096
// workgroups of 256 to 1024 threads, this one held 6.25-6.27 TB/s at every
// grid size and the best was 6.35).  The 32-bit words are XOR-reduced
// (lane, wave, workgroup, then one atomic per workgroup), which keeps every
// load live and gives a result that can be checked exactly.
#include "common.hpp"
#include "launch.hpp"

namespace mq {

__global__ void k_set_u32(uint32_t* __restrict__ p, uint32_t v) { *p = v; }

__device__ __forceinline__ uint32_t xor4(const u32x4& a) { return a.x ^ a.y ^ a.z ^ a.w; }

__global__ __launch_bounds__(1024) void k_stream_read(const u32x4* __restrict__ p, int64_t n16,
                                                      uint32_t* __restrict__ xor_out) {
    __shared__ uint32_t part[16];
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
    const int64_t B = blockDim.x;
    int64_t i = b0 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * B < b1; i += 4 * B) {
        const u32x4 a = p[i], b = p[i + B], c = p[i + 2 * B], d = p[i + 3 * B];
        acc ^= xor4(a) ^ xor4(b) ^ xor4(c) ^ xor4(d);
    }
    for (; i < b1; i += B) acc ^= xor4(p[i]);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, s, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t v = 0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) v ^= part[w];
        atomicXor(xor_out, v);
    }
}

hipError_t launch_stream_read(const void* p, int64_t bytes, uint32_t* xor_out, int workgroups,
                              hipStream_t stream) {
    hipLaunchKernelGGL(k_set_u32, dim3(1), dim3(1), 0, stream, xor_out, 0u);
    const int g = workgroups > 0 ? workgroups : device_cu_count();
    hipLaunchKernelGGL(k_stream_read, dim3(g), dim3(1024), 0, stream, (const u32x4*)p, bytes / 16, xor_out);
    return hipGetLastError();
}

}  // namespace mq
