// Streaming-read probe: the rate a plain read of a large buffer reaches on
// this GPU, measured in the same run as the GEMVs so that their bandwidth can
// be stated as a fraction of it as well as of the data-sheet peak.  Every
// 16-byte chunk is read once, in a grid-stride loop with four independent
// 16-byte loads in flight per lane; the 32-bit words are XOR-reduced (lane,
// wave, workgroup, then one atomic per workgroup), which keeps every load
// live and gives a result that can be checked exactly.
#include "common.hpp"
#include "launch.hpp"

namespace mq {

__global__ void k_set_u32(uint32_t* __restrict__ p, uint32_t v) { *p = v; }

__device__ __forceinline__ uint32_t xor4(const u32x4& a) { return a.x ^ a.y ^ a.z ^ a.w; }

__global__ __launch_bounds__(1024) void k_stream_read(const u32x4* __restrict__ p, int64_t n16,
                                                      uint32_t* __restrict__ xor_out) {
    __shared__ uint32_t part[16];
    const int64_t T = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * T < n16; i += 4 * T) {
        const u32x4 a = p[i], b = p[i + T], c = p[i + 2 * T], d = p[i + 3 * T];
        acc ^= xor4(a) ^ xor4(b) ^ xor4(c) ^ xor4(d);
    }
    for (; i < n16; i += T) acc ^= xor4(p[i]);
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
