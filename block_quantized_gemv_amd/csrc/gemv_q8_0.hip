// q8_0 x q8_0 GEMV (the lm_head of the decode step) for gfx950.
//
// Each lane takes a pair of weight blocks (68 bytes = 17 dwords, dword
// aligned because rows hold an even number of blocks): four 16-byte loads
// plus one dword.  The first block's codes start 2 bytes into the pair and
// are realigned with v_alignbyte; the second block's codes are aligned.
// Rows get aligned lane slots as in the q4_K kernel; the activation is
// staged in LDS with the same layout.
#include "common.hpp"
#include "launch.hpp"

namespace mq {

template <bool DUMP>
__global__ __launch_bounds__(256) void k_gemv_q8_0(const uint8_t* __restrict__ w,
                                                  const uint8_t* __restrict__ xq,
                                                  float* __restrict__ y, int32_t* __restrict__ dump_isum,
                                                  int M, int npairs, int log2s, int passes,
                                                  int n_tiles) {
    extern __shared__ __align__(16) uint8_t lds[];
    stage_q8(xq, 0, 2 * npairs, lds, threadIdx.x, blockDim.x, nullptr);
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int S = 1 << log2s, R = 64 >> log2s;
    const int row_local = lane >> log2s, slot = lane & (S - 1);
    const int wave_stride = gridDim.x * (blockDim.x >> 6);
    for (int tile = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); tile < n_tiles;
         tile += wave_stride) {
        const int row = tile * R + row_local;
        double acc = 0.0;
        for (int p = 0; p < passes; ++p) {
            const int P = p * S + slot;
            if (row < M && P < npairs) {
                const uint8_t* base = w + ((int64_t)row * npairs + P) * (2 * kQ8Bytes);
                const u32x4 v0 = __builtin_nontemporal_load((const u32x4_a4*)(base));
                const u32x4 v1 = __builtin_nontemporal_load((const u32x4_a4*)(base + 16));
                const u32x4 v2 = __builtin_nontemporal_load((const u32x4_a4*)(base + 32));
                const u32x4 v3 = __builtin_nontemporal_load((const u32x4_a4*)(base + 48));
                const uint32_t v4 = __builtin_nontemporal_load((const uint32_t*)(base + 64));
                const uint32_t dw[17] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w,
                                         v2.x, v2.y, v2.z, v2.w, v3.x, v3.y, v3.z, v3.w, v4};
                StagedPair x;
                read_pair(lds, P, x, false);
                int ia = 0, ib = 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    ia = dot4(__builtin_amdgcn_alignbyte(dw[k + 1], dw[k], 2), x.c[k], ia);
                    ib = dot4(dw[9 + k], x.c[8 + k], ib);
                }
                const double da = (double)f16_to_f32(dw[0]);
                const double db = (double)f16_to_f32(dw[8] >> 16);
                // d_w*d_x has < 24 significant bits and |isum| < 2^20: each
                // product is exact in f64.
                acc += (double)ia * (da * x.d0);
                acc += (double)ib * (db * x.d1);
                if (DUMP) {
                    dump_isum[(int64_t)row * 2 * npairs + 2 * P] = ia;
                    dump_isum[(int64_t)row * 2 * npairs + 2 * P + 1] = ib;
                }
            }
        }
        const double v = group_sum_f64(acc, log2s);
        if (slot == 0 && row < M) y[row] = (float)v;
    }
}

Q8Plan plan_q8_0(int64_t m, int npairs) {
    Q8Plan p;
    int l = 0;
    while ((1 << l) < npairs) ++l;
    if (l < 2) l = 2;
    if (l > 6) l = 6;
    p.log2s = l;
    p.rows_per_tile = 64 >> l;
    p.passes = (npairs + (1 << l) - 1) >> l;
    p.n_tiles = (int)((m + p.rows_per_tile - 1) / p.rows_per_tile);
    return p;
}

hipError_t launch_gemv_q8_0(const void* w, const void* xq, float* y, int32_t* dump_isum, int64_t m,
                            int64_t k, hipStream_t stream) {
    const int npairs = (int)(k / 64);
    const Q8Plan p = plan_q8_0(m, npairs);
    const int lds = stage_bytes(2 * npairs);
    const int cap = device_cu_count() * 8;
    int grid = (p.n_tiles + 3) / 4;
    if (grid > cap) grid = cap;
    if (dump_isum)
        hipLaunchKernelGGL(k_gemv_q8_0<true>, dim3(grid), dim3(256), lds, stream, (const uint8_t*)w,
                           (const uint8_t*)xq, y, dump_isum, (int)m, npairs, p.log2s, p.passes, p.n_tiles);
    else
        hipLaunchKernelGGL(k_gemv_q8_0<false>, dim3(grid), dim3(256), lds, stream, (const uint8_t*)w,
                           (const uint8_t*)xq, y, nullptr, (int)m, npairs, p.log2s, p.passes, p.n_tiles);
    return hipGetLastError();
}

}  // namespace mq
