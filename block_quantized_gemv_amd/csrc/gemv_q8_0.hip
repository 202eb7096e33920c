// q8_0 x q8_0 GEMV (the lm_head of the decode step) for gfx950.
//
// Each lane takes a pair of weight blocks (68 bytes = 17 dwords, dword
// aligned because rows hold an even number of blocks): four 16-byte loads
// plus one dword.  The first block's codes start 2 bytes into the pair and
// are realigned with v_alignbyte; the second block's codes are aligned.
// Rows get aligned slots of S lanes, a wave holds 64/S rows; the activation
// is staged in LDS with the same layout as the q4_K kernels, and items are
// streamed with the same ping-pong register buffers.
#include <hip/hip_ext.h>

#include "common.hpp"
#include "glue.hpp"
#include "launch.hpp"

namespace mq {

struct PairLoad {
    u32x4 v0, v1, v2, v3;
    uint32_t v4;
};

// Ordinary loads: neighbouring lanes' pairs share cache lines across the
// five instructions, so a non-temporal hint would cost re-fetches.
__device__ __forceinline__ void load_pair(const uint8_t* __restrict__ p, PairLoad& L) {
    L.v0 = *(const u32x4_a4*)(p);
    L.v1 = *(const u32x4_a4*)(p + 16);
    L.v2 = *(const u32x4_a4*)(p + 32);
    L.v3 = *(const u32x4_a4*)(p + 48);
    L.v4 = *(const uint32_t*)(p + 64);
}

template <bool DUMP>
__device__ __forceinline__ double pair_item(const PairLoad& L, const uint8_t* __restrict__ lds, int P,
                                            int32_t* __restrict__ dump, int64_t dump_off, bool valid) {
    const uint32_t dw[17] = {L.v0.x, L.v0.y, L.v0.z, L.v0.w, L.v1.x, L.v1.y, L.v1.z, L.v1.w,
                             L.v2.x, L.v2.y, L.v2.z, L.v2.w, L.v3.x, L.v3.y, L.v3.z, L.v3.w, L.v4};
    StagedPair x;
    read_pair(lds, P, x, false);
    int ia = 0, ib = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        ia = dot4(__builtin_amdgcn_alignbyte(dw[k + 1], dw[k], 2), x.c[k], ia);
        ib = dot4(dw[9 + k], x.c[8 + k], ib);
    }
    if (DUMP && valid) {
        dump[dump_off + 2 * P] = ia;
        dump[dump_off + 2 * P + 1] = ib;
    }
    // d_w*d_x has < 24 significant bits and |isum| < 2^20: each product is
    // exact in f64, only the addition rounds.
    const double da = (double)f16_to_f32(dw[0]) * x.d0;
    const double db = (double)f16_to_f32(dw[8] >> 16) * x.d1;
    return fma((double)ia, da, (double)ib * db);
}

// With NORM the activation is Q8(RMSNorm(x)) of the f32 vector `nin`
// describes, formed in each workgroup's prologue (workgroups of up to 1024
// threads, about one per CU); otherwise xq holds it.
template <bool DUMP, bool NORM, bool ST = false>
__global__ __launch_bounds__(NORM ? 1024 : 256) void k_gemv_q8_0(const uint8_t* __restrict__ w,
                                                                const uint8_t* __restrict__ xq,
                                                                float* __restrict__ y,
                                                                int32_t* __restrict__ dump_isum, int M,
                                                                int npairs, int log2s, int passes,
                                                                int n_tiles, NormIn nin) {
    const SpanStamp<ST> span(nin.stamp);
    extern __shared__ __align__(16) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int S = 1 << log2s, R = 64 >> log2s;
    const int row_local = lane >> log2s, slot = lane & (S - 1);
    const int W = gridDim.x * (blockDim.x >> 6);
    // With NORM, consecutive units go to different workgroups (one per CU).
    const int wave = NORM ? wave_id() * (int)gridDim.x + (int)blockIdx.x
                          : blockIdx.x * (blockDim.x >> 6) + wave_id();
    const int my_tiles = wave < n_tiles ? (n_tiles - 1 - wave) / W + 1 : 0;
    const int n_items = my_tiles * passes;
    const int64_t row_bytes = (int64_t)npairs * 2 * kQ8Bytes;

    // Items past the wave's last one re-read that item's lines and are not
    // computed (one fixed address for all waves would queue thousands of
    // requests on a single channel).
    struct Item {
        PairLoad L;
        bool valid;
        int row, pass, P;
    };
    auto fetch = [&](int i, Item& it) {
        const bool past = i >= n_items;
        const int ii = past ? (n_items > 0 ? n_items - 1 : 0) : i;
        const int t = wave + (ii / passes) * W;
        it.pass = ii % passes;
        it.row = t * R + row_local;
        it.P = it.pass * S + slot;
        const bool inb = n_items > 0 && it.row < M && it.P < npairs;
        it.valid = inb && !past;
        load_pair(inb ? w + (int64_t)it.row * row_bytes + it.P * (2 * kQ8Bytes) : w, it.L);
        if (past) it.row = M;
    };

    float4 xr[kNormRegChunks];
    const float* xin = nullptr;
    if constexpr (NORM) {
        xin = norm_row(nin, 64 * npairs);
        norm_load(xin, 64 * npairs, xr);
    }
    Item A, B;
    fetch(0, A);
    if constexpr (NORM) fetch(1, B);
    if constexpr (NORM) {
        __shared__ double sh[16];
        stage_norm_input(nin, xin, 64 * npairs, xr, lds, sh);
    } else {
        stage_q8(xq, 0, 2 * npairs, lds, threadIdx.x, blockDim.x, nullptr);
    }
    __syncthreads();

    double acc = 0.0;
    stream_items<NORM>(n_items, A, B, fetch, [&](const Item& it) {
        const double v = pair_item<DUMP>(it.L, lds, it.valid ? it.P : 0, dump_isum,
                                         (int64_t)it.row * 2 * npairs, it.valid);
        acc += it.valid ? v : 0.0;
        if (it.pass != passes - 1) return;
        const double s = group_sum_f64(acc, log2s);
        acc = 0.0;
        if (slot == 0 && it.row < M) y[it.row] = (float)s;
    });
}

Q8Plan plan_q8_0(int64_t m, int npairs) {
    // Slot of S lanes per row: one pass when the row fits in 64 lanes;
    // otherwise 64 lanes and several passes.
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
    const void* fn = dump_isum ? (const void*)k_gemv_q8_0<true, false> : (const void*)k_gemv_q8_0<false, false>;
    const int64_t wmax = (int64_t)device_cu_count() * blocks_per_cu(fn, 256, lds) * 4;
    const int64_t per = (p.n_tiles + wmax - 1) / wmax;
    const int64_t waves = (p.n_tiles + per - 1) / per;
    const int grid = (int)((waves + 3) / 4);
    hipEvent_t e0, e1;
    const bool timed = take_next_launch_events(&e0, &e1);
    if (timed) (void)hipStreamSynchronize(stream);   // start on an idle stream (see MQ_LAUNCH)
    if (dump_isum)
        hipLaunchKernelGGL((k_gemv_q8_0<true, false>), dim3(grid), dim3(256), lds, stream, (const uint8_t*)w,
                           (const uint8_t*)xq, y, dump_isum, (int)m, npairs, p.log2s, p.passes, p.n_tiles,
                           NormIn{});
    else if (timed)
        hipExtLaunchKernelGGL((k_gemv_q8_0<false, false>), dim3(grid), dim3(256), lds, stream, e0, e1, 0,
                              (const uint8_t*)w, (const uint8_t*)xq, y, (int32_t*)nullptr, (int)m, npairs,
                              p.log2s, p.passes, p.n_tiles, NormIn{});
    else
        hipLaunchKernelGGL((k_gemv_q8_0<false, false>), dim3(grid), dim3(256), lds, stream, (const uint8_t*)w,
                           (const uint8_t*)xq, y, (int32_t*)nullptr, (int)m, npairs, p.log2s, p.passes,
                           p.n_tiles, NormIn{});
    return hipGetLastError();
}

hipError_t launch_gemv_q8_0_norm(const void* w, const NormIn& nin, float* y, int64_t m, int64_t k,
                                 hipStream_t stream) {
    const int npairs = (int)(k / 64);
    const Q8Plan p = plan_q8_0(m, npairs);
    const int lds = stage_bytes(2 * npairs);
    int grid = 1, threads = 64;
    prologue_grid(p.n_tiles, k / 4, &grid, &threads, kWavesQ8Norm);
    hipEvent_t e0, e1;
    if (take_next_launch_events(&e0, &e1)) {
        (void)hipStreamSynchronize(stream);
        hipExtLaunchKernelGGL((k_gemv_q8_0<false, true>), dim3(grid), dim3(threads), lds, stream, e0, e1, 0,
                              (const uint8_t*)w, (const uint8_t*)nullptr, y, (int32_t*)nullptr, (int)m, npairs,
                              p.log2s, p.passes, p.n_tiles, nin);
    } else if (nin.stamp) {
        hipLaunchKernelGGL((k_gemv_q8_0<false, true, true>), dim3(grid), dim3(threads), lds, stream,
                           (const uint8_t*)w, (const uint8_t*)nullptr, y, (int32_t*)nullptr, (int)m, npairs, p.log2s,
                           p.passes, p.n_tiles, nin);
    } else {
        hipLaunchKernelGGL((k_gemv_q8_0<false, true>), dim3(grid), dim3(threads), lds, stream, (const uint8_t*)w,
                           (const uint8_t*)nullptr, y, (int32_t*)nullptr, (int)m, npairs, p.log2s, p.passes,
                           p.n_tiles, nin);
    }
    return hipGetLastError();
}

}  // namespace mq
