// Synchronization probes: what a resident ("persistent") decode kernel would
// pay at each GEMV boundary, measured against what a graph pays.
//
// A persistent step keeps one workgroup per CU for the whole step and
// separates consecutive GEMVs with a grid-wide barrier; every GEMV reads the
// whole vector the previous one wrote, so the barrier must also carry that
// vector from every workgroup to every workgroup across the XCDs' separate
// L2 caches.  k_grid_barrier_probe times exactly that, round after round:
// each workgroup writes its slice of a vector with agent-scope (write-
// through) stores, waits for them to complete, meets the others at the
// barrier, then reads the whole vector back with agent-scope loads and
// checks every word.  Two barriers:
//   flat  - every workgroup adds to one agent-scope counter and polls it;
//   xcc   - workgroups first count in per-XCD counters (the XCD read from
//           the XCC_ID hardware register); the last one of each XCD
//           counts in a global counter and, once all XCDs have, releases
//           its XCD through a per-XCD flag that only that XCD polls.
// Every wait is bounded: past kSpinLimit polls the kernel sets an error
// flag that ends every other wait, so the grid always drains.
// k_empty is the graph side: a captured sequence of empty kernels on the
// same grid gives the cost of one kernel boundary in a replay.
#include "common.hpp"
#include "launch.hpp"

namespace mq {
namespace {

struct BarrierCtl {                    // each word on its own 256-byte line
    uint32_t cnt[64], hcnt[64], hrel[64], nx[64], err[64];
    uint32_t xcnt[16][64], xrel[16][64], xn[16][64];
    unsigned long long t[2];
};
constexpr uint32_t kSpinLimit = 1u << 20;

__device__ __forceinline__ uint32_t xcc_id() { return __builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u; }
__device__ __forceinline__ uint32_t ld_agent(uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_agent(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until *p >= target; false once the error flag is set (by this wait
// running out of polls, or by any other).
__device__ bool wait_geq(BarrierCtl* c, uint32_t* p, uint32_t target) {
    for (uint32_t i = 0; i < kSpinLimit; ++i) {
        if (ld_agent(p) >= target) return true;
        if (ld_agent(c->err)) return false;
        __builtin_amdgcn_s_sleep(1);
    }
    st_agent(c->err, 1u);
    return false;
}

// Barrier number e (1, 2, ...) over G workgroups, one thread each.
__device__ void flat_barrier(BarrierCtl* c, uint32_t G, uint32_t e) {
    add_agent(c->cnt, 1u);
    wait_geq(c, c->cnt, e * G);
}
__device__ void xcc_barrier(BarrierCtl* c, uint32_t x, uint32_t n_here, uint32_t n_xcc, uint32_t e) {
    if (add_agent(c->xcnt[x], 1u) == e * n_here - 1) {
        if (add_agent(c->hcnt, 1u) == e * n_xcc - 1) st_agent(c->hrel, e);
        else wait_geq(c, c->hrel, e);
        st_agent(c->xrel[x], e);
    } else {
        wait_geq(c, c->xrel[x], e);
    }
}

__device__ __forceinline__ uint32_t tag(int r, uint32_t i) { return (uint32_t)r * 0x9E3779B1u + i * 2654435761u + 1u; }

__global__ __launch_bounds__(1024) void k_grid_barrier_probe(BarrierCtl* __restrict__ c, int hier, int rounds,
                                                             uint32_t* __restrict__ vec, int words,
                                                             uint32_t* __restrict__ bad) {
    const uint32_t G = gridDim.x, b = blockIdx.x, tid = threadIdx.x;
    __shared__ uint32_t s_x, s_here, s_nxcc;
    if (tid == 0) {
        // set-up: count the workgroups of each XCD (two flat barriers, so
        // that the counts are complete before anyone reads them and read
        // before the counters below are used)
        const uint32_t x = xcc_id();
        if (add_agent(c->xn[x], 1u) == 0) add_agent(c->nx, 1u);
        flat_barrier(c, G, 1);
        s_x = x;
        s_here = ld_agent(c->xn[x]);
        s_nxcc = ld_agent(c->nx);
        flat_barrier(c, G, 2);
    }
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    const uint32_t n = G * (uint32_t)words;
    uint32_t nbad = 0;
    for (int r = 0; r < rounds; ++r) {
        uint32_t* v = vec + (size_t)(r & 1) * n;      // two buffers: round r+2 writes after barrier r+1
        for (uint32_t i = tid; i < (uint32_t)words; i += blockDim.x) st_agent(&v[b * words + i], tag(r, b * words + i));
        __builtin_amdgcn_s_waitcnt(0);                 // this thread's stores have completed
        __syncthreads();
        if (tid == 0) {
            if (hier) xcc_barrier(c, s_x, s_here, s_nxcc, (uint32_t)r + 1);
            else flat_barrier(c, G, (uint32_t)r + 3);
        }
        __syncthreads();
        for (uint32_t i = tid; i < n; i += blockDim.x) nbad += ld_agent(&v[i]) != tag(r, i);
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
    if (nbad) atomicAdd(bad, nbad);
    if (b == 0 && tid == 0) {
        c->t[0] = t0;
        c->t[1] = t1;
    }
}

__global__ void k_empty() {}

}  // namespace

int grid_barrier_probe(int hierarchical, int words, int rounds, int threads, double* us_per_round,
                       uint32_t* bad_words, int* spin_limit_hit, hipStream_t stream) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_grid_barrier_probe, threads, 0) != hipSuccess || occ < 1)
        return 1;                                           // the grid could not be co-resident
    const int G = device_cu_count();
    BarrierCtl* c = nullptr;
    uint32_t *vec = nullptr, *bad = nullptr;
    const size_t vec_bytes = (size_t)2 * G * (words > 0 ? words : 1) * sizeof(uint32_t);
    hipError_t e = hipMalloc(&c, sizeof(BarrierCtl));
    if (e == hipSuccess) e = hipMalloc(&vec, vec_bytes);
    if (e == hipSuccess) e = hipMalloc(&bad, sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemsetAsync(c, 0, sizeof(BarrierCtl), stream);
    if (e == hipSuccess) e = hipMemsetAsync(vec, 0, vec_bytes, stream);
    if (e == hipSuccess) e = hipMemsetAsync(bad, 0, sizeof(uint32_t), stream);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(k_grid_barrier_probe, dim3(G), dim3(threads), 0, stream, c, hierarchical, rounds, vec, words,
                           bad);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    BarrierCtl h;
    if (e == hipSuccess) e = hipMemcpy(&h, c, sizeof(BarrierCtl), hipMemcpyDeviceToHost);
    if (e == hipSuccess) e = hipMemcpy(bad_words, bad, sizeof(uint32_t), hipMemcpyDeviceToHost);
    if (e == hipSuccess) {
        *us_per_round = (double)(h.t[1] - h.t[0]) * 0.01 / rounds;
        *spin_limit_hit = h.err[0] != 0;
    }
    (void)hipFree(c);
    (void)hipFree(vec);
    (void)hipFree(bad);
    return e == hipSuccess ? 0 : 2;
}

int graph_boundary_probe(int n_kernels, int threads, int reps, double* us_per_kernel) {
    const int G = device_cu_count();
    hipStream_t s = nullptr;
    hipGraph_t g = nullptr;
    hipGraphExec_t ge = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
        for (int i = 0; i < n_kernels; ++i) hipLaunchKernelGGL(k_empty, dim3(G), dim3(threads), 0, s);
        e = hipStreamEndCapture(s, &g);
    }
    if (e == hipSuccess) e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
    for (int w = 0; w < 3 && e == hipSuccess; ++w) e = hipGraphLaunch(ge, s);
    if (e == hipSuccess) e = hipEventRecord(e0, s);
    for (int r = 0; r < reps && e == hipSuccess; ++r) e = hipGraphLaunch(ge, s);
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess) *us_per_kernel = (double)ms * 1e3 / ((double)reps * n_kernels);
    if (ge) (void)hipGraphExecDestroy(ge);
    if (g) (void)hipGraphDestroy(g);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (s) (void)hipStreamDestroy(s);
    return e == hipSuccess ? 0 : 2;
}

}  // namespace mq
