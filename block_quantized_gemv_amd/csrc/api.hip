// The extern "C" boundary of libmq: argument validation (host only, before
// any HIP call), error reporting, and the graph-captured decode-step chains.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <functional>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mq.h"
#include "common.hpp"
#include "launch.hpp"

using namespace mq;

namespace {

thread_local std::string g_err;
std::atomic<unsigned> g_fault{MQ_FAULT_NONE};

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return MQ_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(MQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

#define CHECK_ARG(cond, ...) \
    do { if (!(cond)) return fail(MQ_ERR_ARG, __VA_ARGS__); } while (0)
#define CHECK_SHAPE(cond, ...) \
    do { if (!(cond)) return fail(MQ_ERR_SHAPE, __VA_ARGS__); } while (0)

constexpr int64_t kMaxRows = (int64_t)1 << 30;
constexpr int64_t kMaxK = (int64_t)1 << 24;

int check_q4k(const void* w, const void* xq, const float* y, int64_t m, int64_t k) {
    CHECK_ARG(w && xq && y, "null pointer (w=%p xq=%p y=%p)", w, xq, (const void*)y);
    CHECK_ARG(aligned(w, 16), "q4_K weights must be 16-byte aligned");
    CHECK_ARG(aligned(xq, 2), "q8_0 activation must be 2-byte aligned");
    CHECK_ARG(aligned(y, 4), "y must be 4-byte aligned");
    CHECK_SHAPE(m >= 1 && m <= kMaxRows, "m=%lld out of range [1, 2^30]", (long long)m);
    CHECK_SHAPE(k >= 256 && k <= kMaxK && k % 256 == 0, "k=%lld must be a positive multiple of 256", (long long)k);
    return MQ_OK;
}

bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) return false;
    return st != hipStreamCaptureStatusNone;
}

// Device workspaces for the split-k partials of the 4-bit GEMVs: one per
// (device, stream), so that calls on different streams never share partials
// (calls on one stream are ordered by it).  A workspace only grows, and the
// buffer it outgrows is kept until mq_workspace_release: a call already
// enqueued, or a graph captured earlier, may still be using it.
struct Workspace {
    int dev;
    hipStream_t stream;
    void* ptr;
    size_t bytes;
};
std::mutex g_ws_mu;
std::vector<Workspace> g_ws;
std::vector<Workspace> g_ws_retired;

int workspace(size_t need, hipStream_t stream, void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(MQ_ERR_HIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_ws_mu);
    Workspace* ws = nullptr;
    for (Workspace& w : g_ws)
        if (w.dev == dev && w.stream == stream) ws = &w;
    if (ws && ws->bytes >= need) {
        *out = ws->ptr;
        return MQ_OK;
    }
    if (capturing(stream))
        return fail(MQ_ERR_CAPTURE, "the split-k workspace of this stream must grow to %zu bytes while the stream "
                    "is captured; call once outside capture first", need);
    size_t b = (size_t)1 << 20;
    while (b < need) b <<= 1;
    void* p = nullptr;
    if (hipMalloc(&p, b) != hipSuccess) {
        (void)hipGetLastError();
        return fail(MQ_ERR_NOMEM, "hipMalloc(%zu) for the split-k workspace failed", b);
    }
    if (ws) {
        g_ws_retired.push_back(*ws);
        ws->ptr = p;
        ws->bytes = b;
    } else {
        g_ws.push_back(Workspace{dev, stream, p, b});
    }
    *out = p;
    return MQ_OK;
}

// Chooses full staging or split-k for a 4-bit GEMV with ncols columns
// (the debug dump runs with full staging only).
// Which kernel family a batched q4_K GEMV takes.  The matrix cores' cost
// hardly grows with n, the vector kernels' does, and the crossover moves
// to fewer columns as the matrix grows, and to fewer still where the
// vector kernels must split k (their n columns do not fit in 64 KB of
// staging).  Measured on MI355X, cold, launches alternating between the two
// paths (weight bytes -> first n where the matrix cores are faster):
// 0.7-5.6 MB (the 0.5B shapes) none up to n = 8; 7.2 MB (7B O) n = 8;
// 9.3-16.5 MB (7B QKV and 12.4, 16.5 MB matrices) n = 7; 19 MB with
// K = 18944 (split k from n = 3) n = 6; 33 and 38 MB of short rows n = 5-6;
// 38 MB with K = 18944 (the 7B down projection) n = 4; 76 MB (7B gate/up)
// n = 4.  q4_0, the debug dump and matrices beyond the matrix-core kernel's
// 32-bit offsets (mfma_rows_fit) take the vector kernels.
int mfma_min_cols(int64_t m, int64_t k) {
    constexpr int64_t MB = 1000 * 1000;
    const int64_t bytes = m * (k / 256) * kQ4KBytes;
    auto splits_at = [&](int n) { return n * stage_bytes((int)(k / 32)) > kMaxStageLds; };
    if (bytes < 6 * MB) return 9;                 // never
    if (bytes < 8 * MB) return 8;
    if (bytes < 24 * MB) return splits_at(6) ? 6 : 7;
    if (bytes < 60 * MB) return splits_at(4) ? 4 : 6;
    return 4;
}

bool use_mfma(int fmt, int ncols, int64_t m, int64_t k) {
    return fmt == kFmtQ4K && ncols >= mfma_min_cols(m, k) && mfma_rows_fit(m, k);
}

int run_q4k_mfma(const void* w, const void* xq, int64_t col_bytes, float* y, int64_t m, int64_t k, int ncols,
                 hipStream_t stream) {
    void* ws = nullptr;
    const int64_t need = gemv_q4k_mfma_partial_bytes(m, k, ncols);
    if (need > 0) {
        const int rc = workspace((size_t)need, stream, &ws);
        if (rc != MQ_OK) return rc;
    }
    return hip_status(launch_gemv_q4k_mfma(w, xq, col_bytes, y, (double*)ws, m, k, ncols, stream),
                      "matrix-core GEMV launch");
}

int run_q4(int fmt, const void* w, const void* xq, int64_t col_bytes, float* y, int32_t* isum, int32_t* ysum,
           int64_t m, int64_t k, int ncols, hipStream_t stream) {
    if (!isum && use_mfma(fmt, ncols, m, k)) return run_q4k_mfma(w, xq, col_bytes, y, m, k, ncols, stream);
    const int lds = ncols * stage_bytes((int)(k / 32));
    if (lds <= kMaxStageLds)
        return hip_status(launch_gemv_q4k(w, xq, col_bytes, y, isum, ysum, m, k, ncols, stream, fmt),
                          "4-bit GEMV launch");
    if (isum) return fail(MQ_ERR_SHAPE, "k too large for the dump kernel");
    if (ncols * kStageGroupBytes > kMaxStageLds) return fail(MQ_ERR_SHAPE, "too many columns");
    void* ws = nullptr;
    const size_t need = (size_t)gemv_q4k_splitk_nsplit(k) * (size_t)m * ncols * sizeof(double);
    int rc = workspace(need, stream, &ws);
    if (rc != MQ_OK) return rc;
    return hip_status(launch_gemv_q4k_splitk(w, xq, col_bytes, y, (double*)ws, m, k, ncols, stream, fmt),
                      "4-bit split-k GEMV launch");
}

int run_q4k(const void* w, const void* xq, int64_t col_bytes, float* y, int64_t m, int64_t k, int ncols,
            hipStream_t stream) {
    return run_q4(kFmtQ4K, w, xq, col_bytes, y, nullptr, nullptr, m, k, ncols, stream);
}

// The no-allocation batched entry point keeps its split-k partials in this
// fixed array instead of a workspace: every GPU the library runs on holds
// one copy of it until the process ends, and every call on that GPU shares
// it.  In host code `scratch` names a host-side stand-in, not device
// memory: its device address is looked up per device (hipGetSymbolAddress,
// with that device current) and only that address is ever passed on.
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) double scratch[kScratchBytes / sizeof(double)];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

// The current device's address of `scratch`, looked up on the first call
// on each device.
int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(MQ_ERR_HIP, "hipGetDevice failed");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(MQ_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MQ_OK;
}

}  // namespace

// ------------------------------------------------------------------ chains ----

struct mq_chain {
    int kind = 0;                     // 0: decode step, 1: routed-expert token
    std::vector<std::function<hipError_t(hipStream_t)>> ops;
    std::vector<void*> allocs;
    int64_t* step = nullptr;
    int64_t* cur = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    int captured = 0;
    int n_nodes = 0;
    uint8_t* q8_trace = nullptr;
    float* f32_trace = nullptr;
    int64_t q8_bytes = 0, f32_count = 0;
    const float* logits = nullptr;    // decode step: device f32 [vocab]
    int64_t vocab = 0;
    float* host_logits = nullptr;     // MQ_HOST_LOGITS: pinned f32 [vocab], written by the step's last node
    bool lazy = false;                // MQ_LAZY_CAPTURE: capture on the third MQ_GRAPH step
    int32_t* ids_next = nullptr;      // expert chain: routing ids of token (*step mod n_tokens)
    double* gu_part = nullptr;        // decode step: row sums of the split gate/up blocks' halves
    unsigned* gu_cnt = nullptr;       // decode step: one hand-over counter per split gate/up block
    int gu_split = 0;                 // number of split gate/up blocks
    uint64_t* stamps = nullptr;       // MQ_SPAN_STAMPS: [first-wave start, last-wave end] per GEMV kernel
    int n_stamped = 0;                // number of stamped kernels (4 per layer + the lm_head)
    const int32_t* ids_table = nullptr;
    int n_tokens = 0, n_sel = 0;
    bool capture_tried = false;
    int64_t graph_steps = 0;
    double capture_ms = 0.0;
};

namespace {

void* chain_alloc(mq_chain* c, size_t bytes, int* rc) {
    void* p = nullptr;
    if (hipMalloc(&p, bytes < 256 ? 256 : bytes) != hipSuccess) {
        *rc = fail(MQ_ERR_NOMEM, "hipMalloc(%zu) for a chain buffer failed", bytes);
        return nullptr;
    }
    c->allocs.push_back(p);
    return p;
}

// Stamp pairs per kernel: one per wave slot (SpanStamp).
constexpr int kStampPairs = kStampSlots * kStampWaves;

__global__ void k_stamp_clear(uint64_t* __restrict__ p, int64_t n_pairs) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_pairs; i += (int64_t)gridDim.x * blockDim.x) {
        p[2 * i] = ~(uint64_t)0;
        p[2 * i + 1] = 0;
    }
}

// Every stamp pair starts as [max, 0], the mark of a slot that no wave has
// written (a kernel's grid may use fewer slots than it has), so that the
// host's min / max reduction in mq_chain_read_stamps skips it.
int reset_stamps(mq_chain* c) {
    std::vector<uint64_t> init((size_t)c->n_stamped * kStampPairs * 2);
    for (size_t i = 0; i < init.size(); i += 2) {
        init[i] = ~(uint64_t)0;
        init[i + 1] = 0;
    }
    return hip_status(hipMemcpy(c->stamps, init.data(), init.size() * sizeof(uint64_t), hipMemcpyHostToDevice),
                      "span stamp reset");
}

void chain_free(mq_chain* c) {
    if (c->exec) (void)hipGraphExecDestroy(c->exec);
    if (c->graph) (void)hipGraphDestroy(c->graph);
    for (void* p : c->allocs) (void)hipFree(p);
    if (c->host_logits) (void)hipHostFree(c->host_logits);
    delete c;
}

// MQ_HOST_LOGITS: pins the chain's host copy of the logits and appends the
// copy to the step.  Failure to pin leaves the chain without it (one
// warning per process).
void add_host_logits(mq_chain* c) {
    static std::atomic<bool> warned{false};
    void* p = nullptr;
    const size_t bytes = (size_t)c->vocab * sizeof(float);
    const hipError_t e = (g_fault & MQ_FAULT_PINNED_ALLOC) ? hipErrorOutOfMemory
                                                          : hipHostMalloc(&p, bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        if (!warned.exchange(true)) {
            fprintf(stderr, "mq: pinning the %zu-byte host logits of a chain failed (%s); the chain has no host copy\n",
                    bytes, hipGetErrorString(e));
        }
        return;
    }
    c->host_logits = (float*)p;
    float* host = c->host_logits;
    const float* dev = c->logits;
    c->ops.push_back([=](hipStream_t s) { return hipMemcpyAsync(host, dev, bytes, hipMemcpyDeviceToHost, s); });
}

int enqueue(mq_chain* c, hipStream_t s) {
    for (auto& op : c->ops) {
        hipError_t e = op(s);
        if (e != hipSuccess) return hip_status(e, "chain kernel launch");
    }
    return ok();
}

// Warm run, counter reset, then capture; failure to capture leaves an eager chain.
// Sets the step counter; the expert chain's next-token ids follow it.
hipError_t set_step(mq_chain* c, int64_t step, hipStream_t stream) {
    hipError_t e = launch_set_i64(c->step, step, stream);
    if (e == hipSuccess && c->gu_cnt) e = launch_zero_u32(c->gu_cnt, c->gu_split, stream);
    if (e == hipSuccess && c->ids_next)
        e = launch_moe_prime(c->step, c->n_tokens, c->ids_table, c->n_sel, c->ids_next, stream);
    return e;
}

int zero_counters(mq_chain* c, hipStream_t stream) {
    hipError_t e = set_step(c, 0, stream);
    if (e == hipSuccess && c->cur) e = launch_set_i64(c->cur, 0, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    return hip_status(e, "counter reset");
}

// Records the chain's kernels on a private stream (nothing runs) and
// instantiates the graph.  Failure leaves an eager chain and logs once.
void try_capture(mq_chain* c) {
    c->capture_tried = true;
    const auto t0 = std::chrono::steady_clock::now();
    const char* why = nullptr;
    hipStream_t cs = nullptr;
    if (g_fault & MQ_FAULT_CAPTURE) {
        why = "capture failure injected by mq_test_set_fault";
    } else if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) {
        why = "hipStreamCreateWithFlags failed";
        cs = nullptr;
    } else if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
        why = "hipStreamBeginCapture failed";
    } else {
        bool launched = true;
        for (auto& op : c->ops)
            if (op(cs) != hipSuccess) { launched = false; break; }
        hipGraph_t g = nullptr;
        const hipError_t ee = hipStreamEndCapture(cs, &g);
        if (!launched || ee != hipSuccess || !g) {
            why = "a launch failed during capture";
            if (g) (void)hipGraphDestroy(g);
        } else if (hipGraphInstantiate(&c->exec, g, nullptr, nullptr, 0) != hipSuccess) {
            why = "hipGraphInstantiate failed";
            (void)hipGraphDestroy(g);
            c->exec = nullptr;
        } else {
            size_t n = 0;
            (void)hipGraphGetNodes(g, nullptr, &n);
            c->graph = g;
            c->n_nodes = (int)n;
            c->captured = 1;
        }
    }
    if (cs) (void)hipStreamDestroy(cs);
    (void)hipGetLastError();
    c->capture_ms = std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    if (!c->captured)
        fprintf(stderr, "mq: decode-step graph capture failed (%s); this chain runs eagerly\n", why);
}

// Creation's last stage.  Eager-only chains and eager-capture chains run
// one warm step (first launches load code objects and set kernel
// attributes, which must not happen inside a capture) and reset the
// counters; eager-capture chains then capture.  Lazy chains only reset the
// counters: their first two steps run eagerly and warm them.
int chain_finish(mq_chain* c, hipStream_t stream, unsigned flags) {
    const bool eager_only = (flags & MQ_EAGER_ONLY) != 0;
    c->lazy = !eager_only && (flags & MQ_LAZY_CAPTURE) != 0;
    int rc = zero_counters(c, stream);
    if (rc != MQ_OK || c->lazy) return rc;
    if ((rc = enqueue(c, stream)) != MQ_OK) return rc;
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_status(e, "chain warm-up step");
    if ((rc = zero_counters(c, stream)) != MQ_OK) return rc;
    if (!eager_only) try_capture(c);
    return ok();
}

// The process-wide pinned staging buffer of mq_read_to_host.
struct PinnedReadback {
    std::mutex mu;
    void* buf = nullptr;
    size_t bytes = 0;
    int64_t pinned_reads = 0, pageable_reads = 0;
    bool warned = false;
};
PinnedReadback g_rb;
constexpr size_t kReadbackMinBytes = (size_t)4 << 20;

// Makes g_rb.buf hold at least `bytes`; false if pinning failed (warned once).
bool readback_reserve(size_t bytes) {
    if (g_rb.buf && g_rb.bytes >= bytes) return true;
    if (g_rb.buf) (void)hipHostFree(g_rb.buf);
    g_rb.buf = nullptr;
    g_rb.bytes = 0;
    const size_t want = std::max(bytes, kReadbackMinBytes);
    void* p = nullptr;
    const hipError_t e = (g_fault & MQ_FAULT_PINNED_ALLOC) ? hipErrorOutOfMemory
                                                          : hipHostMalloc(&p, want, hipHostMallocDefault);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        if (!g_rb.warned) {
            g_rb.warned = true;
            fprintf(stderr, "mq: pinning a %zu-byte readback buffer failed (%s); reading back through pageable memory\n",
                    want, hipGetErrorString(e));
        }
        return false;
    }
    g_rb.buf = p;
    g_rb.bytes = want;
    return true;
}

}  // namespace

// ------------------------------------------------------------------- C ABI ----

extern "C" {

const char* mq_last_error(void) { return g_err.c_str(); }
const char* mq_version(void) { return "libmq 0.2 (gfx950)"; }

int mq_time_next_launches(const hipEvent_t* starts, const hipEvent_t* stops, int n) {
    CHECK_ARG(n >= 0 && n <= 65536, "n=%d out of range", n);
    CHECK_ARG(n == 0 || (starts && stops), "null event arrays");
    set_next_launch_events(starts, stops, n);
    return ok();
}

int mq_probe_stream_read(const void* p, int64_t bytes, uint32_t* xor_out, int workgroups, hipStream_t stream) {
    CHECK_ARG(xor_out && (p || bytes == 0), "null pointer (p=%p xor_out=%p)", p, (void*)xor_out);
    CHECK_ARG(aligned(p, 16) && aligned(xor_out, 4), "p must be 16-byte aligned, xor_out 4-byte aligned");
    CHECK_ARG(bytes >= 0 && bytes % 16 == 0, "bytes=%lld must be a non-negative multiple of 16", (long long)bytes);
    CHECK_ARG(workgroups <= 65536, "workgroups=%d out of range", workgroups);
    return hip_status(launch_stream_read(p, bytes, xor_out, workgroups, stream), "stream probe launch");
}

int mq_probe_grid_barrier(int hierarchical, int exchange_words, int rounds, int threads, double* us_per_round,
                          uint32_t* bad_words, hipStream_t stream) {
    CHECK_ARG(us_per_round && bad_words, "null output pointer");
    CHECK_ARG(hierarchical == 0 || hierarchical == 1, "hierarchical must be 0 or 1");
    CHECK_ARG(exchange_words >= 0 && exchange_words <= 4096, "exchange_words=%d out of range [0, 4096]", exchange_words);
    CHECK_ARG(rounds >= 1 && rounds <= 100000, "rounds=%d out of range [1, 100000]", rounds);
    CHECK_ARG(threads >= 64 && threads <= 1024 && threads % 64 == 0, "threads=%d must be a multiple of 64 in [64, 1024]",
              threads);
    if (capturing(stream)) return fail(MQ_ERR_CAPTURE, "the barrier probe cannot run inside a stream capture");
    int limit_hit = 0;
    const int rc = grid_barrier_probe(hierarchical, exchange_words, rounds, threads, us_per_round, bad_words,
                                      &limit_hit, stream);
    if (rc == 1) return fail(MQ_ERR_SHAPE, "a grid of one %d-thread workgroup per CU cannot be co-resident", threads);
    if (rc != 0) return fail(MQ_ERR_HIP, "barrier probe: a HIP call failed");
    if (limit_hit) return fail(MQ_ERR_HIP, "barrier probe: a wait ran out of polls");
    return ok();
}

int mq_probe_graph_boundary(int n_kernels, int threads, int reps, double* us_per_kernel) {
    CHECK_ARG(us_per_kernel, "null output pointer");
    CHECK_ARG(n_kernels >= 1 && n_kernels <= 4096, "n_kernels=%d out of range [1, 4096]", n_kernels);
    CHECK_ARG(reps >= 1 && reps <= 10000, "reps=%d out of range [1, 10000]", reps);
    CHECK_ARG(threads >= 64 && threads <= 1024 && threads % 64 == 0, "threads=%d must be a multiple of 64 in [64, 1024]",
              threads);
    if (graph_boundary_probe(n_kernels, threads, reps, us_per_kernel) != 0)
        return fail(MQ_ERR_HIP, "graph boundary probe: a HIP call failed");
    return ok();
}

int mq_read_to_host(const void* src, void* host_dst, int64_t bytes, unsigned flags, hipStream_t stream) {
    CHECK_ARG((flags & ~(unsigned)MQ_READ_PAGEABLE) == 0, "unknown flags %#x", flags);
    CHECK_ARG(bytes >= 0, "bytes=%lld must be >= 0", (long long)bytes);
    CHECK_ARG(bytes == 0 || (src && host_dst), "null pointer (src=%p host_dst=%p)", src, host_dst);
    if (capturing(stream)) return fail(MQ_ERR_CAPTURE, "a blocking readback cannot run inside a stream capture");
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_status(e, "waiting for the stream before the readback");
    if (bytes == 0) return ok();
    std::lock_guard<std::mutex> lock(g_rb.mu);
    if (!(flags & MQ_READ_PAGEABLE) && readback_reserve((size_t)bytes)) {
        e = hipMemcpyAsync(g_rb.buf, src, (size_t)bytes, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_status(e, "pinned readback copy");
        memcpy(host_dst, g_rb.buf, (size_t)bytes);
        ++g_rb.pinned_reads;
        return ok();
    }
    e = hipMemcpyAsync(host_dst, src, (size_t)bytes, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_status(e, "pageable readback copy");
    ++g_rb.pageable_reads;
    return ok();
}

int mq_readback_stats(int64_t* pinned_bytes, int64_t* pinned_reads, int64_t* pageable_reads, int* warned) {
    std::lock_guard<std::mutex> lock(g_rb.mu);
    if (pinned_bytes) *pinned_bytes = (int64_t)g_rb.bytes;
    if (pinned_reads) *pinned_reads = g_rb.pinned_reads;
    if (pageable_reads) *pageable_reads = g_rb.pageable_reads;
    if (warned) *warned = g_rb.warned ? 1 : 0;
    return ok();
}

int mq_readback_release(void) {
    std::lock_guard<std::mutex> lock(g_rb.mu);
    hipError_t e = hipSuccess;
    if (g_rb.buf) e = hipHostFree(g_rb.buf);
    g_rb.buf = nullptr;
    g_rb.bytes = 0;
    return hip_status(e, "freeing the pinned readback buffer");
}

int mq_workspace_release(void) {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    if (g_ws.empty() && g_ws_retired.empty()) return ok();
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return fail(MQ_ERR_HIP, "hipGetDevice failed");
    hipError_t first = hipSuccess;
    auto free_all = [&](std::vector<Workspace>& v) {
        for (const Workspace& w : v) {
            hipError_t e = hipSetDevice(w.dev);
            if (e == hipSuccess) e = hipDeviceSynchronize();
            if (e == hipSuccess) e = hipFree(w.ptr);
            if (first == hipSuccess) first = e;
        }
        v.clear();
    };
    free_all(g_ws);
    free_all(g_ws_retired);
    (void)hipSetDevice(cur);
    return hip_status(first, "freeing the split-k workspaces");
}

int mq_workspace_stats(int64_t* bytes, int* n_streams, int* n_retired) {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    int64_t total = 0;
    for (const Workspace& w : g_ws) total += (int64_t)w.bytes;
    for (const Workspace& w : g_ws_retired) total += (int64_t)w.bytes;
    if (bytes) *bytes = total;
    if (n_streams) *n_streams = (int)g_ws.size();
    if (n_retired) *n_retired = (int)g_ws_retired.size();
    return ok();
}

int mq_test_set_fault(unsigned fault_mask) {
    g_fault = fault_mask;
    return ok();
}

int mq_quantize_q8_0(const float* x, void* xq, int64_t k, int n_cols, hipStream_t stream) {
    CHECK_ARG(x && xq, "null pointer");
    CHECK_ARG(aligned(x, 4) && aligned(xq, 2), "x must be 4-byte and xq 2-byte aligned");
    CHECK_SHAPE(k >= 32 && k <= kMaxK && k % 32 == 0, "k=%lld must be a positive multiple of 32", (long long)k);
    CHECK_SHAPE(n_cols >= 1 && (int64_t)n_cols * k <= ((int64_t)1 << 32), "n_cols=%d out of range", n_cols);
    return hip_status(launch_quantize_q8_0(x, xq, k, n_cols, stream), "quantize launch");
}

int mq_gemv_q4k_q8(const void* w, const void* xq, float* y, int64_t m, int64_t k, hipStream_t stream) {
    int rc = check_q4k(w, xq, y, m, k);
    if (rc != MQ_OK) return rc;
    return run_q4k(w, xq, 0, y, m, k, 1, stream);
}

int mq_gemv_q4k_q8_batched(const void* w, const void* xq, float* y, int64_t m, int64_t k, int n,
                           hipStream_t stream) {
    int rc = check_q4k(w, xq, y, m, k);
    if (rc != MQ_OK) return rc;
    CHECK_SHAPE(n >= 1 && n <= 8, "n=%d must be in 1..8", n);
    return run_q4k(w, xq, (k / 32) * kQ8Bytes, y, m, k, n, stream);
}

int mq_gemv_q4k_q8_batched_noalloc(const void* w, const void* xq, float* y, int64_t m, int64_t k, int n,
                                   hipStream_t stream) {
    int rc = check_q4k(w, xq, y, m, k);
    if (rc != MQ_OK) return rc;
    CHECK_SHAPE(n >= 1 && n <= 8, "n=%d must be in 1..8", n);
    const int64_t col_bytes = (k / 32) * kQ8Bytes;
    if (use_mfma(kFmtQ4K, n, m, k)) {
        const size_t need = (size_t)gemv_q4k_mfma_partial_bytes(m, k, n);
        CHECK_SHAPE(need <= kScratchBytes, "m=%lld, k=%lld, n=%d need %zu bytes of split-k partials; the fixed "
                    "scratch of the no-allocation entry point holds %zu", (long long)m, (long long)k, n, need,
                    kScratchBytes);
        void* part = nullptr;
        if (need > 0 && (rc = scratch_address(&part)) != MQ_OK) return rc;
        return hip_status(launch_gemv_q4k_mfma(w, xq, col_bytes, y, (double*)part, m, k, n, stream),
                          "matrix-core GEMV launch");
    }
    if (n * stage_bytes((int)(k / 32)) <= kMaxStageLds)       // one pass over k: no partials
        return hip_status(launch_gemv_q4k(w, xq, col_bytes, y, nullptr, nullptr, m, k, n, stream, kFmtQ4K),
                          "4-bit GEMV launch");
    const size_t need = (size_t)gemv_q4k_splitk_nsplit(k) * (size_t)m * (size_t)n * sizeof(double);
    CHECK_SHAPE(need <= kScratchBytes, "m=%lld, k=%lld, n=%d need %zu bytes of split-k partials; the fixed "
                "scratch of the no-allocation entry point holds %zu", (long long)m, (long long)k, n, need,
                kScratchBytes);
    void* part = nullptr;
    if ((rc = scratch_address(&part)) != MQ_OK) return rc;
    return hip_status(launch_gemv_q4k_splitk(w, xq, col_bytes, y, (double*)part, m, k, n, stream, kFmtQ4K),
                      "4-bit split-k GEMV launch");
}

int mq_gemv_batched_path(int64_t m, int64_t k, int n, int weight_format, int* path) {
    CHECK_ARG(path, "null path");
    CHECK_ARG(weight_format == MQ_FMT_Q4_K || weight_format == MQ_FMT_Q4_0, "unknown weight_format %d", weight_format);
    CHECK_SHAPE(m >= 1 && m <= kMaxRows, "m=%lld out of range", (long long)m);
    CHECK_SHAPE(k >= 256 && k % 256 == 0 && k <= kMaxK, "k=%lld must be a positive multiple of 256", (long long)k);
    CHECK_SHAPE(n >= 1 && n <= 8, "n=%d must be in 1..8", n);
    *path = use_mfma(weight_format == MQ_FMT_Q4_0 ? kFmtQ4_0 : kFmtQ4K, n, m, k) ? 1 : 0;
    return ok();
}

int mq_debug_gemv_q4k_batched_path(const void* w, const void* xq, float* y, int64_t m, int64_t k, int n, int path,
                                   hipStream_t stream) {
    int rc = check_q4k(w, xq, y, m, k);
    if (rc != MQ_OK) return rc;
    CHECK_SHAPE(n >= 1 && n <= 8, "n=%d must be in 1..8", n);
    CHECK_ARG(path == 0 || path == 1, "path must be 0 (vector kernels) or 1 (matrix cores)");
    CHECK_SHAPE(path == 0 || n >= 2, "the matrix-core path takes n >= 2");
    CHECK_SHAPE(path == 0 || mfma_rows_fit(m, k), "m=%lld rows of k=%lld exceed the matrix-core path's 32-bit offsets",
                (long long)m, (long long)k);
    const int64_t col_bytes = (k / 32) * kQ8Bytes;
    if (path == 1) return run_q4k_mfma(w, xq, col_bytes, y, m, k, n, stream);
    const int lds = n * stage_bytes((int)(k / 32));
    if (lds <= kMaxStageLds)
        return hip_status(launch_gemv_q4k(w, xq, col_bytes, y, nullptr, nullptr, m, k, n, stream, kFmtQ4K),
                          "4-bit GEMV launch");
    void* ws = nullptr;
    const size_t need = (size_t)gemv_q4k_splitk_nsplit(k) * (size_t)m * n * sizeof(double);
    if ((rc = workspace(need, stream, &ws)) != MQ_OK) return rc;
    return hip_status(launch_gemv_q4k_splitk(w, xq, col_bytes, y, (double*)ws, m, k, n, stream, kFmtQ4K),
                      "4-bit split-k GEMV launch");
}

int mq_gemv_q4_0_q8(const void* w, const void* xq, float* y, int64_t m, int64_t k, hipStream_t stream) {
    int rc = check_q4k(w, xq, y, m, k);
    if (rc != MQ_OK) return rc;
    return run_q4(kFmtQ4_0, w, xq, 0, y, nullptr, nullptr, m, k, 1, stream);
}

int mq_gemv_q4_0_q8_batched(const void* w, const void* xq, float* y, int64_t m, int64_t k, int n,
                            hipStream_t stream) {
    int rc = check_q4k(w, xq, y, m, k);
    if (rc != MQ_OK) return rc;
    CHECK_SHAPE(n >= 1 && n <= 8, "n=%d must be in 1..8", n);
    return run_q4(kFmtQ4_0, w, xq, (k / 32) * kQ8Bytes, y, nullptr, nullptr, m, k, n, stream);
}

int mq_debug_gemv_q4_0_q8_isums(const void* w, const void* xq, float* y, int32_t* isum, int32_t* ysum,
                                int64_t m, int64_t k, hipStream_t stream) {
    int rc = check_q4k(w, xq, y, m, k);
    if (rc != MQ_OK) return rc;
    CHECK_ARG(isum && aligned(isum, 4), "isum must be a non-null int32 buffer");
    return run_q4(kFmtQ4_0, w, xq, 0, y, isum, ysum, m, k, 1, stream);
}

int mq_gemv_q4k_grouped(const void* w_all, int64_t expert_bytes, int n_experts, const int32_t* ids,
                        int n_sel, const void* xq, int64_t xq_stride_bytes, float* y,
                        const float* combine, float* y_out, int64_t m, int64_t k, hipStream_t stream) {
    CHECK_ARG(w_all && ids && xq, "null pointer");
    CHECK_ARG(y || combine, "need y, combine or both");
    CHECK_ARG(!combine || y_out, "combine needs y_out");
    CHECK_ARG(aligned(w_all, 16) && aligned(xq, 2) && aligned(ids, 4), "misaligned pointer");
    CHECK_ARG(expert_bytes % 16 == 0, "expert_bytes must be a multiple of 16");
    CHECK_ARG(xq_stride_bytes >= 0 && xq_stride_bytes % 2 == 0, "bad xq_stride_bytes");
    CHECK_SHAPE(m >= 1 && m <= kMaxRows, "m out of range");
    CHECK_SHAPE(k >= 256 && k <= kMaxK && k % 256 == 0, "k must be a positive multiple of 256");
    CHECK_SHAPE(n_sel >= 1 && n_sel <= 16, "n_sel=%d must be in 1..16", n_sel);
    CHECK_SHAPE(n_experts >= 1, "n_experts must be >= 1");
    CHECK_SHAPE(expert_bytes >= m * (k / 256) * kQ4KBytes, "expert_bytes smaller than one expert matrix");
    CHECK_SHAPE(xq_stride_bytes == 0 || xq_stride_bytes >= (k / 32) * kQ8Bytes, "xq_stride_bytes too small");
    const int lds = (xq_stride_bytes ? n_sel : 1) * stage_bytes((int)(k / 32));
    CHECK_SHAPE(lds <= kMaxStageLds, "activations need %d bytes of LDS (max %d)", lds, kMaxStageLds);
    return hip_status(launch_gemv_q4k_grouped(w_all, expert_bytes, n_experts, ids, n_sel, xq, xq_stride_bytes,
                                              y, combine, y_out, nullptr, 1, m, k, nullptr, stream),
                      "grouped GEMV launch");
}

int mq_gemv_q8_0_q8(const void* w, const void* xq, float* y, int64_t m, int64_t k, hipStream_t stream) {
    CHECK_ARG(w && xq && y, "null pointer");
    CHECK_ARG(aligned(w, 4) && aligned(xq, 2) && aligned(y, 4), "misaligned pointer");
    CHECK_SHAPE(m >= 1 && m <= kMaxRows, "m out of range");
    CHECK_SHAPE(k >= 64 && k % 64 == 0 && stage_bytes((int)(k / 32)) <= kMaxStageLds,
                "k=%lld must be a positive multiple of 64 (and at most ~43k)", (long long)k);
    return hip_status(launch_gemv_q8_0(w, xq, y, nullptr, m, k, stream), "q8_0 GEMV launch");
}

int mq_rmsnorm_quantize_q8_0(const float* x, void* xq, int64_t k, float eps, hipStream_t stream) {
    CHECK_ARG(x && xq && aligned(x, 4) && aligned(xq, 2), "null or misaligned pointer");
    CHECK_SHAPE(k >= 32 && k % 32 == 0 && k <= kMaxK, "k must be a positive multiple of 32");
    CHECK_ARG(eps >= 0.0f, "eps must be >= 0");
    return hip_status(launch_rmsnorm_quantize(x, xq, k, eps, nullptr, 1, nullptr, stream), "rmsnorm launch");
}

int mq_swiglu_quantize_q8_0(const float* gu, void* xq, int64_t inter, int n_cols, int64_t k_pad,
                            hipStream_t stream) {
    CHECK_ARG(gu && xq && aligned(gu, 4) && aligned(xq, 2), "null or misaligned pointer");
    CHECK_SHAPE(inter >= 32 && inter % 32 == 0 && inter <= kMaxK, "inter must be a positive multiple of 32");
    CHECK_SHAPE(k_pad >= inter && k_pad % 32 == 0 && k_pad <= kMaxK, "k_pad must be >= inter and a multiple of 32");
    CHECK_SHAPE(n_cols >= 1 && n_cols <= 4096, "n_cols out of range");
    return hip_status(launch_swiglu_quantize(gu, xq, inter, n_cols, k_pad, stream), "swiglu launch");
}

int mq_debug_gemv_q4k_q8_isums(const void* w, const void* xq, float* y, int32_t* isum, int32_t* ysum,
                               int64_t m, int64_t k, hipStream_t stream) {
    int rc = check_q4k(w, xq, y, m, k);
    if (rc != MQ_OK) return rc;
    CHECK_ARG(isum && aligned(isum, 4), "isum must be a non-null int32 buffer");
    CHECK_SHAPE(stage_bytes((int)(k / 32)) <= kMaxStageLds, "k too large for the dump kernel");
    return hip_status(launch_gemv_q4k(w, xq, 0, y, isum, ysum, m, k, 1, stream), "dump GEMV launch");
}

int mq_debug_gemv_q8_0_q8_isums(const void* w, const void* xq, float* y, int32_t* isum, int64_t m,
                                int64_t k, hipStream_t stream) {
    CHECK_ARG(w && xq && y && isum, "null pointer");
    CHECK_ARG(aligned(w, 4) && aligned(xq, 2) && aligned(y, 4) && aligned(isum, 4), "misaligned pointer");
    CHECK_SHAPE(m >= 1 && m <= kMaxRows, "m out of range");
    CHECK_SHAPE(k >= 64 && k % 64 == 0 && stage_bytes((int)(k / 32)) <= kMaxStageLds, "bad k");
    return hip_status(launch_gemv_q8_0(w, xq, y, isum, m, k, stream), "dump GEMV launch");
}

int mq_debug_gate_up_swiglu(const void* w, const float* x, float eps, float* gu_out, void* g_q8, int64_t inter,
                            int64_t k, int n_split, double* part, unsigned* cnt, int weight_format,
                            hipStream_t stream) {
    CHECK_ARG(w && x && g_q8, "null pointer");
    CHECK_ARG(aligned(w, 16) && aligned(x, 16) && aligned(g_q8, 2) && aligned(gu_out, 4), "misaligned pointer");
    CHECK_ARG(weight_format == MQ_FMT_Q4_K || weight_format == MQ_FMT_Q4_0, "unknown weight_format %d",
              weight_format);
    CHECK_ARG(n_split >= 0, "n_split must be >= 0");
    CHECK_SHAPE(inter >= 32 && inter % 32 == 0 && 2 * inter <= kMaxRows, "inter must be a positive multiple of 32");
    CHECK_SHAPE(k >= 256 && k % 256 == 0 && stage_bytes((int)(k / 32)) <= kMaxStageLds,
                "k must be a positive multiple of 256 that fits in LDS");
    CHECK_SHAPE(2 * inter <= max_rows_per_launch(k), "a matrix of 4 GiB or more");
    CHECK_ARG(eps >= 0.0f, "eps must be >= 0");
    const NormIn nin{x, nullptr, 1, eps, nullptr, nullptr, 0};
    const int fmt = weight_format == MQ_FMT_Q4_0 ? kFmtQ4_0 : kFmtQ4K;
    return hip_status(launch_gemv_q4k_swiglu(w, nullptr, &nin, gu_out, g_q8, inter, k, stream, fmt, part, cnt,
                                             n_split),
                      "gate/up launch");
}

int mq_chain_create(const mq_chain_desc* d, hipStream_t stream, mq_chain** out) {
    CHECK_ARG(d && out, "null desc or out");
    *out = nullptr;
    CHECK_SHAPE(d->n_layers >= 1 && d->n_layers <= 4096, "n_layers out of range");
    CHECK_SHAPE(d->hidden >= 256 && d->hidden % 256 == 0 && d->hidden <= kMaxK, "hidden must be a multiple of 256");
    CHECK_SHAPE(d->inter >= 256 && d->inter % 256 == 0 && d->inter <= kMaxK, "inter must be a multiple of 256");
    CHECK_SHAPE(d->o_k == 0 || (d->o_k >= 256 && d->o_k % 256 == 0 && d->o_k <= d->hidden),
                "o_k must be 0 or a multiple of 256 in [256, hidden]");
    const int64_t o_k = d->o_k ? d->o_k : d->hidden;
    CHECK_SHAPE(d->qkv_rows >= o_k && d->qkv_rows <= kMaxRows && d->qkv_rows % 4 == 0,
                "qkv_rows must be >= O's K (o_k, or hidden) and a multiple of 4");
    CHECK_SHAPE(d->vocab >= 1 && d->vocab <= kMaxRows, "vocab out of range");
    CHECK_SHAPE(stage_bytes((int)(d->inter / 32)) <= kMaxStageLds, "inter too large");
    CHECK_SHAPE(d->qkv_rows <= max_rows_per_launch(d->hidden) && 2 * d->inter <= max_rows_per_launch(d->hidden) &&
                    d->hidden <= max_rows_per_launch(d->inter),
                "a layer matrix of 4 GiB or more (the chain's kernels address each with 32-bit offsets)");
    CHECK_ARG(d->w_qkv && d->w_o && d->w_gu && d->w_down && d->w_lm && d->x_table && d->logits,
              "null pointer in the descriptor");
    CHECK_ARG(d->n_inputs >= 1, "n_inputs must be >= 1");
    CHECK_ARG(d->eps >= 0.0f, "eps must be >= 0");
    CHECK_ARG(d->weight_format == MQ_FMT_Q4_K || d->weight_format == MQ_FMT_Q4_0, "unknown weight_format %d",
              d->weight_format);
    CHECK_ARG(aligned(d->w_lm, 4) && aligned(d->x_table, 16) && aligned(d->logits, 4),
              "misaligned pointer (x_table must be 16-byte aligned)");
    for (int l = 0; l < d->n_layers; ++l)
        CHECK_ARG(d->w_qkv[l] && d->w_o[l] && d->w_gu[l] && d->w_down[l] && aligned(d->w_qkv[l], 16) &&
                      aligned(d->w_o[l], 16) && aligned(d->w_gu[l], 16) && aligned(d->w_down[l], 16),
                  "layer %d: null or misaligned weight pointer", l);
    if (capturing(stream)) return fail(MQ_ERR_CAPTURE, "mq_chain_create cannot run inside a stream capture");

    mq_chain* c = new mq_chain();
    c->kind = 0;
    c->logits = d->logits;
    c->vocab = d->vocab;
    const int L = d->n_layers;
    const int64_t H = d->hidden, I = d->inter, QKV = d->qkv_rows, KO = o_k;
    const int64_t qH = H / 32 * kQ8Bytes, qI = I / 32 * kQ8Bytes;
    const bool keep = (d->flags & MQ_KEEP_INTERMEDIATES) != 0;
    const int exact = (d->flags & MQ_EXACT_GLUE) != 0;
    const int fmt = d->weight_format == MQ_FMT_Q4_0 ? kFmtQ4_0 : kFmtQ4K;
    int rc = MQ_OK;
    c->step = (int64_t*)chain_alloc(c, sizeof(int64_t), &rc);
    // Q8 inputs of every GEMV and f32 outputs; with MQ_KEEP_INTERMEDIATES every
    // layer gets its own slice of the trace (same layout as the reference trace).
    const int64_t q8_layer = 3 * qH + qI, f32_layer = QKV + H + 2 * I + H;
    c->q8_bytes = L * q8_layer + qH;
    c->f32_count = L * f32_layer;
    const int64_t q8_alloc = keep ? c->q8_bytes : q8_layer + qH;
    const int64_t f32_alloc = keep ? c->f32_count : f32_layer;
    if (rc == MQ_OK) c->q8_trace = (uint8_t*)chain_alloc(c, q8_alloc, &rc);
    // O's input fills only o_k/32 blocks of its slot: the rest reads as zeros
    if (rc == MQ_OK && keep && KO < H && hipMemset(c->q8_trace, 0, q8_alloc) != hipSuccess)
        rc = fail(MQ_ERR_HIP, "clearing the q8_0 trace");
    if (rc == MQ_OK) c->f32_trace = (float*)chain_alloc(c, f32_alloc * sizeof(float), &rc);
    // gate/up blocks beyond a multiple of the CU count are split in two halves
    // along K (launch_gemv_q4k_swiglu), with this hand-over space
    const int gu_split = (d->flags & MQ_UNFUSED_GLUE) ? 0 : swiglu_split_blocks(I, H);
    if (rc == MQ_OK && gu_split > 0) {
        c->gu_part = (double*)chain_alloc(c, (size_t)gu_split * 128 * sizeof(double), &rc);
        if (rc == MQ_OK) c->gu_cnt = (unsigned*)chain_alloc(c, (size_t)gu_split * sizeof(unsigned), &rc);
        if (rc == MQ_OK) c->gu_split = gu_split;
    }
    const bool stamped = (d->flags & MQ_SPAN_STAMPS) != 0 && !(d->flags & MQ_UNFUSED_GLUE);
    if (rc == MQ_OK && stamped) {
        c->n_stamped = 4 * L + 1;
        c->stamps = (uint64_t*)chain_alloc(c, (size_t)c->n_stamped * kStampPairs * 2 * sizeof(uint64_t), &rc);
        if (rc == MQ_OK) rc = reset_stamps(c);
    }
    if (rc != MQ_OK) { chain_free(c); return rc; }

    const float eps = d->eps;
    int64_t* step = c->step;
    const float* x_table = d->x_table;
    const int n_inputs = d->n_inputs;
    // Per layer four kernels.  QKV, O and gate/up form their q8_0 input
    // Q8(RMSNorm(.)) in their own prologues; gate/up carries the SwiGLU->Q8
    // glue in its epilogue and down reads that.  The first kernel of the step
    // picks the input row with the device step counter; the lm_head kernel,
    // the last one, advances it.  The q8_0 vectors formed in prologues are
    // written out (by one workgroup) only when intermediates are kept.
    const float* h_prev = nullptr;
    if (d->flags & MQ_UNFUSED_GLUE) {
        // The unfused arm: glue kernels between plain q8_0-input GEMVs.
        for (int l = 0; l < L; ++l) {
            uint8_t* q8 = c->q8_trace + (keep ? l * q8_layer : 0);
            float* f = c->f32_trace + (keep ? l * f32_layer : 0);
            uint8_t *qa = q8, *qb = q8 + qH, *qc = q8 + 2 * qH, *qg = q8 + 3 * qH;
            float *t = f, *o = f + QKV, *gu = f + QKV + H, *h = f + QKV + H + 2 * I;
            const void *wq = d->w_qkv[l], *wo = d->w_o[l], *wg = d->w_gu[l], *wd = d->w_down[l];
            const float* xin = l == 0 ? x_table : h_prev;
            const int64_t* sel = l == 0 ? step : nullptr;
            const int nin = l == 0 ? n_inputs : 1;
            c->ops.push_back([=](hipStream_t s) { return launch_rmsnorm_quantize(xin, qa, H, eps, sel, nin, nullptr, s); });
            c->ops.push_back([=](hipStream_t s) { return launch_gemv_q4k(wq, qa, 0, t, nullptr, nullptr, QKV, H, 1, s, fmt); });
            c->ops.push_back([=](hipStream_t s) { return launch_rmsnorm_quantize(t, qb, KO, eps, nullptr, 1, nullptr, s); });
            c->ops.push_back([=](hipStream_t s) { return launch_gemv_q4k(wo, qb, 0, o, nullptr, nullptr, H, KO, 1, s, fmt); });
            c->ops.push_back([=](hipStream_t s) { return launch_rmsnorm_quantize(o, qc, H, eps, nullptr, 1, nullptr, s); });
            c->ops.push_back([=](hipStream_t s) { return launch_gemv_q4k(wg, qc, 0, gu, nullptr, nullptr, 2 * I, H, 1, s, fmt); });
            c->ops.push_back([=](hipStream_t s) { return launch_swiglu_quantize(gu, qg, I, 1, I, s); });
            c->ops.push_back([=](hipStream_t s) { return launch_gemv_q4k(wd, qg, 0, h, nullptr, nullptr, H, I, 1, s, fmt); });
            h_prev = h;
        }
        uint8_t* qz = c->q8_trace + (keep ? L * q8_layer : q8_layer);
        const void* wlm = d->w_lm;
        float* logits = d->logits;
        const int64_t V = d->vocab;
        const float* hl = h_prev;
        c->ops.push_back([=](hipStream_t s) { return launch_rmsnorm_quantize(hl, qz, H, eps, nullptr, 1, step, s); });
        c->ops.push_back([=](hipStream_t s) { return launch_gemv_q8_0(wlm, qz, logits, nullptr, V, H, s); });
        if (d->flags & MQ_HOST_LOGITS) add_host_logits(c);
        if (!keep) c->q8_bytes = c->f32_count = 0;
        rc = chain_finish(c, stream, d->flags);
        if (rc != MQ_OK) { chain_free(c); return rc; }
        *out = c;
        return ok();
    }
    for (int l = 0; l < L; ++l) {
        uint8_t* q8 = c->q8_trace + (keep ? l * q8_layer : 0);
        float* f = c->f32_trace + (keep ? l * f32_layer : 0);
        uint8_t *qa = q8, *qb = q8 + qH, *qc = q8 + 2 * qH, *qg = q8 + 3 * qH;
        float *t = f, *o = f + QKV, *gu = f + QKV + H, *h = f + QKV + H + 2 * I;
        const void *wq = d->w_qkv[l], *wo = d->w_o[l], *wg = d->w_gu[l], *wd = d->w_down[l];
        float* gu_keep = keep ? gu : nullptr;
        // stamp regions: kStampPairs pairs per kernel, in step order
        const int64_t sr = 2 * kStampPairs;
        uint64_t* st = c->stamps ? c->stamps + 4 * l * sr : nullptr;
        const NormIn na = l == 0 ? NormIn{x_table, step, n_inputs, eps, keep ? qa : nullptr, nullptr, exact, st}
                                 : NormIn{h_prev, nullptr, 1, eps, keep ? qa : nullptr, nullptr, exact, st};
        const NormIn nb{t, nullptr, 1, eps, keep ? qb : nullptr, nullptr, exact, st ? st + sr : nullptr};
        const NormIn nc{o, nullptr, 1, eps, keep ? qc : nullptr, nullptr, exact, st ? st + 2 * sr : nullptr};
        c->ops.push_back([=](hipStream_t s) { return launch_gemv_q4k_norm(wq, na, t, QKV, H, s, fmt); });
        c->ops.push_back([=](hipStream_t s) { return launch_gemv_q4k_norm(wo, nb, o, H, KO, s, fmt); });
        double* gp = c->gu_part;
        unsigned* gc = c->gu_cnt;
        const int gn = c->gu_split;
        c->ops.push_back([=](hipStream_t s) { return launch_gemv_q4k_swiglu(wg, nullptr, &nc, gu_keep, qg, I, H, s, fmt, gp, gc, gn); });
        if (st)
            c->ops.push_back([=](hipStream_t s) { return launch_gemv_q4k_q8_stamped(wd, qg, h, H, I, s, fmt, st + 3 * sr); });
        else
            c->ops.push_back([=](hipStream_t s) { return launch_gemv_q4k(wd, qg, 0, h, nullptr, nullptr, H, I, 1, s, fmt); });
        h_prev = h;
    }
    uint8_t* qz = c->q8_trace + (keep ? L * q8_layer : q8_layer);
    const void* wlm = d->w_lm;
    float* logits = d->logits;
    const int64_t V = d->vocab;
    const NormIn nz{h_prev, nullptr, 1, eps, keep ? qz : nullptr, step, exact,
                    c->stamps ? c->stamps + (int64_t)4 * L * 2 * kStampPairs : nullptr};
    c->ops.push_back([=](hipStream_t s) { return launch_gemv_q8_0_norm(wlm, nz, logits, V, H, s); });
    if (d->flags & MQ_HOST_LOGITS) add_host_logits(c);
    if (!keep) c->q8_bytes = c->f32_count = 0;

    rc = chain_finish(c, stream, d->flags);
    if (rc != MQ_OK) { chain_free(c); return rc; }
    *out = c;
    return ok();
}

int mq_moe_create(const mq_moe_desc* d, hipStream_t stream, mq_chain** out) {
    CHECK_ARG(d && out, "null desc or out");
    *out = nullptr;
    CHECK_SHAPE(d->n_experts >= 1 && d->n_sel >= 1 && d->n_sel <= 16, "n_experts/n_sel out of range");
    CHECK_SHAPE(d->hidden >= 256 && d->hidden % 256 == 0 && d->hidden <= kMaxK, "hidden must be a multiple of 256");
    CHECK_SHAPE(d->inter >= 32 && d->inter % 32 == 0 && d->inter <= kMaxK, "inter must be a multiple of 32");
    CHECK_SHAPE(d->n_tokens >= 1, "n_tokens must be >= 1");
    CHECK_SHAPE(d->tokens_per_launch >= 0 && d->tokens_per_launch <= 256, "tokens_per_launch out of range [0, 256]");
    const int64_t H = d->hidden, I = d->inter, KP = (I + 255) / 256 * 256;
    CHECK_SHAPE(d->gu_expert_bytes >= 2 * I * (H / 256) * kQ4KBytes && d->gu_expert_bytes % 16 == 0,
                "gu_expert_bytes too small or not a multiple of 16");
    CHECK_SHAPE(d->dn_expert_bytes >= H * (KP / 256) * kQ4KBytes && d->dn_expert_bytes % 16 == 0,
                "dn_expert_bytes too small or not a multiple of 16");
    CHECK_SHAPE(d->n_sel * stage_bytes((int)(KP / 32)) <= kMaxStageLds, "too many slots for LDS");
    CHECK_ARG(d->w_gu_all && d->w_dn_all && d->ids_table && d->logits_table && d->x_table && d->y_table,
              "null pointer in the descriptor");
    CHECK_ARG(aligned(d->w_gu_all, 16) && aligned(d->w_dn_all, 16) && aligned(d->ids_table, 4) &&
                  aligned(d->logits_table, 4) && aligned(d->x_table, 16) && aligned(d->y_table, 4),
              "misaligned pointer (x_table must be 16-byte aligned)");
    if (capturing(stream)) return fail(MQ_ERR_CAPTURE, "mq_moe_create cannot run inside a stream capture");

    mq_chain* c = new mq_chain();
    c->kind = 1;
    int rc = MQ_OK;
    const int S = d->n_sel;
    c->step = (int64_t*)chain_alloc(c, sizeof(int64_t), &rc);
    if (rc == MQ_OK) c->cur = (int64_t*)chain_alloc(c, sizeof(int64_t), &rc);
    int32_t* ids = rc == MQ_OK ? (int32_t*)chain_alloc(c, 64 * sizeof(int32_t), &rc) : nullptr;
    float* comb = rc == MQ_OK ? (float*)chain_alloc(c, 64 * sizeof(float), &rc) : nullptr;
    const int64_t gstride = KP / 32 * kQ8Bytes;
    uint8_t* gq = rc == MQ_OK ? (uint8_t*)chain_alloc(c, (size_t)S * gstride, &rc) : nullptr;
    int32_t* ids_next = rc == MQ_OK ? (int32_t*)chain_alloc(c, 64 * sizeof(int32_t), &rc) : nullptr;
    // gate/up's working blocks beyond a multiple of the CU count run as two
    // halves along K (launch_moe_gate_up), with this hand-over space
    const int gu_split = moe_split_blocks(d->n_sel, I, H);
    if (rc == MQ_OK && gu_split > 0) {
        c->gu_part = (double*)chain_alloc(c, (size_t)gu_split * 128 * sizeof(double), &rc);
        if (rc == MQ_OK) c->gu_cnt = (unsigned*)chain_alloc(c, (size_t)gu_split * sizeof(unsigned), &rc);
        if (rc == MQ_OK) c->gu_split = gu_split;
    }
    if (rc != MQ_OK) { chain_free(c); return rc; }
    c->ids_next = ids_next;
    double* gpart = c->gu_part;
    unsigned* gcnt = c->gu_cnt;
    const int gsplit = c->gu_split;
    c->ids_table = d->ids_table;
    c->n_tokens = d->n_tokens;
    c->n_sel = S;

    // Two kernels per token: gate/up (reads the counter, quantizes x_t in
    // its prologue, writes the routing, the combine weights and
    // Q8(SwiGLU)), then down with the weighted combine, which advances the
    // counter and leaves the next token's routing ids in ids_next, where the
    // next gate/up reads them without waiting for the counter.
    int64_t *step = c->step, *cur = c->cur;
    const mq_moe_desc dd = *d;
    const int per_launch = d->tokens_per_launch > 0 ? d->tokens_per_launch : 1;
    for (int t = 0; t < per_launch; ++t) {
        c->ops.push_back([=](hipStream_t s) {
            return launch_moe_gate_up(dd.w_gu_all, dd.gu_expert_bytes, dd.n_experts, I, H, step, dd.n_tokens,
                                      dd.ids_table, dd.logits_table, dd.x_table, S, KP, cur, ids, comb, gq, nullptr,
                                      s, ids_next, gpart, gcnt, gsplit);
        });
        c->ops.push_back([=](hipStream_t s) {
            return launch_gemv_q4k_grouped(dd.w_dn_all, dd.dn_expert_bytes, dd.n_experts, ids, S, gq, gstride,
                                           nullptr, comb, dd.y_table, cur, dd.n_tokens, H, KP, step, s, dd.ids_table,
                                           ids_next);
        });
    }
    rc = chain_finish(c, stream, d->flags);
    if (rc != MQ_OK) { chain_free(c); return rc; }
    *out = c;
    return ok();
}

static int chain_step(mq_chain* c, int mode, hipStream_t stream) {
    CHECK_ARG(c, "null chain");
    CHECK_ARG(mode == MQ_GRAPH || mode == MQ_EAGER, "mode must be MQ_GRAPH or MQ_EAGER");
    if (mode == MQ_GRAPH && !capturing(stream)) {
        ++c->graph_steps;
        if (c->lazy && !c->capture_tried && c->graph_steps >= 3) try_capture(c);
    }
    if (mode == MQ_GRAPH && c->captured) return hip_status(hipGraphLaunch(c->exec, stream), "hipGraphLaunch");
    return enqueue(c, stream);
}

int mq_decode_chain(mq_chain* c, int mode, hipStream_t stream) {
    CHECK_ARG(!c || c->kind == 0, "not a decode-step chain");
    return chain_step(c, mode, stream);
}

int mq_moe_step(mq_chain* c, int mode, hipStream_t stream) {
    CHECK_ARG(!c || c->kind == 1, "not a routed-expert chain");
    return chain_step(c, mode, stream);
}

int mq_chain_info(const mq_chain* c, int* captured, int* n_nodes, int64_t* step) {
    CHECK_ARG(c, "null chain");
    if (captured) *captured = c->captured;
    if (n_nodes) *n_nodes = c->n_nodes;
    if (step) {
        hipError_t e = hipDeviceSynchronize();
        if (e == hipSuccess) e = hipMemcpy(step, c->step, sizeof(int64_t), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_status(e, "reading the step counter");
    }
    return ok();
}

int mq_chain_capture_stats(const mq_chain* c, int64_t* graph_steps, double* capture_ms) {
    CHECK_ARG(c, "null chain");
    if (graph_steps) *graph_steps = c->graph_steps;
    if (capture_ms) *capture_ms = c->capture_ms;
    return ok();
}

int mq_chain_read_logits(const mq_chain* c, float* host_out, int64_t n, unsigned flags, hipStream_t stream) {
    CHECK_ARG(c && host_out, "null chain or host_out");
    CHECK_ARG(c->kind == 0, "not a decode-step chain");
    CHECK_SHAPE(n == c->vocab, "n=%lld must equal the chain's vocab %lld", (long long)n, (long long)c->vocab);
    return mq_read_to_host(c->logits, host_out, n * (int64_t)sizeof(float), flags, stream);
}

int mq_chain_host_logits(const mq_chain* c, const float** host_logits) {
    CHECK_ARG(c && host_logits, "null chain or out-param");
    CHECK_ARG(c->kind == 0, "not a decode-step chain");
    *host_logits = c->host_logits;
    return ok();
}

int mq_chain_reset(mq_chain* c, int64_t step, hipStream_t stream) {
    CHECK_ARG(c, "null chain");
    CHECK_ARG(step >= 0, "step must be >= 0");
    return hip_status(set_step(c, step, stream), "counter reset");
}

int mq_chain_trace_sizes(const mq_chain* c, int64_t* q8_bytes, int64_t* f32_count) {
    CHECK_ARG(c, "null chain");
    if (q8_bytes) *q8_bytes = c->q8_bytes;
    if (f32_count) *f32_count = c->f32_count;
    return ok();
}

int mq_chain_read_trace(const mq_chain* c, void* q8_out, float* f32_out, hipStream_t stream) {
    CHECK_ARG(c, "null chain");
    CHECK_ARG(c->q8_bytes > 0, "chain was created without MQ_KEEP_INTERMEDIATES");
    hipError_t e = hipSuccess;
    if (q8_out) e = hipMemcpyAsync(q8_out, c->q8_trace, c->q8_bytes, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess && f32_out)
        e = hipMemcpyAsync(f32_out, c->f32_trace, c->f32_count * sizeof(float), hipMemcpyDeviceToDevice, stream);
    return hip_status(e, "trace copy");
}

int mq_chain_read_stamps(mq_chain* c, uint64_t* host_out, int64_t n_pairs, hipStream_t stream) {
    CHECK_ARG(c && host_out, "null chain or output");
    CHECK_ARG(c->stamps, "chain was created without MQ_SPAN_STAMPS");
    CHECK_SHAPE(n_pairs == c->n_stamped, "n_pairs must be %d (4 per layer + 1)", c->n_stamped);
    if (capturing(stream)) return fail(MQ_ERR_CAPTURE, "mq_chain_read_stamps cannot run inside a stream capture");
    hipError_t e = hipStreamSynchronize(stream);
    std::vector<uint64_t> all((size_t)n_pairs * kStampPairs * 2);
    if (e == hipSuccess)
        e = hipMemcpy(all.data(), c->stamps, all.size() * sizeof(uint64_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_status(e, "span stamp read");
    for (int64_t k = 0; k < n_pairs; ++k) {
        uint64_t lo = ~(uint64_t)0, hi = 0;
        for (int j = 0; j < kStampPairs; ++j) {
            lo = std::min(lo, all[(k * kStampPairs + j) * 2]);
            hi = std::max(hi, all[(k * kStampPairs + j) * 2 + 1]);
        }
        host_out[2 * k] = lo;
        host_out[2 * k + 1] = hi;
    }
    return ok();
}

int mq_chain_clear_stamps(mq_chain* c, hipStream_t stream) {
    CHECK_ARG(c, "null chain");
    CHECK_ARG(c->stamps, "chain was created without MQ_SPAN_STAMPS");
    const int64_t n = (int64_t)c->n_stamped * kStampPairs;
    hipLaunchKernelGGL(k_stamp_clear, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, c->stamps, n);
    return hip_status(hipGetLastError(), "span stamp clear");
}

int mq_chain_destroy(mq_chain* c) {
    if (!c) return ok();
    (void)hipDeviceSynchronize();
    chain_free(c);
    return ok();
}

}  // extern "C"
