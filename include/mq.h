/*
 * libmq — q4_K x q8_0 decode matrix-vector products for AMD MI355X (gfx950).
 *
 * The per-token decode-step GEMV over block-quantized weights: a q4_K weight
 * matrix times an activation requantized to q8_0, with integer 4-way dot
 * products (the MMVQ decode kernel to which '07 · R3 — Small-model
 * per-token overhead', §1, credits a 37% q4_K decode gain), plus the fixed per-step
 * cost around it: one graph per decode step, captured once and replayed
 * ('Part 4 · Lecture 08 — Graph-Resident Decode', §1-§4).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the comment says host.  The caller
 *    owns all of them; the library keeps none of them after the call
 *    returns, except inside a chain object (see mq_chain_create).
 *  - Work is enqueued asynchronously on `stream` (may be NULL for the null
 *    stream).  Nothing synchronizes unless stated.
 *  - Return value: MQ_OK (0) or a negative mq_status.  Argument and shape
 *    errors are found on the host before any HIP call and nothing is
 *    enqueued.  MQ_ERR_HIP reports a launch error; faults during execution
 *    surface at the caller's next synchronization (HIP errors are sticky
 *    and may be reported by a later call — Lecture 08, §3).
 *  - mq_last_error() returns this thread's message for the last failing
 *    call (host memory owned by the library, valid until the next call).
 *  - No exceptions cross this boundary; the library never exits or aborts.
 *  - Threads: the stateless entry points may be called from several host
 *    threads at once, on the same or different streams: the library's
 *    caches (CU counts, occupancy) are guarded, and the split-k workspace
 *    of the batched GEMVs is kept per (device, stream), so calls on
 *    different streams never share it and calls on one stream are ordered
 *    by that stream.  A chain object is not synchronized: calls on one
 *    chain (step, reset, info, reads) must not overlap.  mq_read_to_host
 *    serializes on its mutex.  mq_test_set_fault is a process-wide switch
 *    for single-threaded tests.
 *
 * Formats (little-endian, packed):
 *  - q4_K super-block, 256 weights in 144 bytes: f16 d at 0, f16 dmin at 2,
 *    12 bytes of packed 6-bit scales/mins at 4 (sub-block j<4: sc = s[j]&63,
 *    m = s[j+4]&63; j>=4: sc = (s[j+4]&15) | (s[j-4]>>6)<<4,
 *    m = (s[j+4]>>4) | (s[j]>>6)<<4), 128 bytes of nibbles at 16 (32-byte
 *    chunk c: low nibble of byte l = weight 64c+l, high nibble = weight
 *    64c+32+l).  weight = d*sc_j*q - dmin*m_j, j = index/32.
 *    A q4_K matrix is row-major: row r is ceil(k/256) consecutive
 *    super-blocks, rows back to back.  Base pointers must be 16-byte aligned.
 *  - q8_0 block, 32 values in 34 bytes: f16 d, then 32 int8 q; value = d*q.
 *    A q8_0 vector of k values is k/32 consecutive blocks.  Base pointers
 *    must be 2-byte aligned; q8_0 weight matrices 4-byte aligned.
 *  - q4_0 block, 32 weights in 18 bytes (see mq_gemv_q4_0_q8).
 *  The pages name these formats but do not lay them out; the layout above
 *  is the synthetic workload's definition (q4_0: the plain reading).
 */
#ifndef MQ_H
#define MQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MQ_OK = 0,
    MQ_ERR_ARG = -1,      /* null pointer, bad count, misaligned pointer */
    MQ_ERR_SHAPE = -2,    /* k not a multiple of the block, m < 1, too large */
    MQ_ERR_HIP = -3,      /* a HIP runtime call or launch failed */
    MQ_ERR_CAPTURE = -4,  /* an operation that is illegal while the stream is being captured */
    MQ_ERR_NOMEM = -5     /* device allocation failed */
} mq_status;

const char* mq_last_error(void);
/* "libmq <major>.<minor> (gfx950)".  The minor number rises when a
 * descriptor struct grows (0.2: mq_chain_desc.o_k), so a caller built
 * against an older mq.h can tell that its structs are too short. */
const char* mq_version(void);

/* ---------------------------------------------------------------------------
 * q8_0 activation quantizer.
 * x: f32 [n_cols][k] row-major; xq: n_cols*(k/32) q8_0 blocks, column c's
 * blocks first-to-last at xq + c*(k/32)*34.  k % 32 == 0, 1 <= n_cols.
 * Per block of 32: amax = max|x| (f32), d = f16(amax/127) rounded to
 * nearest even, q = roundf(x/d) with the stored d (halves away from zero),
 * clamped to +-127; a block whose stored d is 0 gets q = 0.  The scan is a
 * max over magnitudes, so the bytes do not depend on reduction order
 * (Lecture 08, §8).  Inputs with |x| > 65504*127 or NaN are out of contract.
 */
int mq_quantize_q8_0(const float* x, void* xq, int64_t k, int n_cols, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * q4_K x q8_0 GEMV (n = 1): y[r] = sum_i w[r,i] * x[i] for r < m.
 * w: q4_K matrix [m][k/256 super-blocks]; xq: k/32 q8_0 blocks; y: f32 [m].
 * k % 256 == 0, m >= 1.  Per 32-value sub-block the kernel forms the exact
 * int32 sums  isum = sum q4*q8 (v_dot4) and ysum = sum q8, then adds
 * d8*(d*sc*isum - dmin*m*ysum) in f64; rows are reduced across the wave in
 * a fixed order and rounded to f32 once.
 */
int mq_gemv_q4k_q8(const void* w, const void* xq, float* y, int64_t m, int64_t k,
                   hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Batched q4_K x q8_0 GEMV, 1 <= n <= 8 activation columns, weights streamed
 * once for all columns.  xq: [n][k/32] q8_0 blocks (column c at
 * xq + c*(k/32)*34); y: f32 [m][n] row-major, y[r*n + c].
 * The kernel family depends on n and the matrix size (mq_gemv_batched_path
 * says which): the vector kernels (v_dot4), with the arithmetic of
 * mq_gemv_q4k_q8 per column, or the matrix cores, whose integer sums feed
 * an f64 fixup that adds the same exact products in another order (results
 * within the same tolerance).  When the kernel splits k across workgroups
 * (vector kernels: the columns do not fit in 64 KB of LDS; matrix cores:
 * rows of more than 16 super-blocks, or too few row tiles to fill the GPU)
 * it sums the f64 partials in a second pass in split order;
 * the partials (vector kernels: ceil(k/4096)*m*n doubles; matrix cores:
 * n_split*m*n doubles, n_split <= k/256, e.g. 10 splits for the
 * 3584 x 18944 matrix) live in a device workspace that
 * the library keeps per (device, stream) and grows on demand to the next
 * power of two (MQ_ERR_NOMEM if that allocation fails; MQ_ERR_CAPTURE if it
 * must grow while `stream` is being captured: call once outside capture
 * first).  A workspace that is outgrown is not freed, because work already
 * enqueued or a graph captured earlier may still use it; all of them are
 * freed by mq_workspace_release.
 */
int mq_gemv_q4k_q8_batched(const void* w, const void* xq, float* y, int64_t m, int64_t k,
                           int n, hipStream_t stream);

/* The batched GEMV for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): same arguments, kernels and results as
 * mq_gemv_q4k_q8_batched, but it never allocates.  When the kernel splits k
 * its partials go to a fixed 4 MiB device array of the library instead of a
 * workspace: the partials described there must fit (for
 * example the 3584 x 18944 matrix takes 0.55 MiB at n = 4 and 2.2 MiB at
 * n = 8), else
 * MQ_ERR_SHAPE, reported on the host before any HIP call.  Each GPU holds
 * its own copy of the array until the process ends, and every call on that
 * GPU uses it: two calls that overlap in time on one GPU (from different
 * streams or threads) race on the partials and give wrong results, so
 * order them on one stream.  Nothing in the array needs clearing between
 * calls (each call writes every partial it reads). */
int mq_gemv_q4k_q8_batched_noalloc(const void* w, const void* xq, float* y, int64_t m, int64_t k,
                                   int n, hipStream_t stream);

/* Test and measurement hook (for comparing the two kernel families): the
 * batched q4_K GEMV of mq_gemv_q4k_q8_batched, forced onto path 0 (the
 * vector kernels: v_dot4 sums, one column per pass over the staged
 * activation) or path 1 (the matrix cores, n >= 2: v_mfma_i32_16x16x64_i8
 * sums of 16 rows x 8 columns x 2 sub-blocks).  The batched entry point
 * itself takes the path mq_gemv_batched_path gives.  Path 1 needs the
 * matrix and one more 16-row tile to fit 32-bit byte offsets (under 4 GiB).
 * Same arguments, errors and workspace as mq_gemv_q4k_q8_batched;
 * MQ_ERR_ARG for another path, MQ_ERR_SHAPE for path 1 with n = 1 or a
 * matrix beyond that size. */
int mq_debug_gemv_q4k_batched_path(const void* w, const void* xq, float* y, int64_t m, int64_t k, int n, int path,
                                   hipStream_t stream);

/* The kernel family the batched entry points (mq_gemv_q4k_q8_batched, its
 * no-allocation form, mq_gemv_q4_0_q8_batched) take for an (m, k, n) shape:
 * *path = 0 for the vector kernels, 1 for the matrix cores.  Host only (no
 * HIP call).  The matrix cores' time hardly grows with n, the vector
 * kernels' does, and the crossover moves to fewer columns as the matrix
 * grows, so q4_K takes the matrix cores from n = min_cols(bytes) with
 * bytes = m*(k/256)*144: below 6 MB never; below 8 MB n = 8; below 24 MB
 * n = 7, or 6 when the vector kernels would split k at n = 6; below 60 MB
 * n = 6, or 4 when they would split k at n = 4 (n columns of k values do
 * not fit in 64 KB of staging); from 60 MB n = 4 — and only while the
 * matrix fits 32-bit offsets.  q4_0 always
 * takes the vector kernels.  weight_format: MQ_FMT_Q4_K or MQ_FMT_Q4_0.
 * Errors: MQ_ERR_ARG for a null path or an unknown format, MQ_ERR_SHAPE as
 * for the batched entry points. */
int mq_gemv_batched_path(int64_t m, int64_t k, int n, int weight_format, int* path);

/* The split-k workspaces (see mq_gemv_q4k_q8_batched).  Host out-params
 * (any may be NULL): bytes held in total, the (device, stream) pairs that
 * have one, and the outgrown buffers still held. */
int mq_workspace_stats(int64_t* bytes, int* n_streams, int* n_retired);
/* Waits for each device that holds a workspace, then frees them all; the
 * next split-k call allocates again.  The caller must not replay a graph
 * captured with a split-k call after this (it would use freed memory). */
int mq_workspace_release(void);

/* ---------------------------------------------------------------------------
 * Grouped GEMV for routed experts.  For slot s < n_sel the expert is
 * e = ids[s] (device int32, read on the device so a captured graph can
 * replay new routing), whose matrix starts at w_all + e*expert_bytes
 * (expert_bytes % 16 == 0, >= m*ceil(k/256)*144).
 * xq_stride_bytes == 0: every slot uses the same activation xq (k/32 blocks);
 * otherwise slot s uses xq + s*xq_stride_bytes.
 * y: f32 [n_sel][m] (y[s*m + r]), may be NULL when combine is given.
 * combine: optional device f32 [n_sel]; when non-NULL, y_out: f32 [m] gets
 * sum_s combine[s]*y_s computed in f64 in slot order s = 0..n_sel-1 and
 * rounded once.  A slot whose id is outside [0, n_experts) is not read; its
 * y row is NaN and so is y_out.  1 <= n_sel <= 16, k % 256 == 0.
 * Each slot's result is the same as mq_gemv_q4k_q8 on that expert.
 */
int mq_gemv_q4k_grouped(const void* w_all, int64_t expert_bytes, int n_experts,
                        const int32_t* ids, int n_sel,
                        const void* xq, int64_t xq_stride_bytes,
                        float* y, const float* combine, float* y_out,
                        int64_t m, int64_t k, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * q4_0 x q8_0 GEMV: the 0.5B model the pages measure is stored in q4_0
 * ('07 · R3 — Small-model per-token overhead', §5), which the pages name but
 * do not lay out.  Read plainly: per 32 weights an 18-byte block, f16 d then
 * 16 quant bytes, byte i holding weight i in its low nibble and weight 16+i
 * in its high nibble, weight = d*(q - 8); rows hold k/32 blocks back to back.
 * w: [m][k/32 blocks] (16-byte aligned); xq: k/32 q8_0 blocks; y: f32 [m].
 * k % 256 == 0 (eight blocks fill one 144-byte group of the 4-bit kernels'
 * lane layout), m >= 1.  Per block the kernel forms the exact int32 sum
 * isum = sum q*q8 of the stored nibbles (v_dot4) and adds
 * d*(d8*isum - 8*d8*ysum) in f64, where d8*ysum is the activation block's
 * scale times its code sum; rows are reduced in a fixed order and rounded
 * to f32 once.  Errors as mq_gemv_q4k_q8.
 */
int mq_gemv_q4_0_q8(const void* w, const void* xq, float* y, int64_t m, int64_t k,
                    hipStream_t stream);
/* 1 <= n <= 8 activation columns; layouts, split-k workspace and errors as
 * mq_gemv_q4k_q8_batched. */
int mq_gemv_q4_0_q8_batched(const void* w, const void* xq, float* y, int64_t m, int64_t k,
                            int n, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * q8_0 x q8_0 GEMV (the lm_head): w: q8_0 matrix [m][k/32 blocks], 4-byte
 * aligned; xq: k/32 blocks; y: f32 [m].  k % 64 == 0.
 * Per block isum = sum w8*x8 (int32), then y += d_w*d_x*isum in f64.
 */
int mq_gemv_q8_0_q8(const void* w, const void* xq, float* y, int64_t m, int64_t k,
                    hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Glue between GEMVs (the elementwise stand-in of the decode step).
 * RMSNorm (unit gain) fused with q8_0 quantization of its output:
 *   y_i = x_i / sqrt(mean(x^2) + eps)  in f64, rounded to f32, then quantized
 *   exactly as mq_quantize_q8_0.  x: f32 [k]; xq: k/32 blocks; k % 32 == 0.
 */
int mq_rmsnorm_quantize_q8_0(const float* x, void* xq, int64_t k, float eps, hipStream_t stream);

/* SwiGLU fused with q8_0 quantization, per column c < n_cols:
 *   gu: f32 [n_cols][2*inter] = [gate | up];  y_i = silu(gate_i)*up_i in f64,
 *   silu(g) = g/(1+exp(-g)), rounded to f32, then quantized.
 *   xq: [n_cols][k_pad/32] blocks; blocks past inter/32 are written as zero
 *   blocks (d = 0, q = 0), so a q4_K matrix padded to k_pad multiplies them
 *   by exact zeros.  inter % 32 == 0, k_pad % 32 == 0, k_pad >= inter.
 */
int mq_swiglu_quantize_q8_0(const float* gu, void* xq, int64_t inter, int n_cols, int64_t k_pad,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Debug dumps of the integer block sums formed inside the production GEMV
 * kernels (the same kernel template, compiled with a dump store).
 * isum: int32 [m][k/32]: isum[r*(k/32)+g] = sum over block g of q4*q8
 * (q4 = stored nibble 0..15) or w8*x8; ysum: int32 [k/32] = sum of the
 * activation codes of each block (q4_K only; may be NULL).  y as the
 * matching GEMV.
 */
int mq_debug_gemv_q4k_q8_isums(const void* w, const void* xq, float* y, int32_t* isum,
                               int32_t* ysum, int64_t m, int64_t k, hipStream_t stream);
int mq_debug_gemv_q8_0_q8_isums(const void* w, const void* xq, float* y, int32_t* isum,
                                int64_t m, int64_t k, hipStream_t stream);
/* The q4_0 kernel's sums: isum as above (q = stored nibble 0..15), ysum as
 * for q4_K (may be NULL).  MQ_ERR_SHAPE when the activation does not fit in
 * LDS (k above about 55,000). */
int mq_debug_gemv_q4_0_q8_isums(const void* w, const void* xq, float* y, int32_t* isum,
                                int32_t* ysum, int64_t m, int64_t k, hipStream_t stream);

/* The decode step's fused gate/up kernel on its own (a test hook):
 * gu = W_gu Q8(RMSNorm(x)) with W_gu's 2*inter rows (gate rows, then up
 * rows) over k = hidden, g_q8 = Q8(SwiGLU(gu)) (inter/32 blocks), gu_out
 * (f32 [2*inter], may be NULL) the GEMV values.  x: f32 [k], 16-byte
 * aligned.  With n_split > 0 the last n_split of the inter/32 output
 * blocks are each computed as two halves along k by two workgroups that
 * hand over through part (128 doubles per split block) and cnt (one
 * unsigned per split block, zero before the call and left zero after it);
 * the chain passes the surplus over a multiple of the CU count.  When the
 * count does not fit the shape (n_split > inter/32, fewer than two passes
 * over k, or part or cnt NULL) every block is computed whole.  Results are
 * the same either way. */
int mq_debug_gate_up_swiglu(const void* w, const float* x, float eps, float* gu_out, void* g_q8, int64_t inter,
                            int64_t k, int n_split, double* part, unsigned* cnt, int weight_format,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Decode-step chain: one decode step of a stand-in model, recorded once as a
 * hipGraph and replayed with one submission per token (Lecture 08, §1).
 * Per layer l (H = hidden, I = inter):
 *   a = Q8(RMSNorm(h));       t  = W_qkv[l]  a   (qkv_rows outputs)
 *   b = Q8(RMSNorm(t[0:H]));  o  = W_o[l]    b   (H)
 *   c = Q8(RMSNorm(o));       gu = W_gu[l]   c   (2I: gate rows then up rows)
 *   g = Q8(SwiGLU(gu));       h  = W_down[l] g   (H)
 * then z = Q8(RMSNorm(h)); logits = W_lm z (q8_0 weights, vocab rows).
 * The step's input h0 is row (step % n_inputs) of x_table, where `step` is
 * a device-resident counter that the last kernel of the step increments:
 * the one thing that must change between replays has to live on the device
 * and be advanced inside the captured region (Lecture 08, §2).
 * Inputs are declared before the step starts and nothing is filled from
 * the host inside it, so the step is one split ('07 · R3', §2).
 * The step is 4 kernels per layer plus the lm_head: each Q8(RMSNorm(.)) is
 * formed in the prologue of the GEMV that consumes it, and Q8(SwiGLU(gu)) in
 * the epilogue of the gate/up GEMV.
 */
typedef struct mq_chain mq_chain;

/* MQ_EXACT_GLUE is a test hook: the RMSNorm->q8_0 prologues compute every
 * value with the divisions themselves instead of reciprocal products that
 * are checked to round the same way; the results are byte-identical.
 * MQ_UNFUSED_GLUE builds the same step without fusion, the measurement arm
 * the fused step is compared against (Lecture 08, §6 re-prices fusion under
 * capture): every Q8(RMSNorm(.)) and Q8(SwiGLU(.)) is its own kernel and the
 * GEMVs read q8_0 inputs, 8 kernels per layer plus 2.  Its RMSNorm sums the
 * squares in another order, so codes can differ from the fused step's by
 * one near a rounding tie; each stage still meets the oracle's bounds. */
/* MQ_LAZY_CAPTURE is the capture policy of '07 · R3' §2: capture costs a
 * one-time host bill (recording plus instantiation, milliseconds) that only
 * repeated use pays back, so the chain is created without a warm step and
 * without a graph, its first two MQ_GRAPH steps run eagerly, and the third
 * captures the step and replays it from then on.  A chain used once or twice
 * never pays for a capture.  Without the flag the chain warms and captures
 * at creation. */
/* MQ_HOST_LOGITS ends the step with a copy of the logits into a pinned host
 * buffer that the chain owns (4*vocab bytes, allocated at creation), so the
 * readback is a node of the captured step instead of a separate blocking
 * copy, and the caller reads the values in place (mq_chain_host_logits) with
 * no host-side copy: a host copy that follows a DMA reads cold memory and
 * costs more than the DMA.  If pinning fails the chain is created without
 * the copy (mq_chain_host_logits gives NULL) and one warning is printed. */
/* MQ_SPAN_STAMPS (measurement; fused step only, ignored with
 * MQ_UNFUSED_GLUE) gives each of the step's 4*n_layers + 1 GEMV kernels a
 * [start, end] pair: the GPU's 100 MHz real-time counter when the
 * kernel's first wave started (minimum over its waves) and when its last
 * wave ended (maximum, taken after the wave's memory operations complete).
 * Each wave stores its own pair (256 KiB of device words per kernel,
 * allocated with the chain); mq_chain_read_stamps reduces and returns
 * them, so that a replay's span (last end minus first start) can be set
 * against the sum of the kernels' own spans without a tracer in the
 * process.  Chains without the flag pass no stamp words; the kernels read
 * the counter at wave start either way (one scalar instruction). */
enum { MQ_EAGER_ONLY = 1u, MQ_KEEP_INTERMEDIATES = 2u, MQ_EXACT_GLUE = 4u, MQ_UNFUSED_GLUE = 8u,
       MQ_LAZY_CAPTURE = 16u, MQ_HOST_LOGITS = 32u, MQ_SPAN_STAMPS = 64u };
enum { MQ_GRAPH = 0, MQ_EAGER = 1 };
/* Weight format of the four layer GEMVs (the lm_head is q8_0 either way). */
enum { MQ_FMT_Q4_K = 0, MQ_FMT_Q4_0 = 1 };

typedef struct {
    int n_layers;                      /* >= 1 */
    int64_t hidden, qkv_rows, inter, vocab;   /* hidden, inter % 256 == 0; qkv_rows >= O's K, % 4 == 0 */
    const void* const* w_qkv;          /* HOST arrays of n_layers device pointers (weight_format) */
    const void* const* w_o;
    const void* const* w_gu;
    const void* const* w_down;
    const void* w_lm;                  /* device q8_0 [vocab][hidden/32] */
    const float* x_table;              /* device f32 [n_inputs][hidden], 16-byte aligned */
    int n_inputs;                      /* >= 1 */
    float* logits;                     /* device f32 [vocab] */
    float eps;
    unsigned flags;                    /* MQ_EAGER_ONLY | MQ_KEEP_INTERMEDIATES | MQ_EXACT_GLUE | MQ_UNFUSED_GLUE
                                          | MQ_LAZY_CAPTURE | MQ_HOST_LOGITS | MQ_SPAN_STAMPS */
    int weight_format;                 /* MQ_FMT_Q4_K or MQ_FMT_Q4_0 (layer matrices) */
    int64_t o_k;                       /* O's K, 0 for hidden: O normalizes and reads the first o_k
                                          QKV outputs (a [hidden][o_k] matrix), as one rank of a
                                          tensor-parallel split takes its own slice of the attention
                                          stand-in; 256 <= o_k <= hidden, o_k % 256 == 0.  With
                                          MQ_KEEP_INTERMEDIATES O's q8_0 input keeps a slot of
                                          hidden/32 blocks, zero past its o_k/32 */
} mq_chain_desc;

/* Validates, allocates every device buffer the step needs (nothing is
 * allocated later: allocation inside a capture is illegal — Lecture 08,
 * §3), runs one eager warm step on `stream` and synchronizes it, resets the
 * step counter to 0, then captures the step into a hipGraph on a private
 * stream (with MQ_LAZY_CAPTURE: only resets the counter; see above).  A
 * capture failure is not an error: it is logged once to stderr and the
 * chain runs eagerly (captured = 0).  Weight, table and logits
 * pointers are baked into the chain: keep them alive and unmoved until
 * mq_chain_destroy.  *out receives the chain (host object owned by the
 * library). */
int mq_chain_create(const mq_chain_desc* desc, hipStream_t stream, mq_chain** out);
/* One decode step on `stream`: MQ_GRAPH replays the graph (falls back to
 * eager launches when not captured), MQ_EAGER launches the same kernels with
 * the same arguments one by one.  The two are byte-identical by
 * construction.  Under MQ_LAZY_CAPTURE the third MQ_GRAPH call captures
 * first (on a private stream; the capture records and runs nothing), then
 * replays; a MQ_GRAPH call made while `stream` is itself being captured
 * neither counts nor captures. */
int mq_decode_chain(mq_chain* c, int mode, hipStream_t stream);
/* Host out-params (any may be NULL): whether a graph exists, its node count,
 * and the device step counter (this call synchronizes the chain's copy). */
int mq_chain_info(const mq_chain* c, int* captured, int* n_nodes, int64_t* step);
/* Host out-params of the capture policy (any may be NULL): the number of
 * MQ_GRAPH steps issued so far and the host wall time, in milliseconds, that
 * recording and instantiating the graph took (0 if it was never captured). */
int mq_chain_capture_stats(const mq_chain* c, int64_t* graph_steps, double* capture_ms);
/* Blocking read of the last step's logits into HOST memory: f32 [n], n must
 * equal the chain's vocab (MQ_ERR_SHAPE otherwise).  Goes through
 * mq_read_to_host with the same flags. */
int mq_chain_read_logits(const mq_chain* c, float* host_out, int64_t n, unsigned flags, hipStream_t stream);
/* *host_logits receives the chain's pinned host copy of the logits, f32
 * [vocab] (NULL if the chain was created without MQ_HOST_LOGITS or pinning
 * failed).  The library owns it until mq_chain_destroy.  It holds the
 * logits of the last step that has completed: synchronize the stream the
 * step ran on before reading, and do not read it while a step is in flight
 * (that step's copy overwrites it). */
int mq_chain_host_logits(const mq_chain* c, const float** host_logits);
/* Set the device step counter (enqueued on `stream` as kernels, capture-safe;
 * a decode-step chain also zeroes the hand-over counters of its split gate/up
 * blocks, and an expert chain refreshes the routing ids it keeps for the
 * token the counter points at). */
int mq_chain_reset(mq_chain* c, int64_t step, hipStream_t stream);
/* With MQ_KEEP_INTERMEDIATES: copy the last step's intermediates into the
 * caller's device buffers (either may be NULL): q8_out gets, per layer, the
 * q8_0 bytes of a, b, c, g, then z; f32_out gets, per layer, t, o, gu, h.
 * Sizes: mq_chain_trace_sizes. */
int mq_chain_trace_sizes(const mq_chain* c, int64_t* q8_bytes, int64_t* f32_count);
int mq_chain_read_trace(const mq_chain* c, void* q8_out, float* f32_out, hipStream_t stream);
/* With MQ_SPAN_STAMPS: synchronize `stream` and write into HOST memory
 * host_out[2*n_pairs] the stamp pair of each GEMV kernel (per layer QKV, O,
 * gate/up, down, then the lm_head): [first wave start, last wave end] in
 * 100 MHz ticks of its most recent launch (each launch overwrites the
 * previous one's words; a kernel not launched since creation or the last
 * mq_chain_clear_stamps reads [UINT64_MAX, 0]).  n_pairs must be
 * 4*n_layers + 1 (MQ_ERR_SHAPE otherwise); MQ_ERR_ARG without the flag;
 * MQ_ERR_CAPTURE while `stream` is being captured.  Blocking. */
int mq_chain_read_stamps(mq_chain* c, uint64_t* host_out, int64_t n_pairs, hipStream_t stream);
/* With MQ_SPAN_STAMPS: enqueue on `stream` a kernel that resets every
 * stamp word to "not launched" (no synchronization).  MQ_ERR_ARG without
 * the flag. */
int mq_chain_clear_stamps(mq_chain* c, hipStream_t stream);
int mq_chain_destroy(mq_chain* c);

/* ---------------------------------------------------------------------------
 * Routed-expert FFN token chain (one token per replay).  Per token t (t is
 * a device counter advanced inside the step):
 *   c = softmax(logits_table[t]) (f64, rounded to f32); xq = Q8(x_table[t]);
 *   gu_s = W_gu[ids_table[t][s]] xq;  g_s = Q8(SwiGLU(gu_s)) padded to
 *   ceil(inter/256)*256;  y_t = sum_s c_s * (W_dn[ids_table[t][s]] g_s).
 * W_gu: n_experts matrices of 2*inter rows x hidden, gu_expert_bytes apart;
 * W_dn: n_experts matrices of hidden rows x ceil(inter/256)*256 (q4_K),
 * dn_expert_bytes apart.  ids/logits/x tables are device arrays of
 * n_tokens rows; y_table: f32 [n_tokens][hidden], row t written by token t.
 * Routing ids are bounds-checked on the device (see mq_gemv_q4k_grouped).
 * A token is two kernels: gate/up with x_t quantized in its prologue and
 * the SwiGLU -> q8_0 glue in its epilogue, then down with the combine.
 * One mq_moe_step runs tokens_per_launch consecutive tokens (their kernels
 * are captured into one graph): a graph launch costs the host about as
 * much as one token's GPU time here, so replaying one token per launch
 * leaves the GPU waiting on the host.
 */
typedef struct {
    int n_experts, n_sel;              /* 1 <= n_sel <= 16 */
    int64_t hidden, inter;             /* hidden % 256 == 0, inter % 32 == 0 */
    const void* w_gu_all;
    int64_t gu_expert_bytes;
    const void* w_dn_all;
    int64_t dn_expert_bytes;
    const int32_t* ids_table;          /* device [n_tokens][n_sel] */
    const float* logits_table;         /* device [n_tokens][n_sel] */
    const float* x_table;              /* device [n_tokens][hidden], 16-byte aligned */
    float* y_table;                    /* device [n_tokens][hidden] */
    int n_tokens;
    unsigned flags;                    /* MQ_EAGER_ONLY | MQ_LAZY_CAPTURE */
    int tokens_per_launch;             /* tokens per mq_moe_step call, 1..256 (0 means 1) */
} mq_moe_desc;

/* Same life cycle and graph/eager semantics as the decode chain; each
 * mq_moe_step runs one token and advances the token counter. */
int mq_moe_create(const mq_moe_desc* desc, hipStream_t stream, mq_chain** out);
int mq_moe_step(mq_chain* c, int mode, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Measurement hook: the next n GEMV kernels (q4_K, batched, grouped, fused
 * chain GEMVs, q8_0) that the calling thread launches, through entry points
 * or eager chain steps, record starts[i] when dispatch i begins executing
 * and stops[i] when it completes: the kernels' own dispatch timestamps, as a
 * kernel trace reports them, with no marker packets between the kernels.
 * Before each timed launch the library synchronizes `stream`, so the
 * dispatch starts on an idle stream and its start timestamp is the kernel's
 * own (a dispatch queued behind a running kernel is stamped early).
 * starts/stops: HOST arrays of n events created by the caller
 * (hipEventCreate); they are copied, so they may be freed after this call.
 * n = 0 clears the hook.  Graph replays are not timed (their kernels were
 * recorded at capture); never arm it while the stream is being captured.
 * 0 <= n <= 65536.
 */
int mq_time_next_launches(const hipEvent_t* starts, const hipEvent_t* stops, int n);

/* ---------------------------------------------------------------------------
 * Measurement: streaming-read probe.  Reads `bytes` at device pointer p once
 * (plain 16-byte loads, one contiguous range per workgroup, four in flight per lane) and writes the
 * XOR of all its 32-bit words to the device uint32 *xor_out (overwritten; the
 * value lets a test check that every word was read).  It gives the read rate
 * this GPU reaches on a large buffer, against which the GEMVs' rates are
 * reported beside the data-sheet HBM peak (the weight stream of
 * 'Part 4 · Lecture 08 — Graph-Resident Decode' is a pure read of this kind).
 * p must be 16-byte aligned and bytes a multiple of 16 (0 allowed);
 * workgroups of 1024 threads, <= 0 for one per CU, at most 65536.
 * Asynchronous on `stream`; the caller owns both buffers.  Errors:
 * MQ_ERR_ARG for null pointers, misalignment, a bad size or workgroup count;
 * MQ_ERR_HIP for a failed launch. */
int mq_probe_stream_read(const void* p, int64_t bytes, uint32_t* xor_out, int workgroups,
                         hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Measurement: what a resident ("persistent") step would pay at each GEMV
 * boundary ('Part 4 · Lecture 08', References: one resident kernel as the
 * endpoint of graph capture), against what a graph replay pays.
 *
 * mq_probe_grid_barrier runs one workgroup of `threads` per CU (refused with
 * MQ_ERR_SHAPE if such a grid cannot be co-resident) for `rounds` rounds of:
 * write this workgroup's exchange_words 32-bit words of a vector with
 * agent-scope stores, wait for them, meet every workgroup at a grid
 * barrier, read the whole vector (CUs * exchange_words words) back with
 * agent-scope loads and check each word.  hierarchical = 0: one agent-scope
 * counter that every workgroup polls; 1: per-XCD counters (XCD from the
 * XCC_ID register), a global count of XCDs, and a per-XCD release flag.
 * Writes the time per round in microseconds (the device's 100 MHz counter)
 * and the number of mismatched words read (0 unless the barrier failed to
 * order the exchange).  Every wait is bounded; a wait that runs out of polls
 * ends the kernel and returns MQ_ERR_HIP.  Allocates and frees its own
 * device buffers; blocking; MQ_ERR_CAPTURE under capture.
 *
 * mq_probe_graph_boundary captures n_kernels empty kernels on one workgroup
 * of `threads` per CU into a graph on a private stream, replays it 3 times,
 * then `reps` times under events, and writes the time per kernel in
 * microseconds: the cost of one kernel boundary inside a replay.  Blocking.
 */
int mq_probe_grid_barrier(int hierarchical, int exchange_words, int rounds, int threads, double* us_per_round,
                          uint32_t* bad_words, hipStream_t stream);
int mq_probe_graph_boundary(int n_kernels, int threads, int reps, double* us_per_kernel);

/* ---------------------------------------------------------------------------
 * Device-to-host readback through a pinned staging buffer ('07 · R3', §2 and
 * §3.1).  A copy into pageable host memory makes the driver bounce it
 * through a pinned buffer of its own (two hops); a copy into memory pinned
 * once and kept skips that, and handing the result to the caller is then a
 * plain host memcpy.
 * mq_read_to_host waits for all work queued on `stream` (the caller wants
 * the value now), copies `bytes` from the device pointer src into the
 * library's pinned buffer, and copies that into host_dst (any host memory,
 * owned by the caller).  The pinned buffer is process-wide, guarded by a
 * mutex, allocated on first use with max(bytes, 4 MiB) (head room so that
 * small changes of size do not reallocate) and reallocated only to grow.
 * If pinning fails the read goes through pageable memory instead and one
 * warning is printed to stderr for the life of the process.  Flag
 * MQ_READ_PAGEABLE skips the pinned buffer (the comparison arm).
 * Errors: MQ_ERR_ARG (null pointer, bytes < 0, unknown flag),
 * MQ_ERR_CAPTURE (stream is being captured: a blocking read cannot be
 * recorded), MQ_ERR_HIP (the wait or the copy failed).  bytes == 0 only
 * waits for the stream. */
enum { MQ_READ_PINNED = 0u, MQ_READ_PAGEABLE = 1u };
int mq_read_to_host(const void* src, void* host_dst, int64_t bytes, unsigned flags, hipStream_t stream);
/* Host out-params (any may be NULL): size of the pinned buffer (0 if none),
 * reads served through it, reads served through pageable memory (by flag
 * or fallback), and whether the fallback warning has been printed. */
int mq_readback_stats(int64_t* pinned_bytes, int64_t* pinned_reads, int64_t* pageable_reads, int* warned);
/* Frees the pinned buffer; the next pinned read allocates it again.  Safe
 * to call at any time from the host (no read holds the buffer after it
 * returns). */
int mq_readback_release(void);

/* ---------------------------------------------------------------------------
 * Test hook, never read from the environment (environment variables are
 * process-global and leak across tests — '07 · R3', §3.3).
 * MQ_FAULT_CAPTURE makes the next chain creations behave as if graph
 * capture failed, to exercise the eager fallback.  MQ_FAULT_PINNED_ALLOC
 * makes the pinned readback buffer's allocation fail (without trying it),
 * to exercise the pageable fallback and its one warning. */
enum { MQ_FAULT_NONE = 0u, MQ_FAULT_CAPTURE = 1u, MQ_FAULT_PINNED_ALLOC = 2u };
int mq_test_set_fault(unsigned fault_mask);

#ifdef __cplusplus
}
#endif

#endif
