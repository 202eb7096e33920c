// Internal host-side launchers (not part of the C ABI).  Each enqueues one
// kernel on `stream` and returns hipGetLastError() of that launch.  Shapes
// are validated by the caller (api.hip) before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "glue.hpp"

namespace mq {

// Lane layout of the q4_K kernels for a row of nsb super-blocks: rows get
// aligned slots of S = 2^log2s lanes (4 lanes per super-block, one 32-byte
// nibble chunk each), R = 64/S rows per wave tile, `passes` sweeps over the
// row's super-blocks.
struct Q4KPlan {
    int log2s, rows_per_tile, passes, n_tiles;
};
Q4KPlan plan_q4k(int64_t m, int nsb);

struct Q8Plan {
    int log2s, rows_per_tile, passes, n_tiles;
};
Q8Plan plan_q8_0(int64_t m, int npairs);

// CUs of the current device, and resident workgroups per CU of a kernel;
// both cached, safe to call from several host threads at once.
int device_cu_count();
int blocks_per_cu(const void* fn, int threads, int lds);

// Events for the next GEMV launches of this thread (see mq_time_next_launches).
void set_next_launch_events(const hipEvent_t* starts, const hipEvent_t* stops, int n);
bool take_next_launch_events(hipEvent_t* start, hipEvent_t* stop);

// Largest LDS a workgroup of the full-staging kernels may take.
constexpr int kMaxStageLds = 64 * 1024;

// Layer weight formats of the 4-bit GEMVs: q4_K super-blocks, or q4_0
// blocks, eight of which fill the same 144 bytes (the plain, RMSNorm,
// batched, split-k and gate/up launchers take either; the grouped and
// expert kernels take q4_K only).
constexpr int kFmtQ4K = 0, kFmtQ4_0 = 1;

// Rows of k weights per launch of the 4-bit kernels, which address the
// matrix with 32-bit byte offsets (launch_gemv_q4k splits taller matrices;
// the chains and the gate/up hook refuse them).
int64_t max_rows_per_launch(int64_t k);
hipError_t launch_gemv_q4k(const void* w, const void* xq, int64_t xq_col_bytes, float* y,
                           int32_t* dump_isum, int32_t* dump_ysum, int64_t m, int64_t k, int ncols,
                           hipStream_t stream, int fmt = kFmtQ4K);
// One q8_0 column, m <= max_rows_per_launch(k), with the kernel's span
// stamps folded into stamp[0..1] (SpanStamp) when stamp is set.
hipError_t launch_gemv_q4k_q8_stamped(const void* w, const void* xq, float* y, int64_t m, int64_t k,
                                      hipStream_t stream, int fmt, uint64_t* stamp);
// The 4-bit GEMV of one activation Q8(RMSNorm(x)) formed in the kernel's
// prologue from the f32 input nin describes (the decode-step chain).
hipError_t launch_gemv_q4k_norm(const void* w, const NormIn& nin, float* y, int64_t m, int64_t k,
                                hipStream_t stream, int fmt = kFmtQ4K);
// Gate/up GEMV with the SwiGLU stand-in fused: rows [0, inter) are gate rows,
// [inter, 2*inter) up rows; writes Q8(silu(gate)*up) (inter/32 blocks) and,
// if gu_out is set, the f32 GEMV outputs.  inter % 32 == 0.  The activation
// is xq, or Q8(RMSNorm(x)) formed in the prologue when nin is set.
// With part/cnt and n_split > 0 (normally swiglu_split_blocks, taken when
// the caller sized part/cnt), the last n_split output blocks are each
// computed as two halves along K by two workgroups that hand over through
// part (128 doubles per block) and cnt (one counter per block, zero before
// the launch and left zero after it); see k_gemv_q4k_swiglu.
hipError_t launch_gemv_q4k_swiglu(const void* w, const void* xq, const NormIn* nin, float* gu_out, void* g_q8,
                                  int64_t inter, int64_t k, hipStream_t stream, int fmt = kFmtQ4K,
                                  double* part = nullptr, unsigned* cnt = nullptr, int n_split = 0);
int swiglu_split_blocks(int64_t inter, int64_t k);
// Workgroups and threads per workgroup for `units` equal work units of a
// kernel whose workgroups each run a prologue of `prologue` per-thread
// steps: about one workgroup per CU, of at most max_waves waves.
void prologue_grid(int64_t units, int64_t prologue, int* grid, int* threads, int max_waves);
// Waves per CU of the one-workgroup-per-CU kernels (measured on the 7B
// decode step: 16 waves 1.260 ms, 12: 1.249, 8: 1.215, 6: 1.334, 4: 1.433).
// More waves compete for each SIMD's issue and lengthen every wave's turn
// from data arrival to its next request, which costs more than their extra
// loads in flight buy; fewer leave the K = 3584 RMSNorm prologue more chunks
// per thread than it keeps in registers.  The q8_0-input GEMV, whose
// prologue is short, takes about kItemsPerWave items per wave within
// [kWavesQ8EarlyMin, kWavesQ8EarlyMax]: 7 waves for the 3584 x 18944 down
// projection (two tiles per wave; 1.207 ms/step), 12 for a 37888 x 3584
// matrix (15.9 against 16.5 us at 8 and 17.2 at 16).
constexpr int kWavesNorm = 8, kWavesQ8Norm = 8;
constexpr int kWavesQ8EarlyMin = 7, kWavesQ8EarlyMax = 12, kItemsPerWave = 10;
// Split-k variant for shapes whose activation does not fit in LDS; `part`
// holds n_split*m*ncols doubles.
int gemv_q4k_splitk_nsplit(int64_t k);
hipError_t launch_gemv_q4k_splitk(const void* w, const void* xq, int64_t xq_col_bytes, float* y,
                                  double* part, int64_t m, int64_t k, int ncols, hipStream_t stream,
                                  int fmt = kFmtQ4K);
hipError_t launch_gemv_q4k_grouped(const void* w_all, int64_t expert_bytes, int n_experts,
                                   const int32_t* ids, int n_sel, const void* xq, int64_t xq_stride,
                                   float* y, const float* combine, float* y_out,
                                   const int64_t* out_row, int64_t out_rows, int64_t m, int64_t k,
                                   int64_t* inc_step, hipStream_t stream, const int32_t* ids_table = nullptr,
                                   int32_t* ids_next = nullptr);
// One routed-expert token's gate/up GEMVs with the SwiGLU -> q8_0 epilogue
// (k_moe_gate_up): token t = *step mod n_tokens; writes cur = t, ids_out,
// combine_out (softmax of the router logits) and g_q8 (n_sel columns of
// k_pad/32 blocks, zero past inter); gu_out, if set, the f32 gate/up rows.
hipError_t launch_moe_gate_up(const void* w_all, int64_t expert_bytes, int n_experts, int64_t inter, int64_t k,
                              const int64_t* step, int n_tokens, const int32_t* ids_table,
                              const float* logits_table, const float* x_table, int n_sel, int64_t k_pad,
                              int64_t* cur, int32_t* ids_out, float* combine_out, void* g_q8, float* gu_out,
                              hipStream_t stream, const int32_t* ids_next = nullptr, double* part = nullptr,
                              unsigned* cnt = nullptr, int n_split = 0);
// Working blocks (n_sel * inter/32) beyond a multiple of the CU count, which
// launch_moe_gate_up splits in two halves along K when given part/cnt sized
// for them and n_split (the hand-over of launch_gemv_q4k_swiglu: 128 doubles
// and one counter, zero before and after a launch, per split block).
int moe_split_blocks(int n_sel, int64_t inter, int64_t k);
// ids_next[0..n_sel) = the routing ids of token (*step mod n_tokens): set
// wherever the expert chain's counter is set, kept current by the down
// kernel that advances it (ids_next of launch_gemv_q4k_grouped), and read
// by the next gate/up kernel (ids_next of launch_moe_gate_up).
hipError_t launch_moe_prime(const int64_t* step, int n_tokens, const int32_t* ids_table, int n_sel,
                            int32_t* ids_next, hipStream_t stream);
hipError_t launch_gemv_q8_0(const void* w, const void* xq, float* y, int32_t* dump_isum, int64_t m,
                            int64_t k, hipStream_t stream);
hipError_t launch_gemv_q8_0_norm(const void* w, const NormIn& nin, float* y, int64_t m, int64_t k,
                                 hipStream_t stream);

hipError_t launch_quantize_q8_0(const float* x, void* xq, int64_t k, int n_cols, hipStream_t stream);
// x row: if sel_step != NULL, row (sel_step % n_inputs) of x (x_table) is
// used; if inc_step != NULL, that counter is advanced by one (a kernel may
// not do both: its workgroups read the counter at different times).
hipError_t launch_rmsnorm_quantize(const float* x, void* xq, int64_t k, float eps, const int64_t* sel_step,
                                   int n_inputs, int64_t* inc_step, hipStream_t stream);
hipError_t launch_swiglu_quantize(const float* gu, void* xq, int64_t inter, int n_cols, int64_t k_pad,
                                  hipStream_t stream);
hipError_t launch_set_i64(int64_t* p, int64_t v, hipStream_t stream);
// p[0..n) = 0 with a kernel (no memset node when the stream is captured).
hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t stream);
// XOR of the 32-bit words of bytes (multiple of 16) at p (16-byte aligned)
// into *xor_out; workgroups <= 0 means one per CU.
// y[i] = sum over s < n_split of part[s*n + i], in that order, as f32.
hipError_t launch_splitk_finalize(const double* part, float* y, int64_t n, int n_split, hipStream_t stream);

// Batched q4_K x q8_0 GEMV on the matrix cores (gemv_mfma.hip), 2 <= ncols
// <= 8, k % 256 == 0.  k is split over n_split ranges of sb_per_split
// super-blocks; with n_split > 1, part receives n_split*m*ncols f64
// partials (gemv_q4k_mfma_partial_bytes; 0 when k is not split).
struct MfmaPlan {
    int n_split, sb_per_split, n_tiles, lds, grid_x, threads;
};
MfmaPlan plan_gemv_q4k_mfma(int64_t m, int nsb);
// The matrix-core kernel addresses the matrix with 32-bit byte offsets: the
// m rows and one more 16-row tile must fit (else launch_gemv_q4k_mfma
// refuses the shape and the batched GEMV takes the vector kernels).
bool mfma_rows_fit(int64_t m, int64_t k);
int64_t gemv_q4k_mfma_partial_bytes(int64_t m, int64_t k, int ncols);
hipError_t launch_gemv_q4k_mfma(const void* w, const void* xq, int64_t xq_col_bytes, float* y, double* part,
                                int64_t m, int64_t k, int ncols, hipStream_t stream);

// Synchronization probes (sync_probe.hip); 0 = measured, 1 = the grid
// cannot be co-resident, 2 = a HIP call failed.
int grid_barrier_probe(int hierarchical, int words, int rounds, int threads, double* us_per_round,
                       uint32_t* bad_words, int* spin_limit_hit, hipStream_t stream);
int graph_boundary_probe(int n_kernels, int threads, int reps, double* us_per_kernel);
hipError_t launch_stream_read(const void* p, int64_t bytes, uint32_t* xor_out, int workgroups,
                              hipStream_t stream);

}  // namespace mq
