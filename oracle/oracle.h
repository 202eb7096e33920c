/*
 * Reference oracle for the q4_K x q8_0 decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, single-threaded CPU
 * implementation that defines what the HIP library must compute.  Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may load or
 * call it; the library itself never does.  It shares no code with the HIP
 * path: its own f16 conversion, its own block decoding, its own glue.
 *
 * Arithmetic: every dequantized value and every dot product is formed in
 * f64 (the pages fix no precision).  The one place where floating point
 * decides an integer, q8_0 quantization, runs in f32 exactly as the GPU
 * quantizer does: an f32 max, an IEEE f32 divide, f16 round-to-nearest-even
 * of the scale, and roundf (half away from zero).
 *
 * Formats (little-endian, packed, no padding):
 *   q4_K super-block, 256 weights in 144 bytes:
 *     [0,2) f16 d   [2,4) f16 dmin   [4,16) 12 bytes of packed 6-bit
 *     scales/mins   [16,144) 128 bytes of 4-bit quants.
 *     weight = d*sc_j*q - dmin*m_j for sub-block j = index/32.
 *   q8_0 block, 32 values in 34 bytes: [0,2) f16 d, [2,34) int8 q[32];
 *     value = d*q.
 *   q4_0 block, 32 weights in 18 bytes: [0,2) f16 d, [2,18) 16 bytes of
 *     4-bit quants, byte i holding weight i in its low nibble and weight
 *     16+i in its high nibble; weight = d*(q - 8).  Rows hold k/32 blocks.
 *     The pages measure a 0.5B model in this format ('07 · R3', §5) without
 *     laying it out; this is the plain reading of the name.
 * The pages name both formats ('07 · R3 — Small-model per-token overhead',
 * §1, credits a 37% q4_K decode gain to an MMVQ kernel that dots q4_K
 * weights against q8_0 activations with 4-way integer products) but do not
 * lay them out; the layout above is the synthetic workload's.
 *
 * Parity pins: see tests/oracle_pins.py.  Every function here is pinned by
 * at least one check that does not re-run its own formula.
 */
#ifndef MQ_ORACLE_H
#define MQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* --- f16 <-> f32 (bit-level, round to nearest even, subnormals, inf, nan) */
float oref_f16_to_f32(uint16_t h);
uint16_t oref_f32_to_f16(float f);
void oref_f16_to_f32_n(const uint16_t* h, float* f, int64_t n);
void oref_f32_to_f16_n(const float* f, uint16_t* h, int64_t n);

/* --- q8_0 ---------------------------------------------------------------- */
/* Quantize k values (k % 32 == 0) into k/32 packed 34-byte blocks. */
void oref_quantize_q8_0(const float* x, int64_t k, uint8_t* out);
/* Dequantize nblk blocks into 32*nblk f64 values. */
void oref_dequant_q8_0(const uint8_t* blocks, int64_t nblk, double* x);

/* --- q4_K ---------------------------------------------------------------- */
/* Scale and min of sub-block j (0..7) from the 12 packed bytes. */
void oref_q4k_scale_min(const uint8_t* s12, int j, int* sc, int* m);
/* Dequantize nsb super-blocks into 256*nsb f64 weights. */
void oref_dequant_q4k(const uint8_t* sbs, int64_t nsb, double* w);

/* --- q4_0 ---------------------------------------------------------------- */
/* Dequantize nblk blocks into 32*nblk f64 weights. */
void oref_dequant_q4_0(const uint8_t* blocks, int64_t nblk, double* w);

/* --- GEMV: dequantize, then dot in f64, ascending index -------------------
 * Rows are stored in ceil(k/256) super-blocks; only the first k weights of
 * a row take part (k % 32 == 0).  xq holds k/32 q8_0 blocks.
 * y[r] = (float) sum_i w[r,i]*x[i];  s_abs[r] = sum_i |w[r,i]*x[i]| (may be NULL). */
void oref_gemv_q4k(const uint8_t* w, int64_t m, int64_t k, const uint8_t* xq,
                   float* y, double* s_abs);
/* Same for the listed rows only: y[i], s_abs[i] belong to rows[i]. */
void oref_gemv_q4k_rows(const uint8_t* w, int64_t k, const uint8_t* xq,
                        const int64_t* rows, int64_t n_rows, float* y, double* s_abs);
/* q8_0 weights: row r holds k/32 blocks. */
void oref_gemv_q8_0(const uint8_t* w, int64_t m, int64_t k, const uint8_t* xq,
                    float* y, double* s_abs);
void oref_gemv_q8_0_rows(const uint8_t* w, int64_t k, const uint8_t* xq,
                         const int64_t* rows, int64_t n_rows, float* y, double* s_abs);
/* q4_0 weights: row r holds k/32 blocks of 18 bytes. */
void oref_gemv_q4_0(const uint8_t* w, int64_t m, int64_t k, const uint8_t* xq,
                    float* y, double* s_abs);
void oref_gemv_q4_0_rows(const uint8_t* w, int64_t k, const uint8_t* xq,
                         const int64_t* rows, int64_t n_rows, float* y, double* s_abs);

/* --- integer block sums ---------------------------------------------------
 * isum[r*(k/32)+g] = sum over the 32 values of block g of q4*q8 (q4 = the
 * stored nibble 0..15); ysum[g] = sum of the 32 int8 activation values. */
void oref_isums_q4k(const uint8_t* w, int64_t m, int64_t k, const uint8_t* xq,
                    int32_t* isum, int32_t* ysum);
/* isum[r*(k/32)+g] = sum over block g of w8*x8. */
void oref_isums_q8_0(const uint8_t* w, int64_t m, int64_t k, const uint8_t* xq,
                     int32_t* isum);
/* isum[r*(k/32)+g] = sum over block g of q4*q8 (q4 = the stored nibble 0..15). */
void oref_isums_q4_0(const uint8_t* w, int64_t m, int64_t k, const uint8_t* xq,
                     int32_t* isum);

/* --- elementwise stand-ins between GEMVs ------------------------------------ */
/* RMSNorm with unit gain: scale = 1/sqrt(mean(x^2) + eps) formed in f64 (sum
 * of squares in index order) and rounded to f32 once; y_i = x_i * scale, one
 * f32 multiply. */
void oref_rmsnorm(const float* x, int64_t n, float eps, float* y);
/* (f64, rounded to f32 once) */
/* gu = [gate(inter) | up(inter)];  y_i = silu(gate_i) * up_i, silu(g) = g/(1+e^-g). */
void oref_swiglu(const float* gu, int64_t inter, float* y);
/* p_i = exp(l_i - max l) / sum_j exp(l_j - max l). */
void oref_softmax(const float* logits, int64_t n, float* p);

/* --- one decode step --------------------------------------------------------
 * Per layer:  a = Q8(RMSNorm(h));        t  = W_qkv  a   (qkv_rows)
 *             b = Q8(RMSNorm(t[0:Ko]));  o  = W_o    b   (H rows, Ko columns)
 *             c = Q8(RMSNorm(o));        gu = W_gu   c   (2*inter: gate rows, then up rows)
 *             g = Q8(SwiGLU(gu));        h  = W_down g   (H)
 * Final:      z = Q8(RMSNorm(h));        logits = W_lm z (q8_0 weights, vocab rows)
 * The four layer GEMVs take q4_K weights, or q4_0 with weight_format
 * OREF_Q4_0.  Weight pointers are host arrays of n_layers host pointers.
 * Optional traces (NULL to skip):
 *   q8_trace: per layer the Q8 bytes of a, b, c, g, then z at the end (b in a
 *             slot of H/32 blocks, zero past its Ko/32);
 *   f32_trace: per layer t, o, gu, h.
 *   s_abs: vocab f64 values for the final GEMV. */
typedef struct {
    int n_layers;
    int64_t hidden, qkv_rows, inter, vocab;
    const uint8_t* const* w_qkv;
    const uint8_t* const* w_o;
    const uint8_t* const* w_gu;
    const uint8_t* const* w_down;
    const uint8_t* w_lm;
    float eps;
    int weight_format;      /* OREF_Q4K or OREF_Q4_0 */
    /* Ko, O's K (0 means H): one rank's share of a tensor-parallel split
     * takes O's columns for its own slice of the attention stand-in, the
     * first Ko outputs of its QKV rows.  256 <= Ko <= H, Ko % 256 == 0,
     * Ko <= qkv_rows. */
    int64_t o_k;
} oref_chain_desc;
enum { OREF_Q4K = 0, OREF_Q4_0 = 1 };

int64_t oref_chain_q8_trace_bytes(const oref_chain_desc* d);
int64_t oref_chain_f32_trace_len(const oref_chain_desc* d);
void oref_chain(const oref_chain_desc* d, const float* h0, float* logits,
                uint8_t* q8_trace, float* f32_trace, double* s_abs);

/* --- one routed-expert FFN token -------------------------------------------
 * c = softmax(logits[0:n_sel]);  xq = Q8(x)
 * per slot s: gu_s = W_gu[ids_s] xq;  g_s = Q8(SwiGLU(gu_s));  y_s = W_dn[ids_s] g_s
 * y = (float) sum_s c_s * y_s in slot order.
 * Expert e's gate/up matrix (2*inter rows, K = hidden) starts at
 * w_gu_all + e*gu_bytes; its down matrix (hidden rows, K = inter, rows stored
 * in ceil(inter/256) super-blocks) at w_dn_all + e*dn_bytes.
 * y_slots (n_sel*hidden) and combine (n_sel) may be NULL. */
void oref_moe_token(const uint8_t* w_gu_all, int64_t gu_bytes,
                    const uint8_t* w_dn_all, int64_t dn_bytes,
                    const int32_t* ids, int n_sel, const float* logits,
                    const float* x, int64_t hidden, int64_t inter,
                    float* y, float* y_slots, float* combine);

#ifdef __cplusplus
}
#endif

#endif
