/*
 * Reference oracle: plain single-threaded definitions (test infrastructure;
 * never linked into or called by the HIP library).  See oracle.h for the
 * formats and the precision rules.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

/* ---------------------------------------------------------------- f16 ---- */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits.
 * Decoded through ldexp in f64, which is exact for every f16 value. */
float oref_f16_to_f32(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1F;
    const int man = h & 0x3FF;
    double v;
    if (e == 0) {
        v = ldexp((double)man, -24);                 /* zero or subnormal */
    } else if (e == 31) {
        v = man ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + man), e - 25);     /* (1 + man/1024) * 2^(e-15) */
    }
    return (float)(sign ? -v : v);
}

/* Round a non-negative f64 holding an integer plus fraction to the nearest
 * integer, ties to even. */
static double round_half_even(double q) {
    double n = floor(q);
    double r = q - n;                                 /* exact: q has < 53 bits */
    if (r > 0.5 || (r == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;
    return n;
}

uint16_t oref_f32_to_f16(float f) {
    uint32_t bits;
    memcpy(&bits, &f, 4);
    const uint16_t sign = (uint16_t)((bits >> 16) & 0x8000);
    if (isnan(f)) return (uint16_t)(sign | 0x7E00);
    const double a = fabs((double)f);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00);   /* rounds past 65504 */
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: a = n * 2^-24; n == 1024 lands on the first normal */
        const double n = round_half_even(a * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int ex;
    frexp(a, &ex);                                    /* a in [2^(ex-1), 2^ex) */
    int E = ex - 1;
    double n = round_half_even(ldexp(a, 10 - E));     /* in [1024, 2048] */
    if (n == 2048.0) { n = 1024.0; E += 1; }
    if (E + 15 >= 31) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(n - 1024.0));
}

void oref_f16_to_f32_n(const uint16_t* h, float* f, int64_t n) {
    for (int64_t i = 0; i < n; ++i) f[i] = oref_f16_to_f32(h[i]);
}

void oref_f32_to_f16_n(const float* f, uint16_t* h, int64_t n) {
    for (int64_t i = 0; i < n; ++i) h[i] = oref_f32_to_f16(f[i]);
}

static uint16_t load_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ---------------------------------------------------------------- q8_0 --- */

/* Per block of 32: amax = max |x|, d = f16(amax / 127), q = round(x / d)
 * with the stored (f16) d, half away from zero, clamped to +-127.  A block
 * whose stored d is zero gets q = 0. */
void oref_quantize_q8_0(const float* x, int64_t k, uint8_t* out) {
    for (int64_t b = 0; b < k / 32; ++b) {
        const float* xb = x + 32 * b;
        uint8_t* ob = out + 34 * b;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            const float a = fabsf(xb[i]);
            if (a > amax) amax = a;
        }
        const float d32 = amax / 127.0f;
        const uint16_t dh = oref_f32_to_f16(d32);
        const float d = oref_f16_to_f32(dh);
        ob[0] = (uint8_t)(dh & 0xFF);
        ob[1] = (uint8_t)(dh >> 8);
        for (int i = 0; i < 32; ++i) {
            int q = 0;
            if (d != 0.0f) {
                const float r = roundf(xb[i] / d);
                q = r > 127.0f ? 127 : (r < -127.0f ? -127 : (int)r);
            }
            ob[2 + i] = (uint8_t)(int8_t)q;
        }
    }
}

void oref_dequant_q8_0(const uint8_t* blocks, int64_t nblk, double* x) {
    for (int64_t b = 0; b < nblk; ++b) {
        const uint8_t* blk = blocks + 34 * b;
        const double d = (double)oref_f16_to_f32(load_u16(blk));
        for (int i = 0; i < 32; ++i) x[32 * b + i] = d * (double)(int8_t)blk[2 + i];
    }
}

/* ---------------------------------------------------------------- q4_K --- */

/* Sixteen 6-bit fields in 12 bytes s[0..11].  Sub-blocks 0-3 keep their
 * scale and min in the low 6 bits of s[j] and s[j+4].  Sub-blocks 4-7 take
 * their low 4 bits from the nibbles of s[j+4] (scale low, min high) and
 * their top 2 bits from the top 2 bits of s[j-4] (scale) and s[j] (min). */
void oref_q4k_scale_min(const uint8_t* s, int j, int* sc, int* m) {
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 0x0F) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Quants: four 32-byte chunks; chunk c covers weights 64c..64c+63, the low
 * nibble of byte l giving weight 64c+l and the high nibble weight 64c+32+l. */
static int q4k_nibble(const uint8_t* qs, int i) {
    const int c = i / 64, l = i % 64;
    const uint8_t byte = qs[32 * c + (l % 32)];
    return l < 32 ? (byte & 0x0F) : (byte >> 4);
}

void oref_dequant_q4k(const uint8_t* sbs, int64_t nsb, double* w) {
    for (int64_t s = 0; s < nsb; ++s) {
        const uint8_t* sb = sbs + 144 * s;
        const double d = (double)oref_f16_to_f32(load_u16(sb));
        const double dmin = (double)oref_f16_to_f32(load_u16(sb + 2));
        for (int i = 0; i < 256; ++i) {
            int sc, m;
            oref_q4k_scale_min(sb + 4, i / 32, &sc, &m);
            w[256 * s + i] = d * sc * q4k_nibble(sb + 16, i) - dmin * m;
        }
    }
}

/* ---------------------------------------------------------------- q4_0 --- */

/* Quants: 16 bytes; byte i holds weight i in its low nibble and weight 16+i
 * in its high nibble. */
static int q4_0_nibble(const uint8_t* qs, int i) {
    return i < 16 ? (qs[i] & 0x0F) : (qs[i - 16] >> 4);
}

void oref_dequant_q4_0(const uint8_t* blocks, int64_t nblk, double* w) {
    for (int64_t b = 0; b < nblk; ++b) {
        const uint8_t* blk = blocks + 18 * b;
        const double d = (double)oref_f16_to_f32(load_u16(blk));
        for (int i = 0; i < 32; ++i) w[32 * b + i] = d * (double)(q4_0_nibble(blk + 2, i) - 8);
    }
}

/* ---------------------------------------------------------------- GEMV --- */

static void dot_row(const double* w, const double* x, int64_t k, float* y, double* s_abs) {
    double acc = 0.0, sa = 0.0;
    for (int64_t i = 0; i < k; ++i) {
        const double p = w[i] * x[i];
        acc += p;
        sa += fabs(p);
    }
    *y = (float)acc;
    if (s_abs) *s_abs = sa;
}

void oref_gemv_q4k_rows(const uint8_t* w, int64_t k, const uint8_t* xq,
                        const int64_t* rows, int64_t n_rows, float* y, double* s_abs) {
    const int64_t nsb = (k + 255) / 256;
    std::vector<double> x(k), wr(256 * nsb);
    oref_dequant_q8_0(xq, k / 32, x.data());
    for (int64_t i = 0; i < n_rows; ++i) {
        oref_dequant_q4k(w + rows[i] * nsb * 144, nsb, wr.data());
        dot_row(wr.data(), x.data(), k, &y[i], s_abs ? &s_abs[i] : nullptr);
    }
}

void oref_gemv_q4k(const uint8_t* w, int64_t m, int64_t k, const uint8_t* xq,
                   float* y, double* s_abs) {
    std::vector<int64_t> rows(m);
    for (int64_t r = 0; r < m; ++r) rows[r] = r;
    oref_gemv_q4k_rows(w, k, xq, rows.data(), m, y, s_abs);
}

void oref_gemv_q8_0_rows(const uint8_t* w, int64_t k, const uint8_t* xq,
                         const int64_t* rows, int64_t n_rows, float* y, double* s_abs) {
    const int64_t nb = k / 32;
    std::vector<double> x(k), wr(k);
    oref_dequant_q8_0(xq, nb, x.data());
    for (int64_t i = 0; i < n_rows; ++i) {
        oref_dequant_q8_0(w + rows[i] * nb * 34, nb, wr.data());
        dot_row(wr.data(), x.data(), k, &y[i], s_abs ? &s_abs[i] : nullptr);
    }
}

void oref_gemv_q8_0(const uint8_t* w, int64_t m, int64_t k, const uint8_t* xq,
                    float* y, double* s_abs) {
    std::vector<int64_t> rows(m);
    for (int64_t r = 0; r < m; ++r) rows[r] = r;
    oref_gemv_q8_0_rows(w, k, xq, rows.data(), m, y, s_abs);
}

void oref_gemv_q4_0_rows(const uint8_t* w, int64_t k, const uint8_t* xq,
                         const int64_t* rows, int64_t n_rows, float* y, double* s_abs) {
    const int64_t nb = k / 32;
    std::vector<double> x(k), wr(k);
    oref_dequant_q8_0(xq, nb, x.data());
    for (int64_t i = 0; i < n_rows; ++i) {
        oref_dequant_q4_0(w + rows[i] * nb * 18, nb, wr.data());
        dot_row(wr.data(), x.data(), k, &y[i], s_abs ? &s_abs[i] : nullptr);
    }
}

void oref_gemv_q4_0(const uint8_t* w, int64_t m, int64_t k, const uint8_t* xq,
                    float* y, double* s_abs) {
    std::vector<int64_t> rows(m);
    for (int64_t r = 0; r < m; ++r) rows[r] = r;
    oref_gemv_q4_0_rows(w, k, xq, rows.data(), m, y, s_abs);
}

/* ---------------------------------------------------------- block sums --- */

void oref_isums_q4k(const uint8_t* w, int64_t m, int64_t k, const uint8_t* xq,
                    int32_t* isum, int32_t* ysum) {
    const int64_t nsb = (k + 255) / 256, nb = k / 32;
    for (int64_t g = 0; g < nb; ++g) {
        int32_t s = 0;
        for (int i = 0; i < 32; ++i) s += (int8_t)xq[34 * g + 2 + i];
        if (ysum) ysum[g] = s;
    }
    for (int64_t r = 0; r < m; ++r) {
        const uint8_t* row = w + r * nsb * 144;
        for (int64_t g = 0; g < nb; ++g) {
            const uint8_t* sb = row + (g / 8) * 144;
            int32_t s = 0;
            for (int i = 0; i < 32; ++i) {
                const int idx = (int)(g % 8) * 32 + i;     /* index inside the super-block */
                s += q4k_nibble(sb + 16, idx) * (int8_t)xq[34 * g + 2 + i];
            }
            isum[r * nb + g] = s;
        }
    }
}

void oref_isums_q8_0(const uint8_t* w, int64_t m, int64_t k, const uint8_t* xq,
                     int32_t* isum) {
    const int64_t nb = k / 32;
    for (int64_t r = 0; r < m; ++r) {
        for (int64_t g = 0; g < nb; ++g) {
            const uint8_t* wb = w + (r * nb + g) * 34;
            int32_t s = 0;
            for (int i = 0; i < 32; ++i) s += (int8_t)wb[2 + i] * (int8_t)xq[34 * g + 2 + i];
            isum[r * nb + g] = s;
        }
    }
}

void oref_isums_q4_0(const uint8_t* w, int64_t m, int64_t k, const uint8_t* xq,
                     int32_t* isum) {
    const int64_t nb = k / 32;
    for (int64_t r = 0; r < m; ++r) {
        for (int64_t g = 0; g < nb; ++g) {
            const uint8_t* blk = w + (r * nb + g) * 18;
            int32_t s = 0;
            for (int i = 0; i < 32; ++i) s += q4_0_nibble(blk + 2, i) * (int8_t)xq[34 * g + 2 + i];
            isum[r * nb + g] = s;
        }
    }
}

/* ---------------------------------------------------------------- glue --- */

void oref_rmsnorm(const float* x, int64_t n, float eps, float* y) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
    const float scale = (float)(1.0 / sqrt(ss / (double)n + (double)eps));
    for (int64_t i = 0; i < n; ++i) y[i] = x[i] * scale;
}

void oref_swiglu(const float* gu, int64_t inter, float* y) {
    for (int64_t i = 0; i < inter; ++i) {
        const double g = gu[i], u = gu[inter + i];
        y[i] = (float)(g / (1.0 + exp(-g)) * u);
    }
}

void oref_softmax(const float* logits, int64_t n, float* p) {
    double mx = -INFINITY;
    for (int64_t i = 0; i < n; ++i) mx = fmax(mx, (double)logits[i]);
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += exp((double)logits[i] - mx);
    for (int64_t i = 0; i < n; ++i) p[i] = (float)(exp((double)logits[i] - mx) / s);
}

/* ---------------------------------------------------------- decode step --- */

int64_t oref_chain_q8_trace_bytes(const oref_chain_desc* d) {
    const int64_t per_layer = (3 * d->hidden + d->inter) / 32 * 34;
    return d->n_layers * per_layer + d->hidden / 32 * 34;
}

int64_t oref_chain_f32_trace_len(const oref_chain_desc* d) {
    return d->n_layers * (d->qkv_rows + d->hidden + 2 * d->inter + d->hidden);
}

void oref_chain(const oref_chain_desc* d, const float* h0, float* logits,
                uint8_t* q8_trace, float* f32_trace, double* s_abs) {
    const int64_t H = d->hidden, I = d->inter, Ko = d->o_k ? d->o_k : d->hidden;
    void (*gemv)(const uint8_t*, int64_t, int64_t, const uint8_t*, float*, double*) =
        d->weight_format == OREF_Q4_0 ? oref_gemv_q4_0 : oref_gemv_q4k;
    std::vector<float> h(h0, h0 + H), t(d->qkv_rows), o(H), gu(2 * I), nrm(I > H ? I : H);
    std::vector<uint8_t> q(I / 32 * 34 > H / 32 * 34 ? I / 32 * 34 : H / 32 * 34);
    uint8_t* q8t = q8_trace;
    float* f32t = f32_trace;
    /* n values kept in a slot of `slot` values, zero past them */
    auto keep_q8 = [&](int64_t n, int64_t slot) {
        if (!q8t) return;
        memcpy(q8t, q.data(), n / 32 * 34);
        memset(q8t + n / 32 * 34, 0, (slot - n) / 32 * 34);
        q8t += slot / 32 * 34;
    };
    auto keep_f32 = [&](const std::vector<float>& v, int64_t n) {
        if (f32t) { memcpy(f32t, v.data(), n * sizeof(float)); f32t += n; }
    };
    for (int l = 0; l < d->n_layers; ++l) {
        oref_rmsnorm(h.data(), H, d->eps, nrm.data());
        oref_quantize_q8_0(nrm.data(), H, q.data());
        keep_q8(H, H);
        gemv(d->w_qkv[l], d->qkv_rows, H, q.data(), t.data(), nullptr);

        oref_rmsnorm(t.data(), Ko, d->eps, nrm.data());     /* first Ko outputs of QKV */
        oref_quantize_q8_0(nrm.data(), Ko, q.data());
        keep_q8(Ko, H);
        gemv(d->w_o[l], H, Ko, q.data(), o.data(), nullptr);

        oref_rmsnorm(o.data(), H, d->eps, nrm.data());
        oref_quantize_q8_0(nrm.data(), H, q.data());
        keep_q8(H, H);
        gemv(d->w_gu[l], 2 * I, H, q.data(), gu.data(), nullptr);

        oref_swiglu(gu.data(), I, nrm.data());
        oref_quantize_q8_0(nrm.data(), I, q.data());
        keep_q8(I, I);
        gemv(d->w_down[l], H, I, q.data(), h.data(), nullptr);

        keep_f32(t, d->qkv_rows);
        keep_f32(o, H);
        keep_f32(gu, 2 * I);
        keep_f32(h, H);
    }
    oref_rmsnorm(h.data(), H, d->eps, nrm.data());
    oref_quantize_q8_0(nrm.data(), H, q.data());
    keep_q8(H, H);
    oref_gemv_q8_0(d->w_lm, d->vocab, H, q.data(), logits, s_abs);
}

/* ------------------------------------------------------ routed experts --- */

void oref_moe_token(const uint8_t* w_gu_all, int64_t gu_bytes,
                    const uint8_t* w_dn_all, int64_t dn_bytes,
                    const int32_t* ids, int n_sel, const float* logits,
                    const float* x, int64_t hidden, int64_t inter,
                    float* y, float* y_slots, float* combine) {
    std::vector<float> c(n_sel), gu(2 * inter), act(inter), ys((size_t)n_sel * hidden);
    std::vector<uint8_t> xq(hidden / 32 * 34), gq(inter / 32 * 34);
    oref_softmax(logits, n_sel, c.data());
    oref_quantize_q8_0(x, hidden, xq.data());
    for (int s = 0; s < n_sel; ++s) {
        const int64_t e = ids[s];
        oref_gemv_q4k(w_gu_all + e * gu_bytes, 2 * inter, hidden, xq.data(), gu.data(), nullptr);
        oref_swiglu(gu.data(), inter, act.data());
        oref_quantize_q8_0(act.data(), inter, gq.data());
        oref_gemv_q4k(w_dn_all + e * dn_bytes, hidden, inter, gq.data(), &ys[(size_t)s * hidden], nullptr);
    }
    for (int64_t r = 0; r < hidden; ++r) {
        double acc = 0.0;
        for (int s = 0; s < n_sel; ++s) acc += (double)c[s] * (double)ys[(size_t)s * hidden + r];
        y[r] = (float)acc;
    }
    if (y_slots) memcpy(y_slots, ys.data(), ys.size() * sizeof(float));
    if (combine) memcpy(combine, c.data(), n_sel * sizeof(float));
}
