"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Each mutation is a plausible slip (a swapped nibble, a wrong source byte for
the high scale bits, a dropped or sign-flipped term, a wrong rounding mode,
a wrong stride or operand).  It is applied to a copy of oracle/oracle.cpp in
a temporary directory, compiled, and run against every pin.  The committed
oracle is never modified.
"""
import os
import shutil

import pytest

import oracle
from oracle import build as obuild
from oracle_pins import ALL_PINS

MUTATIONS = [
    ("nibble order swapped",
     "return l < 32 ? (byte & 0x0F) : (byte >> 4);", "return l < 32 ? (byte >> 4) : (byte & 0x0F);"),
    ("chunk stride 16 instead of 32",
     "qs[32 * c + (l % 32)]", "qs[16 * c + (l % 32)]"),
    ("high scale bits from the min byte",
     "*sc = (s[j + 4] & 0x0F) | ((s[j - 4] >> 6) << 4);", "*sc = (s[j + 4] & 0x0F) | ((s[j] >> 6) << 4);"),
    ("high min bits from the scale byte",
     "*m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);", "*m = (s[j + 4] >> 4) | ((s[j - 4] >> 6) << 4);"),
    ("low scale bits keep all six bits of s[j] for j<4 but mask 31",
     "*sc = s[j] & 63;", "*sc = s[j] & 31;"),
    ("min term sign flipped",
     "w[256 * s + i] = d * sc * q4k_nibble(sb + 16, i) - dmin * m;",
     "w[256 * s + i] = d * sc * q4k_nibble(sb + 16, i) + dmin * m;"),
    ("min term dropped",
     "w[256 * s + i] = d * sc * q4k_nibble(sb + 16, i) - dmin * m;",
     "w[256 * s + i] = d * sc * q4k_nibble(sb + 16, i);"),
    ("d and dmin swapped",
     "const double dmin = (double)oref_f16_to_f32(load_u16(sb + 2));",
     "const double dmin = d; const double dd = (double)oref_f16_to_f32(load_u16(sb + 2)); (void)dd;"),
    ("sub-block index from 64-weight chunks",
     "oref_q4k_scale_min(sb + 4, i / 32, &sc, &m);", "oref_q4k_scale_min(sb + 4, i / 64, &sc, &m);"),
    ("q8 ties to even",
     "const float r = roundf(xb[i] / d);", "const float r = rintf(xb[i] / d);"),
    ("q8 divides by the unrounded scale",
     "const float r = roundf(xb[i] / d);", "const float r = roundf(xb[i] / d32);"),
    ("q8 amax over signed values",
     "const float a = fabsf(xb[i]);", "const float a = xb[i];"),
    ("q8 scale over 128",
     "const float d32 = amax / 127.0f;", "const float d32 = amax / 128.0f;"),
    ("q8 dequant reads from byte 1",
     "x[32 * b + i] = d * (double)(int8_t)blk[2 + i];", "x[32 * b + i] = d * (double)(int8_t)blk[1 + i];"),
    ("f16 ties round up",
     "if (r > 0.5 || (r == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;", "if (r >= 0.5) n += 1.0;"),
    ("f16 subnormal exponent off by one",
     "v = ldexp((double)man, -24);", "v = ldexp((double)man, -25);"),
    ("f16 overflow at the largest finite value",
     "if (a >= 65520.0) return", "if (a > 65504.0) return"),
    ("row stride without the header bytes",
     "oref_dequant_q4k(w + rows[i] * nsb * 144, nsb, wr.data());",
     "oref_dequant_q4k(w + rows[i] * nsb * 128, nsb, wr.data());"),
    ("s_abs without the absolute value",
     "sa += fabs(p);", "sa += p;"),
    ("dot over one block too few",
     "for (int64_t i = 0; i < k; ++i) {\n        const double p", "for (int64_t i = 0; i < k - 32; ++i) {\n        const double p"),
    ("isum reads the activation scale bytes",
     "s += q4k_nibble(sb + 16, idx) * (int8_t)xq[34 * g + 2 + i];",
     "s += q4k_nibble(sb + 16, idx) * (int8_t)xq[34 * g + i];"),
    ("isum nibble from the wrong sub-block",
     "const int idx = (int)(g % 8) * 32 + i;", "const int idx = (int)(g % 4) * 32 + i;"),
    ("q8_0 isum transposed operand index",
     "const uint8_t* wb = w + (r * nb + g) * 34;", "const uint8_t* wb = w + (g * m + r) * 34;"),
    ("rmsnorm without eps",
     "sqrt(ss / (double)n + (double)eps)", "sqrt(ss / (double)n)"),
    ("rmsnorm over the sum instead of the mean",
     "sqrt(ss / (double)n + (double)eps)", "sqrt(ss + (double)eps)"),
    ("swiglu gate and up swapped",
     "const double g = gu[i], u = gu[inter + i];", "const double u = gu[i], g = gu[inter + i];"),
    ("silu sign",
     "y[i] = (float)(g / (1.0 + exp(-g)) * u);", "y[i] = (float)(g / (1.0 + exp(g)) * u);"),
    ("softmax not normalised",
     "p[i] = (float)(exp((double)logits[i] - mx) / s);", "p[i] = (float)(exp((double)logits[i] - mx));"),
    ("chain O normalises all of QKV",
     "oref_rmsnorm(t.data(), Ko, d->eps, nrm.data());     /* first Ko outputs of QKV */",
     "oref_rmsnorm(t.data() + (d->qkv_rows - Ko), Ko, d->eps, nrm.data());"),
    ("chain layer output not carried",
     "gemv(d->w_down[l], H, I, q.data(), h.data(), nullptr);",
     "gemv(d->w_down[l], H, I, q.data(), o.data(), nullptr);"),
    ("q4_0 nibble halves swapped",
     "return i < 16 ? (qs[i] & 0x0F) : (qs[i - 16] >> 4);", "return i < 16 ? (qs[i] >> 4) : (qs[i - 16] & 0x0F);"),
    ("q4_0 nibbles interleaved by byte",
     "return i < 16 ? (qs[i] & 0x0F) : (qs[i - 16] >> 4);", "return (qs[i / 2] >> (4 * (i & 1))) & 0x0F;"),
    ("q4_0 offset 7",
     "w[32 * b + i] = d * (double)(q4_0_nibble(blk + 2, i) - 8);",
     "w[32 * b + i] = d * (double)(q4_0_nibble(blk + 2, i) - 7);"),
    ("q4_0 block stride without the scale",
     "const uint8_t* blk = blocks + 18 * b;", "const uint8_t* blk = blocks + 16 * b;"),
    ("q4_0 row stride of q8_0 blocks",
     "oref_dequant_q4_0(w + rows[i] * nb * 18, nb, wr.data());",
     "oref_dequant_q4_0(w + rows[i] * nb * 34, nb, wr.data());"),
    ("q4_0 isum with the offset applied",
     "s += q4_0_nibble(blk + 2, i) * (int8_t)xq[34 * g + 2 + i];",
     "s += (q4_0_nibble(blk + 2, i) - 8) * (int8_t)xq[34 * g + 2 + i];"),
    ("chain ignores the q4_0 weight format",
     "d->weight_format == OREF_Q4_0 ? oref_gemv_q4_0 : oref_gemv_q4k;",
     "d->weight_format == OREF_Q4K ? oref_gemv_q4_0 : oref_gemv_q4k;"),
    ("moe combine in reverse slot weights",
     "acc += (double)c[s] * (double)ys[(size_t)s * hidden + r];",
     "acc += (double)c[n_sel - 1 - s] * (double)ys[(size_t)s * hidden + r];"),
]


def _apply(src, find, repl):
    assert src.count(find) == 1, f"mutation anchor not unique/absent: {find!r}"
    return src.replace(find, repl)


def test_mutation_anchors_present():
    src = open(obuild.SOURCE).read()
    for name, find, _ in MUTATIONS:
        assert src.count(find) == 1, name


@pytest.mark.parametrize("name,find,repl", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(tmp_path, name, find, repl):
    src = _apply(open(obuild.SOURCE).read(), find, repl)
    path = tmp_path / "oracle.cpp"
    path.write_text(src)
    shutil.copy(os.path.join(obuild.HERE, "oracle.h"), tmp_path / "oracle.h")
    lib = oracle.load(obuild.build(str(path), str(tmp_path / "liboracle_mut.so"), str(tmp_path)))
    o = oracle.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
            break
        except Exception as e:   # a crash or overflow inside a pin also counts as caught
            failed.append(f"{pin.__name__}: {type(e).__name__}")
            break
    assert failed, f"planted mistake '{name}' passes every pin"
