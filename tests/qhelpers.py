"""Test-side block builders: known values -> bytes.

These go the opposite way from the oracle's decoders (bytes -> values), so a
test that builds a block from chosen scales, mins and nibbles knows the
true values without decoding anything.  The packing inverts the scale/min
rule of the q4_K format: sub-blocks 0-3 store scale and min in the low six
bits of bytes j and j+4; sub-blocks 4-7 store their low four bits in the two
nibbles of byte j+4 (scale low, min high) and their top two bits in the top
bits of bytes j-4 (scale) and j (min).
"""
from __future__ import annotations

import numpy as np


def f16_bytes(v: float) -> bytes:
    return np.float16(v).tobytes()


def f16_value(v: float) -> float:
    """The f64 value of v rounded to f16 (numpy, round to nearest even)."""
    return float(np.float16(v))


def pack_scales(sc, m) -> bytes:
    s = [0] * 12
    for j in range(4):
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    return bytes(s)


def nibble_byte(i: int):
    """(byte offset inside the 128 quant bytes, is_high_nibble) of weight i."""
    c, l = divmod(i, 64)
    return 32 * c + (l % 32), l >= 32


def make_sb(d: float, dmin: float, sc, m, q) -> bytes:
    """One 144-byte q4_K super-block from d, dmin, 8 scales, 8 mins, 256 nibbles."""
    qs = bytearray(128)
    for i in range(256):
        off, hi = nibble_byte(i)
        qs[off] |= (int(q[i]) & 15) << (4 if hi else 0)
    return f16_bytes(d) + f16_bytes(dmin) + pack_scales(sc, m) + bytes(qs)


def sb_values(d: float, dmin: float, sc, m, q) -> np.ndarray:
    """The 256 weights of make_sb(...) in f64: d*sc_j*q - dmin*m_j, j = i // 32."""
    d, dmin = f16_value(d), f16_value(dmin)
    j = np.arange(256) // 32
    return d * np.asarray(sc, np.float64)[j] * np.asarray(q, np.float64) - dmin * np.asarray(m, np.float64)[j]


def make_q4_0(d: float, q) -> bytes:
    """One 18-byte q4_0 block from d and 32 nibbles: byte i = q_i | q_{16+i} << 4."""
    q = np.asarray(q, np.int64)
    qs = bytes(int(q[i] & 15) | (int(q[16 + i] & 15) << 4) for i in range(16))
    return f16_bytes(d) + qs


def q4_0_values(d: float, q) -> np.ndarray:
    """The 32 weights of make_q4_0(...) in f64: d*(q - 8)."""
    return f16_value(d) * (np.asarray(q, np.float64) - 8.0)


def make_q8(d: float, q) -> bytes:
    """One 34-byte q8_0 block."""
    return f16_bytes(d) + np.asarray(q, np.int8).tobytes()


def q8_values(d: float, q) -> np.ndarray:
    return f16_value(d) * np.asarray(q, np.float64)


class RandomQ4K:
    """A random q4_K matrix with its known scales, mins, nibbles and weights."""

    def __init__(self, rng: np.random.Generator, m: int, k: int, zero_q=False, zero_dmin=False):
        nsb = -(-k // 256)
        self.m, self.k, self.nsb = m, k, nsb
        self.d = rng.uniform(1e-4, 1e-3, (m, nsb))
        self.dmin = np.zeros((m, nsb)) if zero_dmin else rng.uniform(1e-4, 1e-3, (m, nsb))
        self.sc = rng.integers(0, 64, (m, nsb, 8))
        self.mn = rng.integers(0, 64, (m, nsb, 8))
        self.q = np.zeros((m, nsb, 256), np.int64) if zero_q else rng.integers(0, 16, (m, nsb, 256))
        blob = bytearray()
        vals = np.empty((m, nsb * 256))
        for r in range(m):
            for s in range(nsb):
                args = (self.d[r, s], self.dmin[r, s], self.sc[r, s], self.mn[r, s], self.q[r, s])
                blob += make_sb(*args)
                vals[r, 256 * s:256 * (s + 1)] = sb_values(*args)
        self.bytes = np.frombuffer(bytes(blob), np.uint8).reshape(m, nsb * 144)
        self.values = vals                       # [m, nsb*256] f64


class RandomQ8:
    """k values as q8_0 blocks with known scales and codes."""

    def __init__(self, rng: np.random.Generator, k: int, q=None):
        nb = k // 32
        self.d = rng.uniform(1e-3, 1e-1, nb)
        self.q = rng.integers(-127, 128, (nb, 32)) if q is None else np.asarray(q).reshape(nb, 32)
        self.bytes = np.frombuffer(b"".join(make_q8(self.d[b], self.q[b]) for b in range(nb)), np.uint8)
        self.values = np.concatenate([q8_values(self.d[b], self.q[b]) for b in range(nb)])


class RandomQ4_0:
    """A random q4_0 matrix with its known scales, nibbles and weights."""

    def __init__(self, rng: np.random.Generator, m: int, k: int, q_fill=None):
        nb = k // 32
        self.m, self.k, self.nb = m, k, nb
        self.d = rng.uniform(1e-4, 1e-3, (m, nb))
        self.q = rng.integers(0, 16, (m, nb, 32)) if q_fill is None else np.full((m, nb, 32), q_fill, np.int64)
        blob = bytearray()
        vals = np.empty((m, k))
        for r in range(m):
            for b in range(nb):
                blob += make_q4_0(self.d[r, b], self.q[r, b])
                vals[r, 32 * b:32 * (b + 1)] = q4_0_values(self.d[r, b], self.q[r, b])
        self.bytes = np.frombuffer(bytes(blob), np.uint8).reshape(m, nb * 18)
        self.values = vals                       # [m, k] f64
