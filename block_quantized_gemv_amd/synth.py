"""Seeded synthetic inputs for the q4_K x q8_0 decode path.

This module draws bytes and floats and lays them out in the storage formats;
it holds none of the method's arithmetic (no scale decode, no quantization,
no dot products).  Both the HIP path and the reference oracle consume the
buffers it returns, so the two never share anything but their inputs.

Every tensor comes from its own numpy PCG64 stream keyed by
(workload seed, tensor key), so any tensor can be regenerated alone.

Distributions (the synthetic stand-in for trained weights):

* q4_K super-block (144 B): bytes 0-1 f16 ``d`` and 2-3 f16 ``dmin``, each a
  real uniform draw in [1e-4, 1e-3] rounded to f16 by numpy (round to
  nearest even); bytes 4-15 are 12 uniform random bytes and bytes 16-143 are
  128 uniform random bytes.  The 12 scale bytes hold sixteen 6-bit fields
  (8 scales, 8 mins) that use every one of the 96 bits exactly once, so
  uniform bytes give independent uniform 0..63 scales and mins without this
  module knowing the packing; likewise every nibble is uniform 0..15.
* q8_0 weight block (34 B): f16 ``d`` uniform in [1e-4, 1e-3], then 32 int8
  values uniform in -127..127.
* q4_0 weight block (18 B): f16 ``d`` uniform in [1e-4, 1e-3], then 16
  uniform random bytes (32 uniform nibbles).
* activations: N(0, 1) drawn in f64 and rounded to f32.
* routing: ``n_sel`` distinct expert ids drawn uniformly without
  replacement, and N(0, 1) router logits.
"""
from __future__ import annotations

import numpy as np

Q4K_BLOCK_BYTES = 144   # bytes per q4_K super-block of 256 weights
Q4K_BLOCK_VALUES = 256
Q8_BLOCK_BYTES = 34     # bytes per q8_0 block of 32 values
Q4_0_BLOCK_BYTES = 18   # bytes per q4_0 block of 32 weights
Q8_BLOCK_VALUES = 32

# Tensor keys: the first element says what the tensor is.
KEY_LAYER = 1        # (KEY_LAYER, layer, kind) kind: 0 qkv, 1 o, 2 gate/up, 3 down
KEY_LM_HEAD = 2
KEY_STEP_INPUTS = 3
KEY_EXPERT = 4       # (KEY_EXPERT, expert, 0 gate/up | 1 down)
KEY_ROUTE_IDS = 5
KEY_ROUTE_LOGITS = 6
KEY_TOKEN_X = 7
KEY_COLUMNS = 8
KEY_MATRIX = 9


def rng(seed: int, *key: int) -> np.random.Generator:
    """Independent PCG64 stream for tensor ``key`` of workload ``seed``."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, key)])))


def _uniform_f16(g: np.random.Generator, shape) -> np.ndarray:
    return g.uniform(1e-4, 1e-3, size=shape).astype(np.float16)


def q4k_matrix(seed: int, key: tuple, m: int, k: int) -> np.ndarray:
    """``m`` rows of ceil(k/256) q4_K super-blocks, uint8 ``[m, nsb*144]``."""
    nsb = -(-k // Q4K_BLOCK_VALUES)
    g = rng(seed, *key)
    raw = np.frombuffer(g.bytes(m * nsb * Q4K_BLOCK_BYTES), dtype=np.uint8)
    out = raw.reshape(m, nsb, Q4K_BLOCK_BYTES).copy()
    dd = _uniform_f16(g, (m, nsb, 2))          # [..., 0] = d, [..., 1] = dmin
    out[:, :, 0:4] = dd.view(np.uint8).reshape(m, nsb, 4)
    return out.reshape(m, nsb * Q4K_BLOCK_BYTES)


def q8_0_matrix(seed: int, key: tuple, m: int, k: int) -> np.ndarray:
    """``m`` rows of k/32 q8_0 blocks, uint8 ``[m, (k/32)*34]``."""
    assert k % Q8_BLOCK_VALUES == 0
    nb = k // Q8_BLOCK_VALUES
    g = rng(seed, *key)
    q = g.integers(-127, 128, size=(m, nb, Q8_BLOCK_VALUES), dtype=np.int8)
    d = _uniform_f16(g, (m, nb))
    out = np.empty((m, nb, Q8_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d.view(np.uint8).reshape(m, nb, 2)
    out[:, :, 2:] = q.view(np.uint8)
    return out.reshape(m, nb * Q8_BLOCK_BYTES)


def q4_0_matrix(seed: int, key: tuple, m: int, k: int) -> np.ndarray:
    """``m`` rows of k/32 q4_0 blocks, uint8 ``[m, (k/32)*18]``."""
    assert k % Q8_BLOCK_VALUES == 0
    nb = k // Q8_BLOCK_VALUES
    g = rng(seed, *key)
    raw = np.frombuffer(g.bytes(m * nb * Q4_0_BLOCK_BYTES), dtype=np.uint8)
    out = raw.reshape(m, nb, Q4_0_BLOCK_BYTES).copy()
    out[:, :, 0:2] = _uniform_f16(g, (m, nb)).view(np.uint8).reshape(m, nb, 2)
    return out.reshape(m, nb * Q4_0_BLOCK_BYTES)


def normal_f32(seed: int, key: tuple, shape) -> np.ndarray:
    """N(0, 1) values drawn in f64, rounded to f32."""
    return rng(seed, *key).standard_normal(size=shape).astype(np.float32)


def routing(seed: int, n_tokens: int, n_experts: int, n_sel: int):
    """Per token: ``n_sel`` distinct ids (int32) and N(0,1) logits (f32)."""
    g = rng(seed, KEY_ROUTE_IDS)
    ids = np.stack([g.choice(n_experts, size=n_sel, replace=False) for _ in range(n_tokens)])
    logits = normal_f32(seed, (KEY_ROUTE_LOGITS,), (n_tokens, n_sel))
    return ids.astype(np.int32), logits
