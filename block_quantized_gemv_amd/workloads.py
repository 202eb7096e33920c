"""The synthetic decode workloads: shapes, seeds and byte counts.

Shapes follow the decode steps the pages measure: a 0.5B-class and a
7B-class Qwen2-style model ('07 · R3 — Small-model per-token overhead',
§1 and §5; '04 · 8o — Killing the CPU stall at decode start', §1), each
GEMV at n=1 with q4_K weights and a q8_0 lm_head; plus a small-batch
variant and a routed-expert FFN.
"""
from __future__ import annotations

from dataclasses import dataclass

Q4K_BYTES_PER_WEIGHT = 144 / 256
Q8_BYTES_PER_VALUE = 34 / 32


def q4k_bytes(m: int, k: int) -> int:
    return m * (-(-k // 256)) * 144


def q8_bytes(m: int, k: int) -> int:
    return m * (k // 32) * 34


def q4_0_bytes(m: int, k: int) -> int:
    return m * (k // 32) * 18


@dataclass(frozen=True)
class SingleGemv:
    name: str = "q4_K x q8_0 GEMV 1024x1024"
    m: int = 1024
    k: int = 1024
    seed: int = 0

    def algorithmic_bytes(self) -> int:
        return q4k_bytes(self.m, self.k) + q8_bytes(1, self.k) + 4 * self.m


@dataclass(frozen=True)
class DecodeModel:
    name: str
    hidden: int
    n_layers: int
    qkv_rows: int
    inter: int
    vocab: int
    seed: int
    eps: float = 1e-6
    weight_format: str = "q4_K"      # layer matrices: "q4_K" or "q4_0"
    o_k: int = 0                     # O's K, the first o_k QKV outputs (0: hidden)

    @property
    def o_in(self) -> int:
        return self.o_k or self.hidden

    def layer_shapes(self):
        """(rows, k) of the four 4-bit GEMVs of one layer, in step order."""
        return [(self.qkv_rows, self.hidden), (self.hidden, self.o_in),
                (2 * self.inter, self.hidden), (self.hidden, self.inter)]

    def layer_matrix_bytes(self, m: int, k: int) -> int:
        return q4_0_bytes(m, k) if self.weight_format == "q4_0" else q4k_bytes(m, k)

    def weight_bytes(self) -> int:
        per_layer = sum(self.layer_matrix_bytes(m, k) for m, k in self.layer_shapes())
        return self.n_layers * per_layer + q8_bytes(self.vocab, self.hidden)

    def algorithmic_bytes(self) -> int:
        """Weights + q8_0 activations read + f32 outputs written, per step."""
        acts = 0
        for m, k in self.layer_shapes():
            acts += q8_bytes(1, k) + 4 * m
        acts *= self.n_layers
        acts += q8_bytes(1, self.hidden) + 4 * self.vocab
        return self.weight_bytes() + acts


DECODE_05B = DecodeModel("0.5B-class decode step (hidden 1024, 24 layers, q8_0 lm_head 151552x1024)",
                         hidden=1024, n_layers=24, qkv_rows=1280, inter=4864, vocab=151552, seed=1)
# The format of the 0.5B model the pages measure ('07 · R3', §5: 0.5B q4_0).
DECODE_05B_Q4_0 = DecodeModel("0.5B-class decode step, q4_0 layer weights (hidden 1024, 24 layers, "
                              "q8_0 lm_head 151552x1024)",
                              hidden=1024, n_layers=24, qkv_rows=1280, inter=4864, vocab=151552, seed=5,
                              weight_format="q4_0")
DECODE_7B = DecodeModel("7B-class decode step (hidden 3584, 28 layers, q8_0 lm_head 152064x3584)",
                        hidden=3584, n_layers=28, qkv_rows=4608, inter=18944, vocab=152064, seed=2)
# One rank of the 7B-class step split eight ways (tensor-parallel, the
# collectives left out): QKV and gate/up split by rows, O and down by K on
# super-block boundaries, the lm_head by vocabulary rows.  O's 14 and down's
# 74 super-blocks of K do not divide by 8, so ranks take 2 or 1 and 10 or 9;
# this is the largest rank (O K = 512, down K = 2560, so gate/up 2 x 2560
# rows), whose step bounds the split step.
DECODE_7B_TP8 = DecodeModel("7B-class decode step, largest of 8 tensor-parallel ranks (QKV 576x3584, "
                            "O 3584x512, gate/up 5120x3584, down 3584x2560, q8_0 lm_head 19008x3584; "
                            "collectives not run)",
                            hidden=3584, n_layers=28, qkv_rows=576, inter=2560, vocab=19008, seed=6, o_k=512)


@dataclass(frozen=True)
class Batched:
    name: str = "7B-class shapes, n in {2,4,8} activation columns"
    seed: int = 3
    ns: tuple = (2, 4, 8)
    shapes: tuple = ((4608, 3584), (3584, 3584), (37888, 3584), (3584, 18944))


@dataclass(frozen=True)
class MoE:
    name: str = "routed expert FFN, 64 experts, top-8, hidden 2048, expert inter 1408"
    seed: int = 4
    n_experts: int = 64
    n_sel: int = 8
    hidden: int = 2048
    inter: int = 1408
    n_tokens: int = 1000

    @property
    def k_pad(self) -> int:
        """Down-projection K padded up to whole 256-weight super-blocks."""
        return -(-self.inter // 256) * 256

    def gate_up_bytes(self) -> int:
        return q4k_bytes(2 * self.inter, self.hidden)

    def down_bytes(self) -> int:
        return q4k_bytes(self.hidden, self.k_pad)

    def token_weight_bytes(self) -> int:
        return self.n_sel * (self.gate_up_bytes() + self.down_bytes())


SINGLE = SingleGemv()
BATCHED = Batched()
MOE = MoE()
