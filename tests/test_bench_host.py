"""Host-side logic of bench.py, on the CPU: the algorithmic bytes that the
roofline divides by, the lookup of the committed HBM-traffic record, and the
refusal of more than one GPU.

The per-matrix weight bytes are the figures of the q4_K / q8_0 formats
(144 bytes per 256 weights, 34 bytes per 32) worked out independently for the
two decode steps: 7B-class layer QKV 9,289,728, O 7,225,344, gate/up
76,382,208, down 38,191,104 and lm_head 579,059,712 bytes, 4,249,534,464
weight bytes per step; 0.5B-class 737,280 / 589,824 / 5,603,328 / 2,801,664,
lm_head 164,888,576, 398,458,880 per step; the largest of eight tensor-parallel
ranks of the 7B-class step (QKV 576x3584, O 3584x512, gate/up 5120x3584, down
3584x2560, lm_head 19008x3584) 1,161,216 / 1,032,192 / 10,321,920 / 5,160,960,
lm_head 72,382,464, 567,318,528 per step."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_quantized_gemv_amd import workloads  # noqa: E402

WEIGHTS = {
    "7b": (workloads.DECODE_7B, [9_289_728, 7_225_344, 76_382_208, 38_191_104], 579_059_712, 4_249_534_464),
    "05b": (workloads.DECODE_05B, [737_280, 589_824, 5_603_328, 2_801_664], 164_888_576, 398_458_880),
    "tp8": (workloads.DECODE_7B_TP8, [1_161_216, 1_032_192, 10_321_920, 5_160_960], 72_382_464, 567_318_528),
}


@pytest.mark.parametrize("name", sorted(WEIGHTS))
def test_weight_bytes(name):
    model, layer, lm, step = WEIGHTS[name]
    assert [model.layer_matrix_bytes(m, k) for m, k in model.layer_shapes()] == layer
    assert workloads.q8_bytes(model.vocab, model.hidden) == lm
    assert model.weight_bytes() == step


def test_kernel_bytes_7b():
    """Bytes per launch of each GEMV of the 7B step: weights, the activation
    as the kernel reads it (f32 where its prologue forms Q8(RMSNorm(x)), q8_0
    otherwise) and the output it writes (f32, or q8_0 after SwiGLU)."""
    H, Q, I, V = 3584, 4608, 18944, 152064
    want = {
        "qkv": 9_289_728 + 4 * H + 4 * Q,
        "o": 7_225_344 + 4 * H + 4 * H,
        "gate/up": 76_382_208 + 4 * H + (I // 32) * 34,
        "down": 38_191_104 + (I // 32) * 34 + 4 * H,
        "lm_head": 579_059_712 + 4 * H + 4 * V,
    }
    got = {name: nbytes for name, _, nbytes in bench.gemv_kinds(workloads.DECODE_7B)}
    assert got == want
    assert want["gate/up"] == 76_416_672       # the dominant kernel's bytes per launch


def test_kernel_bytes_tp8_rank():
    """The largest tensor-parallel rank's GEMVs: O reads its 512-wide f32 slice
    of the QKV output and a 3584x512 matrix; down reads the 2560-value q8_0
    SwiGLU vector (80 blocks of 34 bytes)."""
    H = 3584
    want = {
        "qkv": 1_161_216 + 4 * H + 4 * 576,
        "o": 1_032_192 + 4 * 512 + 4 * H,
        "gate/up": 10_321_920 + 4 * H + 80 * 34,
        "down": 5_160_960 + 80 * 34 + 4 * H,
        "lm_head": 72_382_464 + 4 * H + 4 * 19008,
    }
    got = {name: nbytes for name, _, nbytes in bench.gemv_kinds(workloads.DECODE_7B_TP8)}
    assert got == want


def _record(path, kernel, workload, digest, value=79_648_254):
    path.write_text(
        "# a counter record\n\n"
        f"workload: {workload}\n"
        f"dominant_kernel: {kernel}\n"
        f"traffic_bytes_per_launch: {value}\n"
        "kernel_sources: block_quantized_gemv_amd/csrc/gemv_q4k.hip block_quantized_gemv_amd/csrc/common.hpp\n"
        f"kernel_sources_sha256_16: {digest}\n")


def test_traffic_record_lookup(tmp_path, monkeypatch):
    """The record's value is used only for its kernel and workload, and only
    while the listed sources hash to the recorded digest."""
    h = hashlib.sha256()
    for f in ("block_quantized_gemv_amd/csrc/gemv_q4k.hip", "block_quantized_gemv_amd/csrc/common.hpp"):
        h.update(open(os.path.join(ROOT, f), "rb").read())
    digest = h.hexdigest()[:16]
    kernel, wl = "mq::k_gemv_q4k_swiglu<0,true,false>", workloads.DECODE_7B.name
    rec = tmp_path / "record.txt"
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(rec))
    _record(rec, kernel, wl, digest)
    assert bench.measured_traffic(kernel, wl) == 79_648_254
    assert bench.measured_traffic("mq::k_gemv_q4k<0,1,false,1,false>", wl) is None
    assert bench.measured_traffic(kernel, workloads.DECODE_05B.name) is None
    _record(rec, kernel, wl, "0" * 16)
    assert bench.measured_traffic(kernel, wl) is None
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic(kernel, wl) is None


def test_committed_record_is_for_the_dominant_kernel():
    rec = dict(ln.split(": ", 1) for ln in open(bench.TRAFFIC_RECORD).read().splitlines() if ": " in ln)
    kernels = {k for _, k, _ in bench.gemv_kinds(workloads.DECODE_7B)}
    assert rec["dominant_kernel"].strip() in kernels
    assert rec["workload"].strip() == workloads.DECODE_7B.name
    assert int(float(rec["traffic_bytes_per_launch"])) > 76_416_672


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
