"""bench.py's host-side arithmetic and contract, on the CPU: the algorithmic
bytes and flops behind every roofline fraction, the decode-chunk workloads,
the kernel-source hash that gates the committed traffic figures, and the
single-GPU exit."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from routed_expert_prefill_amd import synth  # noqa: E402


def _wl(**kw):
    base = dict(name="t", T=4, d=256, f=128, E=4, k=2, x_std=1.0, w_std=0.02, mask_p=0.0,
                routing="softmax", dtype="bf16")
    base.update(kw)
    return synth.Workload(**base)


def test_work_of_a_hand_counted_case():
    """T = 4 tokens, top-2, 4 experts of which two receive 3 and 2 rows,
    d = 256, f = 128, bf16: every term counted by hand."""
    wl = _wl()
    w = bench.algorithmic_work(wl, [3, 0, 2, 0], wl.T)
    d, f = 256, 128
    assert w["R_act"] == 5 and w["experts_used"] == 2
    gate_up = 2 * (2 * f * d * 2)  # two experts' gate and up matrices, bf16
    gate_up += 4 * d * 2  # x once
    gate_up += 4 * 5  # the sorted route of each active row
    gate_up += 5 * f * 2  # h written
    assert w["stage_bytes"]["gate_up"] == gate_up
    assert w["stage_bytes"]["down"] == 2 * (d * f * 2) + 5 * f * 2 + 5 * d * 4
    assert w["stage_bytes"]["combine"] == 5 * d * 4 + 4 * d * 4
    assert w["stage_bytes"]["route"] == 30 * 8
    assert w["gate_up_flops"] == 2 * 2 * d * f * 5  # two products of 2 d f flops per row
    assert w["path_flops"] == w["gate_up_flops"] * 1.5
    assert w["path_bytes"] == sum(w["stage_bytes"].values())


def test_work_scales_with_used_experts_and_weight_width():
    wl = _wl()
    one = bench.algorithmic_work(wl, [4, 0, 0, 0], wl.T)
    two = bench.algorithmic_work(wl, [2, 2, 0, 0], wl.T)
    # same rows, one more expert's weights: exactly one expert's gate/up matrices more
    assert two["gate_up_bytes"] - one["gate_up_bytes"] == 2 * wl.f * wl.d * 2
    assert two["gate_up_flops"] == one["gate_up_flops"]
    fp8 = bench.algorithmic_work(_wl(dtype="fp8"), [2, 2, 0, 0], wl.T)
    scales = 4 * (wl.f // 128) * (wl.d // 128)
    # one-byte codes plus one fp32 scale per 128 x 128 block
    w_bf16 = 2 * 2 * (2 * wl.f * wl.d)
    w_fp8 = 2 * 2 * (wl.f * wl.d + scales)
    # and x read as codes (one byte) plus one fp32 scale per token
    assert fp8["gate_up_bytes"] - w_fp8 == two["gate_up_bytes"] - w_bf16 - wl.T * wl.d + 4 * wl.T
    assert fp8["gate_up_flops"] == two["gate_up_flops"]


def test_headline_bytes_match_the_weights_it_streams():
    """At 401 tokens every expert is used; the gate/up bytes are the whole
    gate and up weight set plus a few MB of activations."""
    wl = synth.WORKLOADS["prefill_T401_uniform_bf16"]
    counts = [9] * 256  # any histogram that uses all 256 experts
    w = bench.algorithmic_work(wl, counts, wl.T)
    weights = 256 * 2 * wl.f * wl.d * 2
    assert weights <= w["gate_up_bytes"] <= weights + 20e6


def test_chunk_workload():
    wl = bench.chunk_workload("prefill_T401_uniform_bf16", 3)
    base = synth.WORKLOADS["prefill_T401_uniform_bf16"]
    assert wl.T == 3 and (wl.d, wl.f, wl.E, wl.k) == (base.d, base.f, base.E, base.k)
    assert wl.name == "chunk_T3_d4096_f2048_E256_softmax_bf16"


def test_source_hash_ignores_comments_only(tmp_path):
    for p in bench.KERNEL_SOURCES:
        dst = tmp_path / p
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, p), dst)
    h0 = bench.source_hash(str(tmp_path))
    assert h0 == bench.source_hash()
    first = tmp_path / bench.KERNEL_SOURCES[0]
    first.write_text(first.read_text() + "\n// a comment\n\n")
    assert bench.source_hash(str(tmp_path)) == h0
    first.write_text(first.read_text() + "\nstatic int moe_unused_symbol;\n")
    assert bench.source_hash(str(tmp_path)) != h0


def test_median():
    assert bench.med([3, 1, 2]) == 2
    assert bench.med([4, 1, 2, 3]) == 2.5


def test_more_than_one_gpu_exits_with_a_message():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""
