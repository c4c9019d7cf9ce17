"""Host logic of bench.py (no GPU): the algorithmic FLOP and byte models of
the workloads, the roofline bound chosen from the arithmetic intensity, the
profiler-traffic lookup that is dropped once a kernel source changes, and
the refusal of more than one GPU.

The FLOP model counts two matrix products of 2 FLOPs per multiply-add over
the visible (query, key) pairs only ("Transformer" (ai-notes) -- Discussion
(Compute): B h T^2 d_head multiplies per product, halved by the causal
mask); the byte model reads q, k, v and writes o once."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from transformer_causal_self_amd import workloads as wl  # noqa: E402


def brute_visible(Tq, Tk, causal, q_offset):
    return sum(1 for i in range(Tq) for j in range(Tk) if not causal or j <= q_offset + i)


@pytest.mark.parametrize("Tq,Tk,causal,qo", [
    (1, 1, True, 0), (7, 7, True, 0), (5, 9, True, 4), (9, 5, True, 0),
    (4, 30, True, 100), (6, 11, False, 0), (13, 13, True, 3),
])
def test_visible_pairs_match_brute_force(Tq, Tk, causal, qo):
    assert bench.n_visible(Tq, Tk, causal, qo) == brute_visible(Tq, Tk, causal, qo)


# per-configuration figures: T (T + 1) / 2 visible pairs per (batch, head) for
# a causal self-attention of T tokens, 4 d FLOPs per pair; bytes of q, k, v, o
@pytest.mark.parametrize("key,flops,nbytes", [
    (1, 4 * 1 * 4 * 64 * (128 * 129 // 2), 4 * 64 * (2 * 4 * 128 + 2 * 4 * 128)),
    (2, 4 * 8 * 12 * 64 * (1024 * 1025 // 2), 2 * 64 * (2 * 8 * 12 * 1024 + 2 * 8 * 12 * 1024)),
    (3, 4 * 2 * 32 * 128 * (4096 * 4097 // 2), 2 * 128 * (2 * 2 * 32 * 4096 + 2 * 2 * 8 * 4096)),
    (4, 4 * 1 * 32 * 128 * (16384 * 16385 // 2), 2 * 128 * (2 * 32 * 16384 + 2 * 8 * 16384)),
    (5, 4 * 32 * 32 * 128 * 8192, 2 * 128 * (2 * 32 * 32 * 1 + 2 * 32 * 8 * 8192)),
])
def test_workload_flop_and_byte_models(key, flops, nbytes):
    w = wl.WORKLOADS[key]
    assert bench.attn_flops(w) == pytest.approx(flops, rel=0, abs=0.5)
    assert bench.attn_bytes(w) == pytest.approx(nbytes, rel=0, abs=0.5)


def test_roofline_bound_follows_the_ridge():
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    assert bench.RIDGE == pytest.approx(ridge)
    # the d = 64 MHA prefill sits below the ridge (256 FLOP/B): HBM-bound
    w2 = wl.WORKLOADS[2]
    r = bench.roofline(bench.attn_flops(w2), bench.attn_bytes(w2), 0.0206, "bf16", 0.0206)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == bench.PEAK_HBM_GBS
    assert r["frac"] == pytest.approx(bench.attn_bytes(w2) / 20.6e-6 / 1e9 / bench.PEAK_HBM_GBS)
    assert r["frac_of_mfma_peak"] == pytest.approx(bench.attn_flops(w2) / 20.6e-6 / 1e12 / bench.PEAK_BF16_TFLOPS)
    # the long-context prefill is far above it: matrix-core bound
    w4 = wl.WORKLOADS[4]
    r = bench.roofline(bench.attn_flops(w4), bench.attn_bytes(w4), 1.8, "bf16", 1.9)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["frac"] == pytest.approx(bench.attn_flops(w4) / 1.8e-3 / 1e12 / bench.PEAK_BF16_TFLOPS)
    assert r["frac_median"] == pytest.approx(r["frac"] * 1.8 / 1.9)
    # decode: 4 FLOP/B, HBM-bound; float32: the vector ALU peak
    w5 = wl.WORKLOADS[5]
    assert bench.roofline(bench.attn_flops(w5), bench.attn_bytes(w5), 0.17, "bf16")["bound"] == "hbm"
    w1 = wl.WORKLOADS[1]
    r = bench.roofline(bench.attn_flops(w1), bench.attn_bytes(w1), 0.017, "f32")
    assert r["bound"] == "alu" and r["peak"] == bench.PEAK_F32_TFLOPS


def test_traffic_is_dropped_when_the_kernel_source_changed(tmp_path, monkeypatch):
    w = wl.WORKLOADS[5]
    good = bench.source_hash("decode_bf16")
    f = tmp_path / "hbm_traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    f.write_text(json.dumps({f"decode_bf16:{w.name}": {"bytes_per_launch": 123.0, "source_sha256_16": good}}))
    assert bench.measured_traffic("decode_bf16", w.name) == 123.0
    f.write_text(json.dumps({f"decode_bf16:{w.name}": {"bytes_per_launch": 123.0, "source_sha256_16": "0" * 16}}))
    assert bench.measured_traffic("decode_bf16", w.name) is None
    assert bench.measured_traffic("decode_bf16", "no_such_workload") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("decode_bf16", w.name) is None


def test_committed_traffic_matches_the_current_sources():
    """Every entry of profiles/hbm_traffic.json was taken on the kernel
    source now in the tree (else bench.py would report null traffic)."""
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    for key, entry in rec.items():
        kernel = key.split(":")[0]
        assert entry["source_sha256_16"] == bench.source_hash(kernel), key


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _file_hash(rel):
    import hashlib
    with open(os.path.join(ROOT, "transformer_causal_self_amd", "csrc", rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


# each kernel-trace summary under profiles/ names the hash of the sources it was
# profiled on; the summary is stale (and must be taken again) once they change
PROFILE_SOURCES = {
    "attn_bwd_bf16_workloads2_3.txt": lambda: [_file_hash("attn_bwd_bf16.hip")],
    "decode_split_bf16_d128_B32_Hq32_Hkv8_Tk8192.txt": lambda: [_file_hash("attn_decode_bf16.hip")],
    "prefill_bf16_d128_gqa_B2_Hq32_Hkv8_T4096.txt": lambda: [bench.source_hash("prefill_bf16_d128")],
    "prefill_bf16_d64_mha_B8_H12_T1024.txt": lambda: [bench.source_hash("prefill_bf16_d64")],
    "prefill_bf16_d128_gqa_B1_Hq32_Hkv8_T16384.txt": lambda: [bench.source_hash("prefill_bf16_d128"),
                                                              bench.source_hash("attn_fwd_rope_bf16_d128")],
    "rope_bf16_d128_workloads3_4.txt": lambda: [_file_hash("rope.hip")],
    "cached_steps_bf16_d128.txt": lambda: [_file_hash("attn_decode_bf16.hip"), _file_hash("attn_prefill_bf16.hip"),
                                           _file_hash("rope.hip")],
}


@pytest.mark.parametrize("name", sorted(PROFILE_SOURCES))
def test_profile_summaries_were_taken_on_the_current_sources(name):
    import re
    with open(os.path.join(ROOT, "profiles", name)) as f:
        text = f.read()
    line = next(l for l in text.splitlines() if "sha256[:16] at profiling time" in l)
    recorded = re.findall(r"\b[0-9a-f]{16}\b", line)
    assert recorded == PROFILE_SOURCES[name](), (name, line)
