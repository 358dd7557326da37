"""Host-side checks of the benchmark's bookkeeping (no GPU): the refusal of
more than one GPU, the algorithmic byte counts behind the reported bandwidth
and roofline, and the lookup of stored counter traffic by kernel source hash."""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _layer(**kw):
    base = dict(d=8, d_ffn=32, r=4, kind="reglu", w_dtype="f16", p_dtype="f16")
    base.update(kw)
    return SimpleNamespace(**base)


def test_step_bytes_by_hand():
    # ReGLU fp16, d=8, d_ffn=32, r=4, 5 active rows, B=2:
    # predictor (4*8 + 32*4)*2 + 4*(4 + 32) = 320 + 144 = 464
    # rows 5 * (3*16 + 8) = 280; union mask 32; activations 2*(16+4)*4 = 160
    assert bench.step_bytes([_layer()], [5], 2) == 464 + 280 + 32 + 160
    # ReLU 4-bit rows: a row of d=64 is 2 blocks of 18 bytes; 2 matrices
    L = _layer(kind="relu", w_dtype="q4_0", d=64)
    pred = (4 * 64 + 32 * 4) * 2 + 4 * (4 + 32)
    assert bench.step_bytes([L], [3], 1) == pred + 3 * (2 * 36 + 8) + 32 + (128 + 4) * 4
    # two layers add up
    assert bench.step_bytes([_layer(), _layer()], [5, 0], 2) == \
        bench.step_bytes([_layer()], [5], 2) + bench.step_bytes([_layer()], [0], 2)


def test_dominant_kernel_bytes_by_hand():
    # every W2 row + bias + mask byte: 32 * (4*2 + 4 + 1); 5 active rows of
    # gate + up + down (3 * 16 bytes) + bias + list entry; hid and h read once
    assert bench.dominant_kernel_bytes(_layer(), 5, 1) == \
        32 * 13 + 5 * (3 * 16 + 4 + 8) + (4 + 8) * 4
    # ReLU: up + down rows of 8 fp32 values
    assert bench.dominant_kernel_bytes(_layer(kind="relu", w_dtype="f32"), 2, 1) == \
        32 * 13 + 2 * (2 * 32 + 4 + 8) + (4 + 8) * 4
    # ReLU with 4-bit rows, d = 64: two 18-byte blocks per row
    assert bench.dominant_kernel_bytes(_layer(kind="relu", w_dtype="q4_0", d=64), 3, 1) == \
        32 * 13 + 3 * (2 * 36 + 4 + 8) + (4 + 64) * 4


def test_batched_ffn_bytes_by_hand():
    # 7 listed rows of 3 fp16 matrices + bias + index; B=4 tokens: input, residual in/out
    assert bench.batched_ffn_bytes(_layer(), 7, 4) == 7 * (3 * 16 + 8) + 4 * 3 * 8 * 4


def test_dense_step_bytes_by_hand():
    assert bench.dense_step_bytes([_layer()], 1) == 32 * (3 * 16 + 4) + 2 * 8 * 4


def test_traffic_record_lookup(tmp_path, monkeypatch):
    good = dict(kernel="k", workload="w", batch=1, bytes_per_launch=123,
                source_sha256=bench.kernel_source_hash())
    stale = dict(good, workload="w2", source_sha256="0" * 64)
    f = tmp_path / "traffic.md"
    f.write_text("notes\ntraffic_record: " + json.dumps(good) + "\n"
                 "traffic_record: " + json.dumps(stale) + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(f))
    assert bench.measured_traffic("w", 1)["bytes_per_launch"] == 123
    assert bench.measured_traffic("w", 4) is None        # other batch
    assert bench.measured_traffic("w2", 1) is None       # kernel changed since
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("w", 1) is None


def test_source_hash_ignores_comments_only():
    a = "int f(int x) {  // add one\n  return x + 1; /* done */ }\n"
    b = "int f(int x){return x+1;}"
    c = "int f(int x){return x+2;}"
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(b) != bench.code_only(c)


def test_cpu_baseline_pins_one_core_and_restores_affinity():
    from workloads import TINY, make_layer, make_tokens
    keep = [make_layer(TINY, l, seed=0, n_cal=256) for l in range(TINY.layers)]
    X = make_tokens(TINY.d, TINY.tokens, 1, seed=0)
    before = os.sched_getaffinity(0)
    out = bench.cpu_baseline(TINY, keep, X, 1, TINY.layers)
    assert os.sched_getaffinity(0) == before
    assert out["cores"] == 1 and out["kind"] == "oracle"
    assert out["host_nproc"] == os.cpu_count()
    assert out["value"] > 0 and out["dense_tokens_per_s"] > 0
    assert isinstance(out["cpu_model"], str) and out["cpu_model"]
    assert "16 steps" in out["sample"] and "2 of 2 layers" in out["sample"]


def test_fp8_predictor_bytes_by_hand():
    # fp8 predictor: one byte per weight plus a 4-byte scale per row
    L = _layer(p_dtype="fp8")
    pred = (4 * 8 + 32 * 4) * 1 + (4 + 4) * (4 + 32)
    assert bench.step_bytes([L], [5], 2) == pred + 280 + 32 + 160
    assert bench.dominant_kernel_bytes(L, 5, 1) == \
        32 * (4 + 4 + 4 + 1) + 5 * (3 * 16 + 4 + 8) + (4 + 8) * 4


def test_dense_prefix_bytes_by_hand():
    # 6 always-active neurons: their W2 rows, b2 entries are not read (mask
    # bytes still are); the rest as before
    L = _layer(dense_prefix=6)
    pred = (4 * 8 + 26 * 4) * 2 + 4 * (4 + 26)
    assert bench.step_bytes([L], [5], 2) == pred + 280 + 32 + 160
    assert bench.dominant_kernel_bytes(L, 5, 1) == \
        26 * (4 * 2 + 4) + 32 + 5 * (3 * 16 + 4 + 8) + (4 + 8) * 4
