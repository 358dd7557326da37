"""Edge cases of the decode step on the GPU: a neuron count that leaves the
single-token kernel's last row group partly empty, one that fills its
down-projection chunks to capacity with a ragged last chunk, and the two degenerate
predictors -- every neuron active (the step equals the dense step) and none
active (the residual passes through unchanged, bit for bit)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import activation_sparse_mlp_amd as spffn
from tests.gpu_helpers import DEV, gpu_layer
from tests.test_gpu_kernels import _decode_checks
from workloads import TINY, make_layer, make_tokens

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _ragged(kind):
    # fp16 rows, d_ffn = 1003: 8-row groups, the last one has 3 rows
    return replace(TINY, kind=kind, w_dtype="f16", p_dtype="f16", d=256, d_ffn=1003, r=64)


@pytest.mark.parametrize("kind", ["reglu", "relu"])
@pytest.mark.parametrize("B", [1, 3])
def test_decode_ragged_row_groups(kind, B):
    print(f"edge decode ragged {kind} B={B}", flush=True)
    _decode_checks(_ragged(kind), B, 2, seed=51)


def test_decode_most_groups_per_chunk():
    # d_ffn = 65603: 8201 row groups of 8, so the single-token layer kernel uses
    # 129 down-projection chunks of 64 groups (the most a chunk's list holds)
    # and a last chunk of 9 groups
    print("edge decode 8201 row groups", flush=True)
    _decode_checks(replace(_ragged("relu"), d_ffn=65603), 1, 2, seed=53)


def test_layer_kernel_wait_gives_up_with_nan():
    # the single-token layer kernel's down-projection workgroups wait (bounded)
    # for their chunk's row groups; with a limit of 0 polls every one of them
    # gives up at once, and the step must complete with NaN rather than hang
    cfg = _ragged("relu")
    model = _model(cfg, tau=0.5)
    x = make_tokens(cfg.d, 1, 1, seed=5, device=DEV)[0]
    ref = spffn.decode_step(model, x)
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    try:
        spffn.set_wait_limit(0)
        h = spffn.decode_step(model, x)
        torch.cuda.synchronize()
    finally:
        spffn.set_wait_limit(spffn.WAIT_LIMIT_DEFAULT)
    assert torch.isnan(h).all()
    again = spffn.decode_step(model, x)
    torch.cuda.synchronize()
    assert torch.equal(again, ref)  # bitwise: fixed summation order


def _model(cfg, tau, layers=2):
    ws = [make_layer(replace(cfg, tau=tau), l, seed=7, n_cal=512) for l in range(layers)]
    return spffn.Model([gpu_layer(w) for w in ws], rms_eps=1e-5)


@pytest.mark.parametrize("B", [1, 4])
def test_every_neuron_active_equals_dense(B):
    cfg = _ragged("reglu")
    model = _model(cfg, tau=1e-6)  # logit threshold about -13.8: every neuron passes
    x = make_tokens(cfg.d, 1, B, seed=3, device=DEV)[0]
    counts = torch.empty(2, dtype=torch.int32, device=DEV)
    h = spffn.decode_step(model, x, layer_counts=counts)
    hd = spffn.decode_step(model, x, dense=True)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), [cfg.d_ffn, cfg.d_ffn])
    rel = float((h - hd).norm() / hd.norm())
    assert rel < 1e-5, rel  # same sums; only the order of the per-neuron terms differs


@pytest.mark.parametrize("B", [1, 4])
def test_no_neuron_active_keeps_residual(B):
    cfg = _ragged("relu")
    model = _model(cfg, tau=1.0 - 1e-6)  # threshold about +13.8: no neuron passes
    x = make_tokens(cfg.d, 1, B, seed=4, device=DEV)[0]
    counts = torch.full((2,), -1, dtype=torch.int32, device=DEV)
    h = spffn.decode_step(model, x, layer_counts=counts)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), [0, 0])
    assert torch.equal(h, x)
