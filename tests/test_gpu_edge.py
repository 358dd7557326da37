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
    # fp16 rows, d_ffn = 1003: 4-row groups (one pass), the last one has 3 rows
    return replace(TINY, kind=kind, w_dtype="f16", p_dtype="f16", d=256, d_ffn=1003, r=64)


@pytest.mark.parametrize("kind", ["reglu", "relu"])
@pytest.mark.parametrize("B", [1, 3])
def test_decode_ragged_row_groups(kind, B):
    print(f"edge decode ragged {kind} B={B}", flush=True)
    _decode_checks(_ragged(kind), B, 2, seed=51)


def test_decode_most_groups_per_chunk():
    # d_ffn = 170003: row groups of 64 rows (the most a group has), 2657 of
    # them with a last group of 19 rows, so the single-token layer kernel's
    # 133 down-projection chunks hold 20 groups each (1280 list slots, the
    # most a chunk's list holds) and the last chunk 17 groups
    print("edge decode 2657 row groups of 64", flush=True)
    _decode_checks(replace(_ragged("relu"), d_ffn=170003), 1, 2, seed=53)


def test_layer_kernel_wait_gives_up_with_nan():
    # the single-token layer kernel's down-projection workgroups wait (bounded)
    # for their chunk's row groups; with a limit of 0 polls every one of them
    # gives up at once, and the step must complete with NaN rather than hang
    # and count every give-up in the workspace status word
    cfg = _ragged("relu")
    model = _model(cfg, tau=0.5)
    ws = model.workspace(1)  # status cleared
    x = make_tokens(cfg.d, 1, 1, seed=5, device=DEV)[0]
    ref = spffn.decode_step(model, x, ws=ws)
    assert int(spffn.workspace_status(ws)) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    counts = torch.full((2,), -1, dtype=torch.int32, device=DEV)
    try:
        spffn.set_wait_limit(0)
        h = spffn.decode_step(model, x, layer_counts=counts, ws=ws)
        torch.cuda.synchronize()
    finally:
        spffn.set_wait_limit(spffn.WAIT_LIMIT_DEFAULT)
    assert torch.isnan(h).all()
    gave_up = int(spffn.workspace_status(ws))
    assert gave_up > 0  # every down-projection workgroup of both layers
    assert np.array_equal(counts.cpu().numpy(), [0, 0])  # no chunk listed rows
    # the count accumulates until cleared
    again = spffn.decode_step(model, x, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(again, ref)  # bitwise: fixed summation order
    assert int(spffn.workspace_status(ws)) == gave_up
    spffn.workspace_clear_status(ws)
    spffn.decode_step(model, x, ws=ws)
    assert int(spffn.workspace_status(ws)) == 0


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


@pytest.mark.parametrize("kind", ["reglu", "relu"])
@pytest.mark.parametrize("w_dtype,d", [("f16", 12288), ("f32", 8192), ("f32", 4096)])
def test_decode_wide_rows_single_token(kind, w_dtype, d):
    """The single-token layer kernel with eight (fp16 d = 12288, fp32 d = 8192)
    or four (fp32 d = 4096) packets per lane per gathered row."""
    print(f"edge decode wide rows {kind} {w_dtype} d={d}", flush=True)
    cfg = replace(TINY, kind=kind, w_dtype=w_dtype, p_dtype=w_dtype, d=d, d_ffn=1000, r=64,
                  w_std=d ** -0.5)
    _decode_checks(cfg, 1, 2, seed=57, n_cal=512)


@pytest.mark.parametrize("B", [1, 3])
def test_decode_q4_gated(B):
    """4-bit gated rows (gate, up and down all in 4-bit blocks)."""
    print(f"edge decode 4-bit ReGLU B={B}", flush=True)
    from workloads import OPT_175B_Q4
    cfg = replace(OPT_175B_Q4, kind="reglu", d=512, d_ffn=1530, r=64, layers=2)
    _decode_checks(cfg, B, 2, seed=59, n_cal=512)
