"""GPU parity at the workloads' full layer shapes, in the launch configuration
the benchmark times (decode step, hot-first rows for the 70B shape), checked
layer by layer against the CPU oracle (teacher forced through the trace).
Stacks are generated as the benchmark generates them (make_stack: every layer
calibrated on the inputs it receives; 4096 calibration tokens; 256 profile
tokens for the hot-first order; the benchmark's first token), and the deep
stacks (7B, 40B, 70B, 175B) are checked at their first, second, middle and
last layers.  Large batches are checked on sampled tokens."""
import numpy as np
import pytest
import torch

import activation_sparse_mlp_amd as spffn
import oracle
from tests.gpu_helpers import DEV, REL_L2, check_mask_agreement, np_layer, rel_l2
from workloads import (FALCON_40B, LLAMA2_7B, LLAMA2_70B, OPT_175B_Q4, make_layer,
                       make_profile_tokens, make_stack, make_tokens)

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def teardown_function(function):
    torch.cuda.empty_cache()


def _build(cfg, layers, hot_first, n_cal=4096):
    """The first `layers` layers of cfg's stack, as the benchmark builds them."""
    hosts, gl = [], []
    calib = make_profile_tokens(cfg.d, 256, seed=1, device=DEV) if hot_first else None
    for l, w in enumerate(make_stack(cfg, seed=0, device=DEV, n_cal=n_cal, n_layers=layers)):
        if hot_first:
            w, perm, counts = spffn.hot_first_permute(w, calib, dense_prefix=cfg.dense_prefix)
            if cfg.dense_prefix:
                # the prefix is every neuron that fired on all profiling tokens
                assert w["dense_prefix"] == int((counts == 256).sum()) > 0
            if l < 2:
                c = counts.cpu().numpy()
                assert np.array_equal(perm.cpu().numpy(), oracle.hot_first_perm(c))
        gl.append(spffn.Layer(w))
        hosts.append(w)
        if l % 16 == 15:
            print(f"  built {l + 1}/{layers}", flush=True)
    return hosts, gl


def _decode_check(cfg, B, layers, hot_first, tokens_checked=None, layers_checked=None):
    print(f"decode {cfg.name} B={B} layers={layers}", flush=True)
    hosts, gl = _build(cfg, layers, hot_first)
    model = spffn.Model(gl, rms_eps=1e-5)
    ws = model.workspace(B)
    F, d = cfg.d_ffn, cfg.d
    x = make_tokens(d, cfg.tokens, B, seed=0, device=DEV)[0]  # the benchmark's first token
    trace = dict(h_in=torch.empty(layers, B, d, device=DEV),
                 union_mask=torch.empty(layers * F, dtype=torch.uint8, device=DEV),
                 logits=torch.empty(layers * B * F, device=DEV))
    counts = torch.empty(layers, dtype=torch.int32, device=DEV)
    h = spffn.decode_step(model, x, layer_counts=counts, trace=trace, ws=ws)
    torch.cuda.synchronize()
    assert int(spffn.workspace_status(ws)) == 0
    assert torch.isfinite(h).all()
    h_in = trace["h_in"].cpu().numpy().astype(np.float64)
    outs = np.concatenate([h_in[1:], h.cpu().numpy()[None].astype(np.float64)])
    masks = trace["union_mask"].cpu().numpy().reshape(layers, F)
    lg = trace["logits"].cpu().numpy().reshape(layers, B, F)
    cnts = counts.cpu().numpy()
    # every layer: the count is the union's popcount, and the union is the OR
    # of the per-token decisions on the GPU's own logits
    for l in range(layers):
        assert cnts[l] == masks[l].sum()
    acts = cnts / F
    print(f"  realised activity: min {acts.min():.4f} mean {acts.mean():.4f} "
          f"max {acts.max():.4f}", flush=True)
    check = range(B) if tokens_checked is None else tokens_checked
    for l in (range(layers) if layers_checked is None else layers_checked):
        L = np_layer(hosts[l])
        U = masks[l]
        assert np.array_equal(U, oracle.union(oracle.threshold(lg[l], L["t"])))
        for b in check:
            n = oracle.rmsnorm(h_in[l][b], 1e-5)
            _, ref_lg, _ = oracle.predict(L, n)
            fin = np.isfinite(ref_lg)  # the always-active prefix reports +inf on both sides
            assert np.array_equal(np.isposinf(lg[l][b]), ~fin)
            assert np.max(np.abs(lg[l][b][fin] - ref_lg[fin])) < 1e-3
            check_mask_agreement(oracle.threshold(lg[l][b], L["t"]), ref_lg, L["t"])
            y_ref = oracle.ffn_masked(L, n, U)
            err = rel_l2(outs[l][b] - h_in[l][b], y_ref)
            print(f"  layer {l} token {b}: active {int(U.sum())}, rel-L2 {err:.2e}", flush=True)
            assert err <= REL_L2
        del L
    # the step is bit-stable
    h2 = spffn.decode_step(model, x, ws=ws)
    assert torch.equal(h, h2)
    return acts


def test_llama2_70b_decode_b1_hot_first():
    _decode_check(LLAMA2_70B, 1, 2, hot_first=True)


@pytest.mark.timeout(600)
def test_llama2_70b_benchmarked_stack_deep_layers():
    """The whole 80-layer stack the benchmark times, one traced step, checked
    at layers 0, 1, 40 and 79."""
    acts = _decode_check(LLAMA2_70B, 1, LLAMA2_70B.layers, hot_first=True,
                         layers_checked=[0, 1, 40, 79])
    assert abs(acts.mean() - LLAMA2_70B.mean_activity) < 0.02


def test_llama2_7b_decode_b1():
    _decode_check(LLAMA2_7B, 1, 2, hot_first=False)


@pytest.mark.timeout(600)
def test_llama2_7b_benchmarked_stack_deep_layers():
    """The whole 32-layer 7B-shaped stack the benchmark times, one traced step,
    checked at layers 0, 1, 16 and 31."""
    acts = _decode_check(LLAMA2_7B, 1, LLAMA2_7B.layers, hot_first=False,
                         layers_checked=[0, 1, 16, 31])
    assert abs(acts.mean() - LLAMA2_7B.mean_activity) < 0.02


@pytest.mark.timeout(600)
def test_falcon_40b_benchmarked_stack_deep_layers():
    """The whole 60-layer 40B-shaped ReLU stack the benchmark times, one traced
    step, checked at layers 0, 1, 30 and 59."""
    acts = _decode_check(FALCON_40B, 1, FALCON_40B.layers, hot_first=False,
                         layers_checked=[0, 1, 30, 59])
    assert abs(acts.mean() - FALCON_40B.mean_activity) < 0.02


def test_falcon_40b_decode_b1():
    """The non-gated fp16 single-token layer kernel at d = 8192 (12-row groups,
    four packets per lane per gathered row)."""
    _decode_check(FALCON_40B, 1, 2, hot_first=False)


@pytest.mark.parametrize("B", [4, 16])
def test_llama2_70b_decode_batched(B):
    _decode_check(LLAMA2_70B, B, 1, hot_first=True, tokens_checked=[0, B - 1])


def test_falcon_40b_decode_b8():
    _decode_check(FALCON_40B, 8, 1, hot_first=False, tokens_checked=[0, 7])


@pytest.mark.timeout(600)
def test_llama2_70b_benchmarked_stack_deep_layers_b16():
    """The 80-layer stack at B = 16 (the matrix-core path the benchmark times),
    one traced step, checked at layers 0, 40 and 79 on the first and last
    tokens."""
    _decode_check(LLAMA2_70B, 16, LLAMA2_70B.layers, hot_first=True, tokens_checked=[0, 15],
                  layers_checked=[0, 40, 79])


@pytest.mark.timeout(600)
def test_falcon_40b_benchmarked_stack_deep_layers_b8():
    """The 60-layer ReLU stack at B = 8, one traced step, checked at layers 0,
    30 and 59 on the first and last tokens."""
    _decode_check(FALCON_40B, 8, FALCON_40B.layers, hot_first=False, tokens_checked=[0, 7],
                  layers_checked=[0, 30, 59])


def test_opt_175b_q4_0_decode_b1():
    _decode_check(OPT_175B_Q4, 1, 1, hot_first=False)


@pytest.mark.timeout(600)
def test_opt_175b_q4_0_benchmarked_stack_deep_layers():
    """The whole 96-layer 4-bit stack the benchmark times, one traced step,
    checked at layers 0, 1, 48 and 95.  The stack keeps the configured 5%
    activity at depth on average (one token's layers scatter around it: the
    4-bit codes' mean of -0.5 gives the residual stream a common direction,
    so a token's activity moves all neurons of a layer together)."""
    acts = _decode_check(OPT_175B_Q4, 1, OPT_175B_Q4.layers, hot_first=False,
                         layers_checked=[0, 1, 48, 95])
    assert abs(acts.mean() - OPT_175B_Q4.mean_activity) < 0.025
    assert acts.max() < 3 * OPT_175B_Q4.mean_activity


def test_opt_175b_q4_0_forward_dense_row_sample():
    """The dense 4-bit FFN (every neuron) at full shape against the oracle on
    the same dequantised weights."""
    cfg = OPT_175B_Q4
    w = make_layer(cfg, 0, seed=2, device=DEV, n_cal=1024)
    G = spffn.Layer(w)
    L = np_layer(w)
    x = make_tokens(cfg.d, 1, 1, seed=4, device=DEV)[0]
    # a sampled neuron set: every 97th neuron (keeps the oracle fast)
    idx = torch.arange(0, cfg.d_ffn, 97, dtype=torch.int32, device=DEV)
    idx_full = torch.zeros(cfg.d_ffn, dtype=torch.int32, device=DEV)
    idx_full[:idx.numel()] = idx
    cnt = torch.tensor([idx.numel()], dtype=torch.int32, device=DEV)
    y = spffn.forward(G, x, idx=idx_full, count=cnt).cpu().numpy()[0]
    ref, _ = oracle.ffn_sparse(L, x[0].cpu().numpy(), idx.cpu().numpy())
    assert rel_l2(y, ref) <= REL_L2
