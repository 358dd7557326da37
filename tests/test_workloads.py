"""The synthetic-workload generator: firing statistics, reproducibility and the
4-bit block packing.  CPU only (tiny shapes)."""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import (ALL, TINY, firing_probs, layer_to_numpy, make_layer, make_tokens,
                       q4_0_pack, q4_0_values)


@pytest.mark.parametrize("name", list(ALL))
def test_firing_probs(name):
    c = ALL[name]
    p = firing_probs(c.d_ffn, c.gamma, c.mean_activity)
    assert abs(p.mean() - c.mean_activity) < 1e-12
    assert np.all(np.diff(p) <= 0) and p.max() < 1.0 and p.min() > 0.0
    # unsaturated ranks follow k^-gamma exactly
    k = np.arange(1, c.d_ffn + 1)
    free = p < p.max()
    slope = np.polyfit(np.log(k[free]), np.log(p[free]), 1)[0]
    assert abs(slope + c.gamma) < 1e-9


@pytest.fixture(scope="module")
def tiny_layer():
    return layer_to_numpy(make_layer(TINY, 0, seed=0))


def test_realised_activity(tiny_layer):
    """Exact-mask firing on fresh N(0, I) tokens matches the target p_i."""
    L = tiny_layer
    N = 800
    X = make_tokens(TINY.d, N, 1, seed=5).numpy()[:, 0, :]
    counts = oracle.profile(L, X)
    rate = counts / N
    p = L["p_fire"]
    # aggregate activity within 4 sigma of the binomial mean
    sigma = math.sqrt((p * (1 - p)).sum() * N)
    assert abs(counts.sum() - p.sum() * N) < 4 * sigma
    # per neuron: |rate - p| within 4.5 sigma for almost every neuron
    s = np.sqrt(p * (1 - p) / N)
    assert np.mean(np.abs(rate - p) <= 4.5 * s + 1.0 / N) > 0.99
    # realised hot-first ordering recovers the planted power law roughly
    perm = oracle.hot_first_perm(counts)
    top = int(0.2 * L["d_ffn"])
    share = counts[perm[:top]].sum() / counts.sum()
    assert 0.65 < share < 0.85


def test_predictor_density(tiny_layer):
    """The fitted predictor marks about the configured share of neurons active
    and agrees with the exact mask far better than chance."""
    L = dict(tiny_layer, t=oracle.logit_threshold(TINY.tau))
    X = make_tokens(TINY.d, 64, 1, seed=6).numpy()[:, 0, :]
    dens, rec = [], []
    for x in X:
        m = oracle.predict(L, x)[2]
        em = oracle.preact(L, x)[2]
        dens.append(m.mean())
        rec.append((m & em).sum() / max(1, em.sum()))
    assert abs(np.mean(dens) - TINY.mean_activity) < 0.02
    assert np.mean(rec) > 3 * TINY.mean_activity


def test_seed_reproducible():
    a = make_layer(TINY, 1, seed=3)
    b = make_layer(TINY, 1, seed=3)
    c = make_layer(TINY, 1, seed=4)
    for k in ("w_up", "w_down_t", "b_act", "p_w1", "p_w2", "p_b2"):
        assert torch.equal(a[k], b[k])
        assert not torch.equal(a[k], c[k])
    assert torch.equal(make_tokens(64, 3, 2, seed=1), make_tokens(64, 3, 2, seed=1))


def test_q4_0_pack_layout():
    """Packed blocks read back through the oracle's block reader give exactly
    (code - 8) * scale."""
    g = torch.Generator().manual_seed(0)
    rows, cols = 5, 96
    codes = torch.randint(0, 16, (rows, cols), generator=g, dtype=torch.uint8)
    scales = (torch.randn(rows, cols // 32, generator=g) * 0.01).abs().half()
    packed = q4_0_pack(codes, scales).numpy()
    assert packed.shape == (rows, cols // 32 * 18)
    vals = oracle.deq(packed, "q4_0", cols)
    assert np.array_equal(vals, q4_0_values(codes, scales).double().numpy())


def test_q4_0_layer_generation():
    from dataclasses import replace
    cfg = replace(ALL["opt_175b_relu_q4_0"], d=128, d_ffn=256, r=32, layers=1)
    L = make_layer(cfg, 0, seed=0, n_cal=512, return_values=True)
    assert L["w_up"].dtype == torch.uint8 and L["w_up"].shape == (256, 128 // 32 * 18)
    vals = oracle.deq(L["w_up"].numpy(), "q4_0", 128)
    assert np.array_equal(vals, L["act_values"].double().numpy())


def test_stack_keeps_configured_activity_at_depth():
    """A stack of 4-bit ReLU layers (codes with mean -0.5 make every layer add
    a common direction to the residual stream) realises its configured
    activity in every layer when each layer is calibrated on the inputs it
    receives (make_stack); the first layer is the independent layer 0."""
    from dataclasses import replace

    from workloads import OPT_175B_Q4, make_stack
    cfg = replace(OPT_175B_Q4, d=512, d_ffn=2048, r=64, layers=6)
    ws = list(make_stack(cfg, seed=0, n_cal=2048))
    w0 = make_layer(cfg, 0, seed=0, n_cal=2048)
    for k, v in w0.items():
        if isinstance(v, torch.Tensor):
            assert torch.equal(v, ws[0][k]), k
    Ls = []
    for w in ws:
        L = layer_to_numpy(w)
        L["t"] = oracle.logit_threshold(L["tau"])
        Ls.append(L)
    X = make_tokens(cfg.d, 24, 1, seed=0)
    act = np.zeros(cfg.layers)
    for k in range(24):
        h = X[k].double().numpy()
        for l, L in enumerate(Ls):
            o = oracle.decode_layer(L, h, 1e-5)
            act[l] += o["union"].mean() / 24
            h = o["h"]
    assert np.all(np.abs(act - cfg.mean_activity) < 0.015), act


def test_fp8_predictor_layer():
    """An fp8 predictor is stored as E4M3 codes plus one scale per row, the
    scale maps each row's largest weight to 448, and the predictor still
    realises the configured density on fresh tokens (the shift is fitted on
    the decoded weights)."""
    from dataclasses import replace

    from workloads import fp8_pack
    cfg = replace(TINY, p_dtype="fp8")
    w = make_layer(cfg, 0, seed=0, n_cal=2048)
    r, d, F = cfg.r, cfg.d, cfg.d_ffn
    assert w["p_w1"].dtype == torch.uint8 and w["p_w1"].numel() == r * (d + 4)
    assert w["p_w2"].numel() == F * (r + 4)
    L = layer_to_numpy(w)
    W1 = oracle.deq(L["p_w1"], "fp8", d)
    scales = L["p_w1"][r * d:].view(np.float32)
    assert np.array_equal(np.abs(W1).max(axis=1), 448.0 * scales.astype(np.float64))
    # the values the generator works with are the codes times the scales
    buf, vals = fp8_pack(torch.from_numpy(W1.astype(np.float32)))
    codes = buf[:r * d].numpy().reshape(r, d)
    sc = buf[r * d:].numpy().view(np.float32)
    assert np.array_equal(vals.numpy(), (oracle.e4m3_to_f64(codes) * sc[:, None]).astype(np.float32))
    L["t"] = oracle.logit_threshold(L["tau"])
    X = make_tokens(d, 64, 1, seed=5)[:, 0, :].double().numpy()
    dens = np.mean([oracle.predict(L, x)[2].mean() for x in X])
    assert abs(dens - cfg.mean_activity) < 0.03, dens


def test_swiglu_layer_is_magnitude_sparse():
    """The SwiGLU workload's wide gate makes SiLU activations magnitude-sparse:
    few neurons exceed 1e-3 of the token's largest activation, while the
    predictor keeps the configured density."""
    from dataclasses import replace

    from workloads import LLAMA2_7B_SWIGLU
    cfg = replace(LLAMA2_7B_SWIGLU, d=512, d_ffn=1536, r=64, gate_std=0.1 * 8 ** 0.5)
    L = layer_to_numpy(make_layer(cfg, 0, seed=0, n_cal=2048))
    L["t"] = oracle.logit_threshold(L["tau"])
    X = make_tokens(cfg.d, 16, 1, seed=3)[:, 0, :].double().numpy()
    mag, dens = [], []
    for x in X:
        _, act = oracle.ffn_dense(L, x)
        mag.append(np.mean(np.abs(act) > 1e-3 * np.abs(act).max()))
        dens.append(oracle.predict(L, x)[2].mean())
    assert np.mean(mag) < 0.25, np.mean(mag)
    assert abs(np.mean(dens) - cfg.mean_activity) < 0.03, np.mean(dens)
