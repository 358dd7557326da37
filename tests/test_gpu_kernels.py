"""GPU parity of every entry point against the CPU oracle at small and ragged
shapes (several tiles and a ragged tail), through the C ABI."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import activation_sparse_mlp_amd as spffn
import oracle
from tests.gpu_helpers import (DEV, REL_L2, check_mask_agreement, gpu_layer, np_layer, rel_l2,
                               to_dev)
from workloads import TINY, LLAMA2_7B, OPT_175B_Q4, make_layer, make_tokens, q4_0_pack

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# --------------------------------------------------------------------------- #
# threshold and compaction: bit-exact
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("n", [1, 7, 1000, 28672, 49152, 100003])
def test_threshold_bit_exact(n):
    rng = np.random.default_rng(n)
    lg = (rng.standard_normal(n) * 3).astype(np.float32)
    lg[:: max(1, n // 7)] = 0.0
    if n > 10:
        lg[3] = np.nan
        lg[5] = -0.0
        lg[7] = np.float32(0.25)
    for t in (0.0, 0.25, -0.2006707):
        print(f"threshold n={n} t={t}", flush=True)
        got = spffn.threshold(torch.from_numpy(lg).to(DEV), t).cpu().numpy()
        assert np.array_equal(got, oracle.threshold(lg, t))


@pytest.mark.parametrize("n", [1, 15, 16, 17, 1023, 1024, 4099, 11008, 28672, 49152, 131077])
def test_compact_bit_exact(n):
    rng = np.random.default_rng(1000 + n)
    for p in (0.0, 0.01, 0.1, 0.5, 1.0):
        m = (rng.random(n) < p).astype(np.uint8)
        m[m == 1] = rng.integers(1, 256, size=int(m.sum()), dtype=np.uint8)
        print(f"compact n={n} p={p}", flush=True)
        md = torch.from_numpy(m).to(DEV)
        idx, cnt = spffn.compact(md)
        c = int(cnt.item())
        ref = oracle.compact(m)
        assert c == ref.size
        assert np.array_equal(idx[:c].cpu().numpy(), ref)


def test_compact_unaligned_mask():
    rng = np.random.default_rng(7)
    m = (rng.random(5001) < 0.2).astype(np.uint8)
    buf = torch.zeros(5001 + 3, dtype=torch.uint8, device=DEV)
    buf[3:] = torch.from_numpy(m).to(DEV)
    idx, cnt = spffn.compact(buf[3:])
    c = int(cnt.item())
    assert np.array_equal(idx[:c].cpu().numpy(), oracle.compact(m))


# --------------------------------------------------------------------------- #
# predictor
# --------------------------------------------------------------------------- #
def _predict_case(cfg, B, seed=0, n_cal=2048):
    w = make_layer(cfg, 0, seed=seed, n_cal=n_cal)
    G, L = gpu_layer(w), np_layer(w)
    x = make_tokens(cfg.d, 1, B, seed=seed + 1)[0]
    out = spffn.predict(G, x.to(DEV))
    torch.cuda.synchronize()
    lg = out["logits"].cpu().numpy()
    mk = out["mask"].cpu().numpy()
    un = out["union"].cpu().numpy()
    for b in range(B):
        _, ref_lg, _ = oracle.predict(L, x[b].numpy())
        assert np.max(np.abs(lg[b] - ref_lg)) < 1e-3 * max(1.0, np.max(np.abs(ref_lg)))
        check_mask_agreement(mk[b], ref_lg, L["t"])
        # the GPU decision from its own fp32 logits is the fp32 threshold rule
        assert np.array_equal(mk[b], oracle.threshold(lg[b], L["t"]))
    assert np.array_equal(un, oracle.union(mk))
    return G, L, x, mk, un


@pytest.mark.parametrize("B", [1, 3, 16])
def test_predict_tiny(B):
    _predict_case(TINY, B)


def test_predict_fp16_edge_shape():
    cfg = replace(LLAMA2_7B, d=200, d_ffn=1000, r=24, tau=0.45)
    _predict_case(cfg, 5, seed=3)


# --------------------------------------------------------------------------- #
# forward
# --------------------------------------------------------------------------- #
def _forward_checks(cfg, B, seed=0, n_cal=1024):
    w = make_layer(cfg, 0, seed=seed, n_cal=n_cal)
    G, L = gpu_layer(w), np_layer(w)
    x = make_tokens(cfg.d, 1, B, seed=seed + 2)[0]
    xd = x.to(DEV)
    xs = x.numpy()
    # the oracle's own predicted union mask drives both sides
    masks = np.stack([oracle.predict(L, xs[b])[2] for b in range(B)])
    U = oracle.union(masks)
    print(f"forward {cfg.name} d={cfg.d} d_ffn={cfg.d_ffn} B={B} active={int(U.sum())}",
          flush=True)
    y = spffn.forward(G, xd, mask=torch.from_numpy(U).to(DEV)).cpu().numpy()
    for b in range(B):
        assert rel_l2(y[b], oracle.ffn_masked(L, xs[b], U)) <= REL_L2
    # same set as an index list (in a buffer with room for d_ffn entries)
    lst = oracle.compact(U)
    idx = torch.zeros(cfg.d_ffn, dtype=torch.int32, device=DEV)
    idx[:lst.size] = torch.from_numpy(lst).to(DEV)
    cnt = torch.tensor([lst.size], dtype=torch.int32, device=DEV)
    y2 = spffn.forward(G, xd, idx=idx, count=cnt).cpu().numpy()
    assert np.array_equal(y2, y)  # same kernels, same order
    # dense
    yd = spffn.forward(G, xd).cpu().numpy()
    for b in range(B):
        assert rel_l2(yd[b], oracle.ffn_dense(L, xs[b])[0]) <= REL_L2
    # all-ones mask equals dense; empty mask gives exact zeros
    ones = torch.ones(cfg.d_ffn, dtype=torch.uint8, device=DEV)
    assert np.array_equal(spffn.forward(G, xd, mask=ones).cpu().numpy(), yd)
    zeros = torch.zeros(cfg.d_ffn, dtype=torch.uint8, device=DEV)
    assert np.all(spffn.forward(G, xd, mask=zeros).cpu().numpy() == 0.0)
    # bit-stable reruns
    y3 = spffn.forward(G, xd, mask=torch.from_numpy(U).to(DEV)).cpu().numpy()
    assert np.array_equal(y3, y)


@pytest.mark.parametrize("B", [1, 4, 16])
def test_forward_tiny(B):
    _forward_checks(TINY, B)


@pytest.mark.parametrize("kind,w_dtype", [("relu", "f32"), ("reglu", "f32"), ("relu", "f16"),
                                          ("reglu", "f16")])
@pytest.mark.parametrize("B", [1, 5])
def test_forward_edge_shapes(kind, w_dtype, B):
    cfg = replace(TINY, kind=kind, w_dtype=w_dtype, p_dtype=w_dtype, d=200, d_ffn=1000, r=16,
                  w_std=0.05)
    _forward_checks(cfg, B, seed=11)


def test_forward_count_zero_and_clamped():
    w = make_layer(TINY, 0, seed=5, n_cal=512)
    G = gpu_layer(w)
    x = make_tokens(TINY.d, 1, 1, seed=9)[0].to(DEV)
    idx = torch.arange(TINY.d_ffn, dtype=torch.int32, device=DEV)
    zero = torch.zeros(1, dtype=torch.int32, device=DEV)
    assert torch.all(spffn.forward(G, x, idx=idx, count=zero) == 0)
    # a count above d_ffn is clamped to d_ffn (the dense result)
    big = torch.tensor([TINY.d_ffn + 500], dtype=torch.int32, device=DEV)
    assert torch.equal(spffn.forward(G, x, idx=idx, count=big), spffn.forward(G, x))


# --------------------------------------------------------------------------- #
# decode step (teacher forced through the trace)
# --------------------------------------------------------------------------- #
def _decode_checks(cfg, B, layers, seed=0, n_cal=1024, dense=False):
    hosts = [make_layer(cfg, l, seed=seed, n_cal=n_cal) for l in range(layers)]
    G = [gpu_layer(w) for w in hosts]
    Ls = [np_layer(w) for w in hosts]
    model = spffn.Model(G, rms_eps=1e-5)
    x = make_tokens(cfg.d, 1, B, seed=seed + 4)[0].to(DEV)
    F = cfg.d_ffn
    trace = dict(h_in=torch.empty(layers, B, cfg.d, device=DEV),
                 union_mask=torch.empty(layers * F, dtype=torch.uint8, device=DEV),
                 logits=torch.empty(layers * B * F, device=DEV))
    counts = torch.empty(layers, dtype=torch.int32, device=DEV)
    h = spffn.decode_step(model, x, dense=dense, layer_counts=counts, trace=trace)
    torch.cuda.synchronize()
    h_in = trace["h_in"].cpu().numpy().astype(np.float64)
    assert np.array_equal(h_in[0], x.cpu().numpy())
    outs = np.concatenate([h_in[1:], h.cpu().numpy()[None].astype(np.float64)])
    masks = trace["union_mask"].cpu().numpy().reshape(layers, F)
    cnts = counts.cpu().numpy()
    for l in range(layers):
        if dense:
            U = np.ones(F, np.uint8)
            assert cnts[l] == F
        else:
            U = masks[l]
            assert cnts[l] == U.sum()
        ref = oracle.decode_layer(Ls[l], h_in[l], 1e-5, mask=U)
        if not dense:
            lg = trace["logits"].cpu().numpy().reshape(layers, B, F)[l]
            for b in range(B):
                check_mask_agreement(oracle.threshold(lg[b], Ls[l]["t"]), ref["logits"][b],
                                     Ls[l]["t"])
            assert np.array_equal(U, oracle.union(oracle.threshold(lg, Ls[l]["t"])))
        for b in range(B):
            assert rel_l2(outs[l][b] - h_in[l][b], ref["y"][b]) <= REL_L2, (l, b)
    # bit-stable rerun
    h2 = spffn.decode_step(model, x, dense=dense)
    assert torch.equal(h, h2)
    return model, h


@pytest.mark.parametrize("B", [1, 4])
def test_decode_tiny(B):
    _decode_checks(TINY, B, 2)


def test_decode_tiny_dense():
    _decode_checks(TINY, 1, 2, dense=True)


def test_decode_in_place():
    hosts = [make_layer(TINY, l, seed=2, n_cal=512) for l in range(2)]
    model = spffn.Model([gpu_layer(w) for w in hosts])
    x = make_tokens(TINY.d, 1, 2, seed=8)[0].to(DEV)
    h_out = spffn.decode_step(model, x)
    hx = x.clone()
    spffn.decode_step(model, hx, h=hx)
    assert torch.equal(hx, h_out)


# --------------------------------------------------------------------------- #
# load-time utilities
# --------------------------------------------------------------------------- #
def test_profile_counts():
    w = make_layer(TINY, 0, seed=6, n_cal=512)
    G, L = gpu_layer(w), np_layer(w)
    X = make_tokens(TINY.d, 40, 1, seed=12)[:, 0, :]
    got = spffn.profile(G, X.to(DEV)).cpu().numpy()
    ref = oracle.profile(L, X.numpy())
    # a count may differ only by tokens whose pre-activation is within fp32
    # rounding of zero
    near = np.zeros(TINY.d_ffn, np.int64)
    for x in X.numpy():
        z = oracle.preact(L, x)[0]
        near += np.abs(z) < 1e-4
    assert np.all(np.abs(got - ref) <= near)
    assert np.mean(got == ref) > 0.99


_PROF_F16 = replace(LLAMA2_7B, d=1024, d_ffn=1000, r=64)      # fp16 rows, d a multiple of 512
_PROF_RELU = replace(LLAMA2_7B, kind="relu", d=512, d_ffn=700, r=64)


def _near_zero_tokens(L, X):
    near = np.zeros(L["d_ffn"], np.int64)
    for x in X:
        z = oracle.preact(L, x)[0]
        near += np.abs(z) < 1e-4
    return near


@pytest.mark.parametrize("cfg", [_PROF_F16, _PROF_RELU])
@pytest.mark.parametrize("N", [1, 5, 13, 40])
def test_profile_counts_matrix_cores(cfg, N):
    """fp16 rows are profiled on the matrix cores when the library gets its
    scratch (tokens in groups of 16: one or two halves per instruction, and a
    ragged last group); counts against the oracle, and against the vector
    kernels, within the tokens whose pre-activation is near zero."""
    w = make_layer(cfg, 0, seed=16, n_cal=512)
    G, L = gpu_layer(w), np_layer(w)
    X = make_tokens(cfg.d, N, 1, seed=17)[:, 0, :]
    assert spffn.load().spffn_profile_workspace_bytes(G.handle) == 64 * cfg.d
    got = spffn.profile(G, X.to(DEV)).cpu().numpy()
    vec = spffn.profile(G, X.to(DEV), scratch=False).cpu().numpy()
    ref = oracle.profile(L, X.numpy())
    near = _near_zero_tokens(L, X.numpy())
    assert np.all(np.abs(got - ref) <= near)
    assert np.all(np.abs(got - vec) <= near)
    assert np.mean(got == ref) > 0.99
    # counts accumulate across calls
    twice = spffn.profile(G, X.to(DEV), counts=torch.from_numpy(got).to(DEV)).cpu().numpy()
    assert np.array_equal(twice, 2 * got)


# sizes around the kernel's 64-neuron blocks and 1024-entry tiles, and the
# full 70B width
@pytest.mark.parametrize("n", [1, 5, 63, 64, 65, 1000, 1023, 1024, 1025, 28672])
def test_hot_first_order_bit_exact(n):
    rng = np.random.default_rng(n)
    counts = rng.integers(0, 20, size=n).astype(np.int32)
    got = spffn.hot_first_order(torch.from_numpy(counts).to(DEV)).cpu().numpy()
    assert np.array_equal(got, oracle.hot_first_perm(counts))


def test_permute_rows_bit_exact():
    rng = np.random.default_rng(3)
    for shape, dt in (((37, 24), np.float16), ((100, 7), np.float32), ((9, 1), np.float32),
                      ((64, 36), np.uint8)):
        a = (rng.standard_normal(shape) * 10).astype(dt)
        perm = rng.permutation(shape[0]).astype(np.int32)
        got = spffn.permute_rows(torch.from_numpy(a).to(DEV),
                                 torch.from_numpy(perm).to(DEV)).cpu().numpy()
        assert np.array_equal(got, a[perm])


def test_hot_first_permute_layer():
    w = make_layer(TINY, 0, seed=4, n_cal=512)
    wd = to_dev(w)
    X = make_tokens(TINY.d, 64, 1, seed=13)[:, 0, :]
    pw, perm, counts = spffn.hot_first_permute(wd, X.to(DEV))
    perm = perm.cpu().numpy()
    c = counts.cpu().numpy()
    assert np.array_equal(perm, oracle.hot_first_perm(c))
    L = np_layer(w)
    P = oracle.permute_layer(L, perm)
    G = spffn.Layer(pw)
    x = make_tokens(TINY.d, 1, 1, seed=14)[0]
    m = oracle.predict(P, x[0].numpy())[2]
    y = spffn.forward(G, x.to(DEV), mask=torch.from_numpy(m).to(DEV)).cpu().numpy()[0]
    assert rel_l2(y, oracle.ffn_masked(P, x[0].numpy(), m)) <= REL_L2
    # permuting back through perm gives the unpermuted layer's sparse FFN
    m0 = np.zeros_like(m)
    m0[perm[m == 1]] = 1
    assert rel_l2(y, oracle.ffn_masked(L, x[0].numpy(), m0)) <= REL_L2


# --------------------------------------------------------------------------- #
# 4-bit blocks
# --------------------------------------------------------------------------- #
def test_q4_0_repack_bit_exact():
    g = torch.Generator().manual_seed(1)
    rows, cols = 33, 96
    codes = torch.randint(0, 16, (rows, cols), generator=g, dtype=torch.uint8)
    scales = torch.randn(rows, cols // 32, generator=g).half()
    aos = q4_0_pack(codes, scales)
    soa = spffn.q4_0_repack(aos.to(DEV), rows, cols).cpu().numpy()
    blocks = aos.numpy().reshape(rows * cols // 32, 18)
    ref = np.concatenate([blocks[:, 2:].ravel(), blocks[:, :2].ravel()])
    assert np.array_equal(soa, ref)


@pytest.mark.parametrize("B", [1, 3])
def test_q4_0_forward_and_predict(B):
    cfg = replace(OPT_175B_Q4, d=512, d_ffn=1536, r=64, layers=1)
    _forward_checks(cfg, B, seed=21)
    _predict_case(cfg, B, seed=21, n_cal=1024)


def test_q4_0_decode_b1_ragged_groups():
    """Single-token decode with 4-bit rows (layer kernel, 20-row groups): 1530
    neurons leave the last group half empty."""
    cfg = replace(OPT_175B_Q4, d=512, d_ffn=1530, r=64, layers=2)
    _decode_checks(cfg, 1, 2, seed=29)


def test_q4_0_profile():
    cfg = replace(OPT_175B_Q4, d=256, d_ffn=512, r=32, layers=1)
    w = make_layer(cfg, 0, seed=3, n_cal=512)
    G, L = gpu_layer(w), np_layer(w)
    X = make_tokens(cfg.d, 20, 1, seed=15)[:, 0, :]
    got = spffn.profile(G, X.to(DEV)).cpu().numpy()
    ref = oracle.profile(L, X.numpy())
    assert np.mean(got == ref) > 0.99
