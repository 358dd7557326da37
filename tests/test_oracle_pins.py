"""Pins of the CPU oracle to things other than itself: hand-derived values,
closed forms, exhaustive enumeration, invariants, and special cases that
reduce to a library routine.  No GPU involved."""
import itertools
import math

import numpy as np
import pytest

import oracle
from tests.conftest import load_golden


def _hand_layer(kind):
    g = load_golden("hand_ffn.json")
    s = g[kind]
    f64 = lambda v: np.asarray(v, dtype=np.float32)  # noqa: E731  small integers/halves are exact
    L = dict(kind=kind, w_dtype="f32", p_dtype="f32", d=3, d_ffn=4, r=2,
             w_gate=f64(s["w_gate"]) if kind == "reglu" else None, w_up=f64(s["w_up"]),
             w_down_t=f64(s["w_down_t"]), b_act=f64(s["b_act"]),
             p_w1=f64(g["predictor"]["p_w1"]), p_b1=f64(g["predictor"]["p_b1"]),
             p_w2=f64(g["predictor"]["p_w2"]), p_b2=f64(g["predictor"]["p_b2"]), t=0.0)
    return L, np.asarray(g["x"], np.float64), s, g["predictor"]


def _rand_layer(rng, kind, d, d_ffn, r=8, w_dtype="f32", density=0.3):
    """Small random layer; biases put about `density` of the neurons above zero."""
    def mat(rows, cols):
        w = rng.standard_normal((rows, cols)) / math.sqrt(cols)
        return w.astype(np.float16 if w_dtype == "f16" else np.float32)
    L = dict(kind=kind, w_dtype=w_dtype, p_dtype=w_dtype, d=d, d_ffn=d_ffn, r=r,
             w_gate=mat(d_ffn, d) if kind == "reglu" else None, w_up=mat(d_ffn, d),
             w_down_t=mat(d_ffn, d),
             b_act=(rng.standard_normal(d_ffn) * 0.3 - 0.5 * (1 - density)).astype(np.float32),
             p_w1=mat(r, d), p_b1=np.zeros(r, np.float32), p_w2=mat(d_ffn, r),
             p_b2=(rng.standard_normal(d_ffn) * 0.1).astype(np.float32), t=0.0)
    return L


# --------------------------------------------------------------------------- #
# element formats
# --------------------------------------------------------------------------- #
def test_f16_decode_all_bit_patterns():
    """Every binary16 pattern against numpy's float16 -> float64 widening."""
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.f16_bits_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, ours[0x8000]) == -1.0


@pytest.mark.parametrize("kind", ["relu", "reglu"])
def test_dense_prefix_hand(kind):
    """The hand example with an always-active prefix of two neurons
    (golden/hand_prefix.json): not scored, forced active, computed."""
    g = load_golden("hand_prefix.json")
    L, x, _, _ = _hand_layer(kind)
    L = dict(L, dense_prefix=g["dense_prefix"])
    _, logits, mask = oracle.predict(L, x)
    want = np.array([float(v) for v in g["logits"]])
    assert np.array_equal(logits, want)
    assert np.array_equal(mask, np.asarray(g["mask"], np.uint8))
    assert np.array_equal(oracle.ffn_masked(L, x, mask), np.asarray(g[f"y_{kind}"], np.float64))


def test_dense_prefix_invariants():
    """A prefix leaves the other neurons' logits and decisions as they are; a
    prefix of every neuron gives the dense FFN bit for bit; and since a
    forced-on neuron that is in fact inactive contributes an exact zero, the
    prefix joined with the exact mask still gives the dense FFN exactly."""
    rng = np.random.default_rng(21)
    L = _rand_layer(rng, "reglu", 16, 40, r=8)
    x = rng.standard_normal(16)
    _, l0, m0 = oracle.predict(L, x)
    for k in (1, 7, 39):
        _, lk, mk = oracle.predict(dict(L, dense_prefix=k), x)
        assert np.all(np.isinf(lk[:k])) and np.all(mk[:k] == 1)
        assert np.array_equal(lk[k:], l0[k:]) and np.array_equal(mk[k:], m0[k:])
    Lall = dict(L, dense_prefix=40)
    h = np.atleast_2d(x)
    out = oracle.decode_layer(Lall, h, 1e-5)
    n = oracle.rmsnorm(x, 1e-5)
    assert np.all(out["union"] == 1)
    assert np.array_equal(out["y"][0], oracle.ffn_dense(L, n)[0])
    _, _, exact = oracle.preact(L, n)
    pre = exact.copy()
    pre[:12] = 1
    assert np.array_equal(oracle.ffn_masked(L, n, pre), oracle.ffn_dense(L, n)[0])


def _swiglu_hand():
    g = load_golden("hand_swiglu.json")
    f = lambda v: np.asarray(v, dtype=np.float32)  # noqa: E731
    L = dict(kind="swiglu", w_dtype="f32", p_dtype="f32", d=2, d_ffn=3, r=1,
             w_gate=f(g["w_gate"]), w_up=f(g["w_up"]), w_down_t=f(g["w_down_t"]),
             b_act=f(g["b_act"]), p_w1=f([[0, 0]]), p_b1=f([0]), p_w2=f([[0], [0], [0]]),
             p_b2=f([1, 1, 1]), t=0.0)
    x = np.array([math.log(3.0), 2.0])
    return g, L, x


def test_swiglu_hand():
    """SiLU on the hand-derived layer (golden/hand_swiglu.json): the
    activations, the dense output, and a mask that leaves a near-zero neuron
    out, whose error is exactly that neuron's contribution."""
    g, L, x = _swiglu_hand()
    ln3 = math.log(3.0)
    y, act = oracle.ffn_dense(L, x)
    np.testing.assert_allclose(act, ln3 * np.array(g["act_over_ln3"]), rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(y, ln3 * np.array(g["y_over_ln3"]), rtol=1e-15, atol=1e-16)
    y01 = oracle.ffn_masked(L, x, np.uint8([1, 1, 0]))
    np.testing.assert_allclose(y01, ln3 * np.array(g["y_mask01_over_ln3"]), rtol=1e-15,
                               atol=1e-16)
    # every neuron: the masked FFN is the dense one bit for bit
    assert np.array_equal(oracle.ffn_masked(L, x, np.ones(3, np.uint8)), y)


def test_swiglu_silu_against_expit_and_magnitude_bound():
    """SiLU against scipy's logistic function (a library the oracle does not
    use); the magnitude mask {|a_i| > eps} loses at most the skipped |a_i|
    times their W_down column norms, and reproduces the dense FFN as eps -> 0."""
    special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(31)
    L = _rand_layer(rng, "reglu", 24, 60, r=8)
    L["kind"] = "swiglu"
    L["w_gate"] = (L["w_gate"] * 6).astype(np.float32)  # wide gate: magnitude-sparse
    x = rng.standard_normal(24)
    z, u, _ = oracle.preact(L, x)
    y, act = oracle.ffn_dense(L, x)
    np.testing.assert_allclose(act, z * special.expit(z) * u, rtol=1e-13, atol=1e-300)
    W = oracle.deq(L["w_down_t"], "f32", 24)
    for eps in (1e-1, 1e-2, 1e-3):
        M = (np.abs(act) > eps).astype(np.uint8)
        err = np.linalg.norm(oracle.ffn_masked(L, x, M) - y)
        bound = np.sum(np.abs(act[M == 0]) * np.linalg.norm(W[M == 0], axis=1))
        assert err <= bound * (1 + 1e-12) + 1e-15, (eps, err, bound)
        assert M.sum() < 60  # something was skipped
    M0 = (act != 0).astype(np.uint8)
    np.testing.assert_allclose(oracle.ffn_masked(L, x, M0), y, rtol=1e-14, atol=1e-300)


def test_e4m3_decode_all_codes():
    """Every OCP E4M3 code against torch's float8_e4m3fn widening (a library
    the oracle does not use), and hand values from the format's definition:
    1.0 = 0x38 (exponent 7 = bias), the largest finite 448 = 0x7E, the
    smallest normal 2^-6 = 0x08, the smallest subnormal 2^-9 = 0x01, signed
    zero, and the two NaN codes (no infinities)."""
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x38] == 1.0 and ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9 and ours[0x07] == 7 * 2.0 ** -9
    assert ours[0x39] == 1.125 and ours[0x40] == 2.0 and ours[0xC0] == -2.0
    assert ours[0] == 0.0 and math.copysign(1.0, ours[0x80]) == -1.0
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def _fp8_buffer(codes, scales):
    return np.concatenate([np.ascontiguousarray(codes, np.uint8).ravel(),
                           np.asarray(scales, np.float32).view(np.uint8)])


def test_fp8_rows_scale_per_row():
    """A matrix of fp8 codes with one fp32 scale per row: weight (i, k) =
    e4m3(code) * scale_i, exactly (compared in binary64 with torch's decode)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    rows, cols = 5, 48
    codes = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A  # no NaN codes
    scales = np.float32([0.5, 3e-3, 1.0, 7.25, 1e-5])
    got = oracle.deq(_fp8_buffer(codes, scales), "fp8", cols)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(got, vals * scales.astype(np.float64)[:, None])


def test_fp8_predictor_equals_its_exact_values():
    """A predictor stored as fp8 rows with power-of-two row scales (so every
    weight is exactly a binary32 value) gives bit for bit the logits and mask
    of the same predictor stored as fp32."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    d, F, r = 32, 40, 16
    L = _rand_layer(rng, "relu", d, F, r=r)
    c1 = rng.integers(0, 0x7F, (r, d), dtype=np.uint8) | (rng.integers(0, 2, (r, d)) << 7)
    c2 = rng.integers(0, 0x7F, (F, r), dtype=np.uint8) | (rng.integers(0, 2, (F, r)) << 7)
    c1, c2 = c1.astype(np.uint8), c2.astype(np.uint8)
    s1 = np.float32(2.0) ** rng.integers(-12, -6, r)
    s2 = np.float32(2.0) ** rng.integers(-10, -4, F)
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()  # noqa
    L32 = dict(L, p_w1=(dec(c1) * s1[:, None]).astype(np.float32),
               p_w2=(dec(c2) * s2[:, None]).astype(np.float32))
    L8 = dict(L, p_dtype="fp8", p_w1=_fp8_buffer(c1, s1), p_w2=_fp8_buffer(c2, s2))
    assert np.array_equal(oracle.deq(L8["p_w1"], "fp8", d), L32["p_w1"].astype(np.float64))
    x = rng.standard_normal(d)
    h32, l32, m32 = oracle.predict(L32, x)
    h8, l8, m8 = oracle.predict(L8, x)
    assert np.array_equal(h8, h32) and np.array_equal(l8, l32) and np.array_equal(m8, m32)


def test_q4_0_block_hand_values():
    """One block with scale 0.5 (fp16 0x3800): code k in the low nibble of
    byte k, code k+16 in the high nibble; value (code - 8) * scale."""
    codes = np.array([(k * 7 + 3) % 16 for k in range(32)], dtype=np.uint8)
    blk = np.zeros(18, np.uint8)
    blk[0], blk[1] = 0x00, 0x38
    for k in range(16):
        blk[2 + k] = codes[k] | (codes[k + 16] << 4)
    vals = oracle.deq(blk[None, :], "q4_0", 32)[0]
    assert np.array_equal(vals, (codes.astype(np.float64) - 8.0) * 0.5)
    # the three anchor codes
    blk2 = blk.copy()
    blk2[2] = 0x80 | 0x00     # code 0 -> 0, code 16 -> 8
    blk2[3] = 0x0F            # code 1 -> 15, code 17 -> 0
    v2 = oracle.deq(blk2[None, :], "q4_0", 32)[0]
    assert v2[0] == -8 * 0.5 and v2[16] == 0.0 and v2[1] == 7 * 0.5 and v2[17] == -8 * 0.5


def test_q4_0_zero_scale_and_rows():
    rng = np.random.default_rng(1)
    rows, cols = 3, 64
    blocks = rng.integers(0, 256, size=(rows, cols // 32, 18), dtype=np.uint8)
    blocks[1, 0, 0:2] = 0  # zero scale -> all zero (both signs of zero allowed)
    vals = oracle.deq(blocks.reshape(rows, -1), "q4_0", cols)
    assert np.all(vals[1, :32] == 0.0)
    for i in range(rows):
        for b in range(cols // 32):
            s = np.frombuffer(blocks[i, b, 0:2].tobytes(), dtype="<f2")[0].astype(np.float64)
            q = np.concatenate([blocks[i, b, 2:] & 15, blocks[i, b, 2:] >> 4]).astype(np.float64)
            exp = (q - 8.0) * s
            got = vals[i, b * 32:(b + 1) * 32]
            fin = np.isfinite(exp)
            assert np.array_equal(got[fin], exp[fin])


# --------------------------------------------------------------------------- #
# hand example: FFN and predictor
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("kind", ["relu", "reglu"])
def test_hand_ffn(kind):
    L, x, s, _ = _hand_layer(kind)
    y, act = oracle.ffn_dense(L, x)
    assert y.tolist() == s["y"]
    assert act.tolist() == s["act"]
    z, u, m = oracle.preact(L, x)
    assert z.tolist() == s["z"]
    assert m.tolist() == s["exact_mask"]
    if kind == "reglu":
        assert u.tolist() == s["u"]
    assert oracle.ffn_masked(L, x, m).tolist() == s["y"]
    ys, acts = oracle.ffn_sparse(L, x, oracle.compact(m))
    assert ys.tolist() == s["y"]
    assert acts.tolist() == [a for a, mm in zip(s["act"], s["exact_mask"]) if mm]


def test_hand_predictor():
    L, x, _, p = _hand_layer("relu")
    hid, logits, mask = oracle.predict(L, x)
    assert hid.tolist() == p["hid"]
    assert logits.tolist() == p["logits"]
    assert mask.tolist() == p["mask_tau_0.5"]
    L6 = dict(L, t=oracle.logit_threshold(0.6))
    assert oracle.predict(L6, x)[2].tolist() == p["mask_tau_0.6"]


# --------------------------------------------------------------------------- #
# threshold
# --------------------------------------------------------------------------- #
def test_threshold_equals_sigmoid_rule():
    """logit > ln(tau/(1-tau)) selects the same neurons as sigmoid(logit) > tau
    away from the boundary; at exactly t the neuron is inactive."""
    rng = np.random.default_rng(2)
    lg = (rng.standard_normal(20000) * 4).astype(np.float32)
    for tau in (0.3, 0.45, 0.5, 0.6, 0.9):
        t = oracle.logit_threshold(tau)
        m = oracle.threshold(lg, t)
        sig = 1.0 / (1.0 + np.exp(-lg.astype(np.float64)))
        far = np.abs(lg.astype(np.float64) - t) > 1e-6
        assert np.array_equal(m[far], (sig > tau)[far].astype(np.uint8))
    assert oracle.threshold(np.array([0.0, -0.0, 1e-45, -1e-45], np.float32), 0.0).tolist() == \
        [0, 0, 1, 0]
    assert oracle.logit_threshold(0.5) == 0.0
    assert oracle.threshold(np.array([np.nan], np.float32), 0.0).tolist() == [0]


def test_predictor_linear_special_case():
    """W1 = I, b1 = 0 and x >= 0 make the hidden layer the identity, so the
    logits are the affine map W2 x + b2 (numpy matmul)."""
    rng = np.random.default_rng(3)
    d = r = 16
    F = 40
    x = rng.random(d)
    L = dict(d=d, d_ffn=F, r=r, p_dtype="f32", p_w1=np.eye(d, dtype=np.float32),
             p_b1=np.zeros(r, np.float32), p_w2=rng.standard_normal((F, r)).astype(np.float32),
             p_b2=rng.standard_normal(F).astype(np.float32), t=0.0)
    hid, logits, mask = oracle.predict(L, x)
    assert np.array_equal(hid, x)
    ref = L["p_w2"].astype(np.float64) @ x + L["p_b2"]
    np.testing.assert_allclose(logits, ref, rtol=1e-13, atol=1e-13)
    assert np.array_equal(mask, (ref > 0).astype(np.uint8))


def test_predictor_hidden_relu_kills_negative_units():
    """With W2 reading only hidden units whose pre-activation is negative, every
    logit equals its bias."""
    d, r, F = 4, 2, 3
    L = dict(d=d, d_ffn=F, r=r, p_dtype="f32",
             p_w1=np.array([[1, 0, 0, 0], [-1, 0, 0, 0]], np.float32),
             p_b1=np.zeros(r, np.float32),
             p_w2=np.array([[0, 7], [0, -3], [0, 1]], np.float32),
             p_b2=np.array([0.5, -0.5, 0.0], np.float32), t=0.0)
    hid, logits, mask = oracle.predict(L, np.array([2.0, 1, 1, 1]))
    assert hid.tolist() == [2.0, 0.0]
    assert logits.tolist() == [0.5, -0.5, 0.0]
    assert mask.tolist() == [1, 0, 0]


# --------------------------------------------------------------------------- #
# compaction and union
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("n", [0, 1, 5, 12, 16])
def test_compact_exhaustive(n):
    for bits in range(1 << n):
        m = np.array([(bits >> i) & 1 for i in range(n)], dtype=np.uint8)
        idx = oracle.compact(m)
        assert np.array_equal(idx, np.flatnonzero(m))
        if n and bits in (0, (1 << n) - 1):
            assert idx.size == (0 if bits == 0 else n)


def test_compact_random_large():
    rng = np.random.default_rng(4)
    for n in (100_000, 28672, 49152):
        for p in (0.0, 0.01, 0.1, 0.5, 1.0):
            m = (rng.random(n) < p).astype(np.uint8)
            m[m == 1] = rng.integers(1, 256, size=int(m.sum()), dtype=np.uint8)  # any nonzero
            idx = oracle.compact(m)
            assert idx.dtype == np.int32
            assert idx.size == np.count_nonzero(m)
            assert np.all(np.diff(idx) > 0)
            assert np.array_equal(idx, np.flatnonzero(m))


def test_union():
    rng = np.random.default_rng(5)
    for B in (1, 2, 4, 16):
        masks = (rng.random((B, 300)) < 0.1).astype(np.uint8)
        U = oracle.union(masks)
        assert np.array_equal(U, masks.any(axis=0).astype(np.uint8))
        assert U.sum() >= masks.sum(axis=1).max()
        if B == 1:
            assert np.array_equal(U, masks[0])
    # exhaustive over two 3-bit masks
    for a, b in itertools.product(range(8), repeat=2):
        m = np.array([[(a >> i) & 1 for i in range(3)], [(b >> i) & 1 for i in range(3)]],
                     np.uint8)
        assert oracle.union(m).tolist() == [((a | b) >> i) & 1 for i in range(3)]


# --------------------------------------------------------------------------- #
# FFN invariants and special cases
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("kind", ["relu", "reglu"])
@pytest.mark.parametrize("w_dtype", ["f32", "f16"])
def test_exact_mask_and_all_ones_equal_dense(kind, w_dtype):
    """Sparse FFN on the exact mask (z > 0) and on the all-ones mask equal the
    dense FFN exactly: the skipped terms are exact zeros."""
    rng = np.random.default_rng(6)
    L = _rand_layer(rng, kind, 24, 70, w_dtype=w_dtype)
    for _ in range(5):
        x = rng.standard_normal(24)
        y, act = oracle.ffn_dense(L, x)
        _, _, em = oracle.preact(L, x)
        assert 0 < em.sum() < 70
        assert np.array_equal(oracle.ffn_masked(L, x, em), y)
        assert np.array_equal(oracle.ffn_masked(L, x, np.ones(70, np.uint8)), y)
        assert np.all(act[em == 0] == 0)


@pytest.mark.parametrize("kind", ["relu", "reglu"])
def test_predicted_mask_equals_dense_with_zeroed_neurons(kind):
    """Sparse FFN on the predictor's mask equals the dense FFN of the same layer
    with the down column of every non-predicted neuron set to zero."""
    rng = np.random.default_rng(7)
    L = _rand_layer(rng, kind, 20, 50, r=6)
    for _ in range(5):
        x = rng.standard_normal(20)
        _, _, pm = oracle.predict(L, x)
        Lz = dict(L, w_down_t=L["w_down_t"] * pm[:, None].astype(np.float32))
        assert np.array_equal(oracle.ffn_masked(L, x, pm), oracle.ffn_dense(Lz, x)[0])


@pytest.mark.parametrize("kind", ["relu", "reglu"])
def test_masked_ffn_brute_force_all_masks(kind):
    """For every one of the 2^10 masks, the masked FFN is the sum of the
    single-neuron FFNs it contains, and a single neuron i gives
    a_i * W_downT[i] with a_i from the closed form."""
    rng = np.random.default_rng(8)
    d, F = 5, 10
    L = _rand_layer(rng, kind, d, F)
    x = rng.standard_normal(d)
    wu = L["w_up"].astype(np.float64)
    wd = L["w_down_t"].astype(np.float64)
    b = L["b_act"].astype(np.float64)
    single = []
    for i in range(F):
        if kind == "relu":
            a = max(float(wu[i] @ x + b[i]), 0.0)
        else:
            a = max(float(L["w_gate"][i].astype(np.float64) @ x + b[i]), 0.0) * float(wu[i] @ x)
        single.append(a * wd[i])
        one = np.zeros(F, np.uint8)
        one[i] = 1
        np.testing.assert_allclose(oracle.ffn_masked(L, x, one), a * wd[i], rtol=1e-13,
                                   atol=1e-15)
    single = np.array(single)
    for bits in range(1 << F):
        m = np.array([(bits >> i) & 1 for i in range(F)], np.uint8)
        y = oracle.ffn_masked(L, x, m)
        np.testing.assert_allclose(y, single[m == 1].sum(axis=0), rtol=1e-12, atol=1e-14)


def test_all_active_relu_is_affine_map():
    """With every pre-activation positive the ReLU FFN is the affine map
    W_down (W_up x + b) -- a plain matrix product."""
    rng = np.random.default_rng(9)
    d, F = 12, 33
    L = _rand_layer(rng, "relu", d, F)
    L["b_act"] = np.full(F, 100.0, np.float32)
    x = rng.standard_normal(d)
    y, _ = oracle.ffn_dense(L, x)
    ref = L["w_down_t"].astype(np.float64).T @ (L["w_up"].astype(np.float64) @ x + 100.0)
    np.testing.assert_allclose(y, ref, rtol=1e-12)


def test_all_active_reglu_is_quadratic_form():
    """With every gate pre-activation positive the ReGLU FFN is
    W_down ((W_gate x + b) * (W_up x))."""
    rng = np.random.default_rng(10)
    d, F = 12, 33
    L = _rand_layer(rng, "reglu", d, F)
    L["b_act"] = np.full(F, 100.0, np.float32)
    x = rng.standard_normal(d)
    y, _ = oracle.ffn_dense(L, x)
    g = L["w_gate"].astype(np.float64) @ x + 100.0
    u = L["w_up"].astype(np.float64) @ x
    ref = L["w_down_t"].astype(np.float64).T @ (g * u)
    np.testing.assert_allclose(y, ref, rtol=1e-12)


def test_homogeneity_without_bias():
    """Without bias, ReLU FFN is positively homogeneous of degree 1 and ReGLU of
    degree 2 (powers of two keep it exact)."""
    rng = np.random.default_rng(11)
    for kind, deg in (("relu", 1), ("reglu", 2)):
        L = _rand_layer(rng, kind, 16, 40)
        L["b_act"] = None
        x = rng.standard_normal(16)
        y1 = oracle.ffn_dense(L, x)[0]
        y4 = oracle.ffn_dense(L, 4.0 * x)[0]
        assert np.array_equal(y4, (4.0 ** deg) * y1)


def test_empty_mask_gives_zero():
    rng = np.random.default_rng(12)
    L = _rand_layer(rng, "reglu", 8, 20)
    y = oracle.ffn_masked(L, rng.standard_normal(8), np.zeros(20, np.uint8))
    assert np.all(y == 0.0)


def test_sparse_rejects_bad_index():
    rng = np.random.default_rng(13)
    L = _rand_layer(rng, "relu", 8, 20)
    with pytest.raises(ValueError):
        oracle.ffn_sparse(L, np.zeros(8), np.array([3, 20], np.int32))


def test_q4_0_ffn_matches_values():
    """A 4-bit layer gives the same FFN as the fp32 layer holding its exact
    dequantised values (which are exactly representable in fp32)."""
    rng = np.random.default_rng(14)
    d, F = 64, 24

    def q4():
        blocks = np.zeros((F, d // 32, 18), np.uint8)
        s = np.abs(rng.standard_normal((F, d // 32)) * 0.05).astype(np.float16)
        blocks[:, :, 0:2] = s.view(np.uint8).reshape(F, d // 32, 2)
        blocks[:, :, 2:] = rng.integers(0, 256, size=(F, d // 32, 16), dtype=np.uint8)
        return blocks.reshape(F, -1)
    Lq = dict(kind="relu", w_dtype="q4_0", d=d, d_ffn=F, w_gate=None, w_up=q4(),
              w_down_t=q4(), b_act=rng.standard_normal(F).astype(np.float32) * 0.1)
    Lf = dict(Lq, w_dtype="f32", w_up=oracle.deq(Lq["w_up"], "q4_0", d).astype(np.float32),
              w_down_t=oracle.deq(Lq["w_down_t"], "q4_0", d).astype(np.float32))
    x = rng.standard_normal(d)
    assert np.array_equal(oracle.ffn_dense(Lq, x)[0], oracle.ffn_dense(Lf, x)[0])


# --------------------------------------------------------------------------- #
# rms norm and decode glue
# --------------------------------------------------------------------------- #
def test_rmsnorm_closed_forms():
    d = 64
    c = 3.0
    n = oracle.rmsnorm(np.full(d, c), 1e-5)
    np.testing.assert_allclose(n, np.full(d, c / math.sqrt(c * c + 1e-5)), rtol=1e-15)
    assert np.all(oracle.rmsnorm(np.zeros(d), 1e-5) == 0)
    x = np.array([3.0, 4.0])  # mean square 12.5
    np.testing.assert_allclose(oracle.rmsnorm(x, 0.0), x / math.sqrt(12.5), rtol=1e-15)


def test_decode_zero_down_leaves_h_unchanged():
    rng = np.random.default_rng(15)
    L = _rand_layer(rng, "reglu", 16, 30)
    L["w_down_t"] = np.zeros_like(L["w_down_t"])
    h = rng.standard_normal((3, 16))
    out = oracle.decode_layer(L, h, 1e-5)
    assert np.array_equal(out["h"], h)


def test_decode_layer_batch_union():
    """Every token of a batch is computed on the union of the batch's masks."""
    rng = np.random.default_rng(16)
    L = _rand_layer(rng, "relu", 16, 40, r=8)
    h = rng.standard_normal((4, 16)) * 2.0
    out = oracle.decode_layer(L, h, 1e-5)
    assert np.array_equal(out["union"], out["masks"].any(axis=0).astype(np.uint8))
    for b in range(4):
        n = oracle.rmsnorm(h[b], 1e-5)
        assert np.array_equal(out["n"][b], n)
        assert np.array_equal(out["y"][b], oracle.ffn_masked(L, n, out["union"]))


@pytest.mark.parametrize("case", [0, 1])
def test_decode_layer_per_token_thresholds_hand(case):
    """Per-token logit thresholds (adaptive thresholding) on the hand-derived
    two-token example: each token's own mask, their union, and every token
    computed on the union (golden/hand_adaptive.json)."""
    g = load_golden("hand_adaptive.json")
    L, _, _, _ = _hand_layer("relu")
    c = g["cases"][case]
    out = oracle.decode_layer(L, np.asarray(g["h"], np.float64), g["eps"],
                              thresholds=np.asarray(c["t"], np.float32))
    assert np.array_equal(out["logits"], np.asarray(g["logits"], np.float64))
    assert np.array_equal(out["masks"], np.asarray(c["masks"], np.uint8))
    assert np.array_equal(out["union"], np.asarray(c["union"], np.uint8))
    assert np.array_equal(out["y"], np.asarray(c["y"], np.float64))
    assert np.array_equal(out["h"], np.asarray(c["h_next"], np.float64))


def test_decode_per_token_thresholds_reduce_to_the_layer_threshold():
    """Thresholds all equal to the layer's own t give the plain decode bit for
    bit; a threshold below every logit for one token makes the union all ones,
    so every token then gets the dense FFN of its input."""
    rng = np.random.default_rng(17)
    L = _rand_layer(rng, "reglu", 16, 40, r=8)
    L["t"] = float(np.float32(0.1))
    h = rng.standard_normal((3, 16))
    plain = oracle.decode_layer(L, h, 1e-5)
    same = oracle.decode_layer(L, h, 1e-5, thresholds=np.full(3, L["t"], np.float32))
    for k in ("logits", "masks", "union", "y", "h"):
        assert np.array_equal(plain[k], same[k]), k
    low = oracle.decode_layer(L, h, 1e-5, thresholds=np.float32([1e30, -1e30, 1e30]))
    assert np.all(low["masks"][1] == 1) and np.all(low["masks"][0] == 0)
    for b in range(3):
        n = oracle.rmsnorm(h[b], 1e-5)
        assert np.array_equal(low["y"][b], oracle.ffn_dense(L, n)[0])
    # a stack with per-layer, per-token thresholds runs each layer with its row
    L2 = dict(L, t=-0.3)
    T = np.float32([[0.1, 0.1, 0.1], [-0.3, -0.3, -0.3]])
    assert np.array_equal(oracle.decode_step([L, L2], h, 1e-5, thresholds=T),
                          oracle.decode_step([L, L2], h, 1e-5))


def _one_neuron_layer(v):
    """d = 4, two ReLU neurons, predictor fixed to fire neuron 0 only (zero
    weights, logit biases +5 / -5); neuron 0 reads n[0] and writes v, neuron 1
    would add 1000 everywhere if it were ever computed."""
    f = lambda a: np.asarray(a, dtype=np.float32)  # noqa: E731
    return dict(kind="relu", w_dtype="f32", p_dtype="f32", d=4, d_ffn=2, r=1, w_gate=None,
                w_up=f([[1, 0, 0, 0], [1, 1, 1, 1]]), w_down_t=f([v, [1000] * 4]),
                b_act=f([0, 0]), p_w1=f([[0, 0, 0, 0]]), p_b1=f([0]), p_w2=f([[0], [0]]),
                p_b2=f([5, -5]), t=0.0)


def test_decode_step_two_layers_closed_form():
    """A constant vector h = a stays constant through these layers: each adds
    b * max(s(h), 0), s(z) = z / sqrt(z^2 + eps) being the RMS-normalised
    entry (all neurons but the first predicted off).  The order of the layers,
    the residual, the ReLU and the carried state all show in the result."""
    eps, a, b1, b2 = 0.5, 1.5, 0.25, -2.0
    A, B = _one_neuron_layer([b1] * 4), _one_neuron_layer([b2] * 4)
    step = lambda z, b: z + b * max(z / math.sqrt(z * z + eps), 0.0)  # noqa: E731
    want_ab = step(step(a, b1), b2)
    got = oracle.decode_step([A, B], np.full((1, 4), a), eps)
    np.testing.assert_allclose(got, np.full((1, 4), want_ab), rtol=1e-14)
    # the other order: B drives h negative, so A's neuron stays off
    want_ba = step(step(a, b2), b1)
    assert step(a, b2) < 0 and want_ba == step(a, b2)
    got_ba = oracle.decode_step([B, A], np.full((1, 4), a), eps)
    np.testing.assert_allclose(got_ba, np.full((1, 4), want_ba), rtol=1e-14)
    assert abs(want_ab - want_ba) > 1e-3


# --------------------------------------------------------------------------- #
# profile and hot-first permutation
# --------------------------------------------------------------------------- #
def test_profile_counts_brute_force():
    rng = np.random.default_rng(17)
    L = _rand_layer(rng, "reglu", 10, 25)
    X = rng.standard_normal((30, 10))
    counts = oracle.profile(L, X)
    brute = np.zeros(25, np.int64)
    for x in X:
        brute += oracle.preact(L, x)[2]
    assert np.array_equal(counts, brute)


def test_hot_first_perm_properties():
    rng = np.random.default_rng(18)
    counts = rng.integers(0, 6, size=500)
    perm = oracle.hot_first_perm(counts)
    assert np.array_equal(np.sort(perm), np.arange(500))
    c = counts[perm]
    assert np.all(np.diff(c) <= 0)
    for v in np.unique(counts):  # ties keep ascending original index
        assert np.all(np.diff(perm[c == v]) > 0)
    assert np.array_equal(perm, np.lexsort((np.arange(500), -counts)))


def test_permuted_layer_same_output():
    rng = np.random.default_rng(19)
    L = _rand_layer(rng, "reglu", 16, 40, r=8)
    X = rng.standard_normal((20, 16))
    perm = oracle.hot_first_perm(oracle.profile(L, X))
    P = oracle.permute_layer(L, perm)
    for x in X[:5]:
        y0 = oracle.ffn_dense(L, x)[0]
        y1 = oracle.ffn_dense(P, x)[0]
        np.testing.assert_allclose(y1, y0, rtol=1e-12, atol=1e-14)
        m0 = oracle.predict(L, x)[2]
        m1 = oracle.predict(P, x)[2]
        assert np.array_equal(m1, m0[perm])
        # stored indices map back through perm to the original active neurons
        assert np.array_equal(np.sort(perm[oracle.compact(m1)]), oracle.compact(m0))


def test_prototype_harness_structure():
    """The Guide's Step 4 harness: budget 0.2 of 8192 neurons is 1638 hot; its
    hand-built mask holds 400 + 50 = 450 neurons (5.49%); hot share of its
    synthetic activations is about 0.774."""
    g = load_golden("prototype_harness.json")
    F = g["intermediate_size"]
    rng = np.random.default_rng(20)
    acts = np.zeros((g["profiled_tokens"], F), np.uint8)
    acts[:, :g["hot_block"]] = rng.random((g["profiled_tokens"], g["hot_block"])) > 1 - g["p_hot"]
    acts[:, g["hot_block"]:] = rng.random((g["profiled_tokens"], F - g["hot_block"])) > \
        1 - g["p_cold"]
    counts = acts.sum(axis=0)
    k_hot, share = oracle.hot_share(counts, g["gpu_budget_ratio"])
    assert k_hot == g["k_hot"]
    assert abs(share - g["expected_hot_share_approx"]) < g["hot_share_tolerance"]
    perm = oracle.hot_first_perm(counts)
    hot, cold = perm[:k_hot], perm[k_hot:]
    mask = np.zeros(F, np.uint8)
    mask[hot[:g["mask_hot"]]] = 1
    mask[cold[:g["mask_cold"]]] = 1
    idx = oracle.compact(mask)
    assert idx.size == g["mask_active"]
    assert round(100.0 * idx.size / F, 2) == g["mask_active_percent_2dp"]
