"""Exercise every function of the C oracle on small inputs of every storage
type, with a few identities checked along the way.  Run by
test_oracle_sanitized.py in a child process whose oracle library is the
AddressSanitizer + UndefinedBehaviorSanitizer build; numpy only."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402

rng = np.random.default_rng(7)


def q4_rows(rows, cols):
    nb = cols // 32
    blk = np.zeros((rows, nb, 18), np.uint8)
    blk[:, :, :2] = np.abs(rng.normal(0, 0.05, (rows, nb))).astype(np.float16) \
        .view(np.uint8).reshape(rows, nb, 2)
    blk[:, :, 2:] = rng.integers(0, 256, (rows, nb, 16), dtype=np.uint8)
    return blk.reshape(rows, nb * 18)


def layer(kind, w_dtype, p_dtype, d=64, F=96, r=16):
    def w(rows, cols, dt):
        if dt == "q4_0":
            return q4_rows(rows, cols)
        v = rng.normal(0, cols ** -0.5, (rows, cols))
        return v.astype(np.float16 if dt == "f16" else np.float32)
    return dict(kind=kind, w_dtype=w_dtype, p_dtype=p_dtype, d=d, d_ffn=F, r=r,
                w_gate=w(F, d, w_dtype) if kind == "reglu" else None, w_up=w(F, d, w_dtype),
                w_down_t=w(F, d, w_dtype), b_act=rng.normal(0, 0.3, F).astype(np.float32),
                p_w1=w(r, d, p_dtype), p_b1=np.zeros(r, np.float32), p_w2=w(F, r, p_dtype),
                p_b2=rng.normal(0, 0.3, F).astype(np.float32), t=np.float32(0.0), tau=0.5)


for h in (0x0000, 0x0001, 0x3C00, 0x7BFF, 0x7C00, 0xFC00, 0x7E00, 0x8000):
    oracle.f16_bits_to_f64(h)
for kind in ("relu", "reglu"):
    for w_dtype in ("f32", "f16", "q4_0"):
        for p_dtype in ("f32", "f16"):
            L = layer(kind, w_dtype, p_dtype)
            x = rng.normal(0, 1, (3, L["d"]))
            out = oracle.decode_layer(L, x, 1e-5)
            assert out["h"].shape == x.shape and np.all(np.isfinite(out["h"]))
            n = oracle.rmsnorm(x[0], 1e-5)
            hid, logits, mask = oracle.predict(L, n)
            assert np.array_equal(mask, oracle.threshold(logits.astype(np.float32), L["t"]))
            idx = oracle.compact(mask)
            ys, _ = oracle.ffn_sparse(L, n, idx)
            ym = oracle.ffn_masked(L, n, mask)
            assert np.array_equal(ys, ym)
            yd, act = oracle.ffn_dense(L, n)
            ones = np.ones(L["d_ffn"], np.uint8)
            assert np.array_equal(oracle.ffn_masked(L, n, ones), yd)
            _, _, exact = oracle.preact(L, n)
            assert np.array_equal(oracle.ffn_masked(L, n, exact), yd)
            oracle.ffn_sparse(L, n, np.zeros(0, np.int32))
            oracle.profile(L, x)
            oracle.deq(L["w_up"], L["w_dtype"], L["d"])
            oracle.deq(L["p_w2"], L["p_dtype"], L["r"])
            assert np.array_equal(oracle.union(np.stack([mask, ones * 0])), mask)
print("oracle under sanitizers: OK")
