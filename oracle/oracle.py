"""numpy front end of the C oracle (test infrastructure only).

A layer is a plain dict of numpy arrays and ints:

  kind      "relu" (non-gated up/down), "reglu" or "swiglu" (gated; SiLU
            on the gate for SwiGLU)
  w_dtype   "f32" | "f16" | "q4_0"   storage of w_gate / w_up / w_down_t
  p_dtype   "f32" | "f16" | "fp8"    storage of p_w1 / p_w2
  d, d_ffn, r
  w_gate    [d_ffn, d]  (ReGLU only; None for ReLU)
  w_up      [d_ffn, d]
  w_down_t  [d_ffn, d]  W_down transposed: row i is neuron i's output column
  b_act     float32 [d_ffn] or None: bias of the activated projection
  p_w1      [r, d],  p_b1 float32 [r]
  p_w2      [d_ffn, r],  p_b2 float32 [d_ffn]
  t         logit threshold (float32 value); a neuron is predicted active
            when its logit is > t
  dense_prefix  optional k: the first k neurons are always active and not
            scored (logit +inf)

fp16 arrays are numpy float16; 4-bit arrays are uint8 [rows, cols/32*18] in
the 18-byte block layout described in oracle.c; fp8 (OCP E4M3) matrices are a
flat uint8 buffer of rows*cols codes followed by rows fp32 scales.

Sources (page titles abbreviated): [Guide] "PowerInfer Guide: Exploiting
Activation Sparsity for LLM AI"; [x64] "PowerInfer_x64: Neuron-Level Sparse
Inference Makes Large Models Fly on Consumer GPUs".
"""
import ctypes as C
import math
import os

import numpy as np

from . import LIB, build

_DT = {"f32": 0, "f16": 1, "q4_0": 2, "fp8": 3}
_KIND = {"relu": 0, "reglu": 1, "swiglu": 2}

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = C.CDLL(LIB)
        vp, i64, i32, dp = C.c_void_p, C.c_int64, C.c_int, C.c_double
        lib.oracle_f16_to_f64.argtypes = [C.c_uint16]
        lib.oracle_f16_to_f64.restype = dp
        lib.oracle_e4m3_to_f64.argtypes = [C.c_uint8]
        lib.oracle_e4m3_to_f64.restype = dp
        lib.oracle_deq_row.argtypes = [vp, i32, i64, i64, i64, vp]
        lib.oracle_deq_row.restype = i32
        lib.oracle_predict.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, dp, i64, vp, vp,
                                       vp]
        lib.oracle_predict.restype = i32
        lib.oracle_threshold.argtypes = [vp, i64, C.c_float, vp]
        lib.oracle_threshold.restype = None
        lib.oracle_compact.argtypes = [vp, i64, vp]
        lib.oracle_compact.restype = i64
        lib.oracle_union.argtypes = [vp, i64, i64, vp]
        lib.oracle_union.restype = None
        lib.oracle_ffn_dense.argtypes = [i32, i32, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_ffn_dense.restype = i32
        lib.oracle_ffn_sparse.argtypes = [i32, i32, i64, i64, vp, vp, vp, vp, vp, vp, i64, vp, vp]
        lib.oracle_ffn_sparse.restype = i64
        lib.oracle_ffn_masked.argtypes = [i32, i32, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_ffn_masked.restype = i64
        lib.oracle_preact.argtypes = [i32, i32, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_preact.restype = i32
        lib.oracle_profile.argtypes = [i32, i32, i64, i64, vp, vp, vp, vp, i64, vp]
        lib.oracle_profile.restype = i32
        lib.oracle_rmsnorm.argtypes = [vp, i64, dp, vp]
        lib.oracle_rmsnorm.restype = None
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def _x64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _rc(rc, what):
    if rc < 0:
        raise ValueError(f"oracle {what} failed with status {rc}")
    return rc


# --------------------------------------------------------------------------- #
# element formats
# --------------------------------------------------------------------------- #
def f16_bits_to_f64(bits):
    """binary16 bit patterns (uint16 array) -> float64, one C call per value."""
    lib = _load()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    out = np.array([lib.oracle_f16_to_f64(int(b)) for b in flat], dtype=np.float64)
    return out.reshape(np.shape(bits))


def e4m3_to_f64(codes):
    """OCP E4M3 codes (uint8 array) -> float64, one C call per value."""
    lib = _load()
    flat = np.asarray(codes, dtype=np.uint8).ravel()
    out = np.array([lib.oracle_e4m3_to_f64(int(c)) for c in flat], dtype=np.float64)
    return out.reshape(np.shape(codes))


def deq(w, dtype, cols):
    """Whole [rows, cols] weight matrix widened to float64 (row by row).  An
    fp8 matrix is the flat buffer of its codes followed by its row scales."""
    lib = _load()
    w = _c(w)
    rows = w.size // (cols + 4) if dtype == "fp8" else w.shape[0]
    out = np.empty((rows, cols), dtype=np.float64)
    for i in range(rows):
        _rc(lib.oracle_deq_row(_p(w), _DT[dtype], rows, cols, i, _p(out[i])), "deq_row")
    return out


# --------------------------------------------------------------------------- #
# predictor, threshold, compaction, union
# --------------------------------------------------------------------------- #
def predict(layer, x):
    """One token: returns (hid [r], logits [d_ffn], mask [d_ffn] uint8)."""
    lib = _load()
    L = layer
    x = _x64(x)
    hid = np.empty(L["r"], np.float64)
    logits = np.empty(L["d_ffn"], np.float64)
    mask = np.empty(L["d_ffn"], np.uint8)
    w1, w2 = _c(L["p_w1"]), _c(L["p_w2"])
    b1, b2 = _c(L["p_b1"], np.float32), _c(L["p_b2"], np.float32)
    _rc(lib.oracle_predict(L["d"], L["d_ffn"], L["r"], _DT[L["p_dtype"]], _p(w1), _p(b1),
                           _p(w2), _p(b2), _p(x), float(L["t"]),
                           int(L.get("dense_prefix", 0) or 0), _p(hid), _p(logits), _p(mask)),
        "predict")
    return hid, logits, mask


def threshold(logits_f32, t):
    lib = _load()
    lg = _c(np.asarray(logits_f32), np.float32)
    mask = np.empty(lg.size, np.uint8)
    lib.oracle_threshold(_p(lg), lg.size, float(np.float32(t)), _p(mask))
    return mask.reshape(lg.shape)


def compact(mask):
    """Ascending indices of the set mask entries (int32)."""
    lib = _load()
    m = _c(np.asarray(mask), np.uint8).ravel()
    idx = np.empty(max(1, m.size), np.int32)
    n = lib.oracle_compact(_p(m), m.size, _p(idx))
    return idx[:n].copy()


def union(masks):
    lib = _load()
    m = _c(np.asarray(masks), np.uint8)
    if m.ndim == 1:
        m = m[None, :]
    out = np.empty(m.shape[1], np.uint8)
    lib.oracle_union(_p(m), m.shape[0], m.shape[1], _p(out))
    return out


def logit_threshold(tau):
    """t = ln(tau / (1 - tau)) in binary64 from tau as a binary32 value (the
    precision a layer carries it in), rounded once to binary32.

    [Guide] section 3 thresholds sigmoid(logit) > tau; sigmoid is increasing,
    so the same neurons satisfy logit > t."""
    tau32 = float(np.float32(tau))
    if not 0.0 < tau32 < 1.0:
        raise ValueError("tau must lie in (0, 1)")
    return float(np.float32(math.log(tau32 / (1.0 - tau32))))


# --------------------------------------------------------------------------- #
# FFN
# --------------------------------------------------------------------------- #
def _ffn_args(L):
    wg = _c(L["w_gate"]) if L["kind"] != "relu" else None
    wu, wd = _c(L["w_up"]), _c(L["w_down_t"])
    b = _c(L["b_act"], np.float32) if L.get("b_act") is not None else None
    return wg, wu, wd, b


def ffn_dense(layer, x):
    """Dense FFN of one token over every neuron: (y [d], act [d_ffn])."""
    lib = _load()
    L = layer
    wg, wu, wd, b = _ffn_args(L)
    x = _x64(x)
    y = np.empty(L["d"], np.float64)
    act = np.empty(L["d_ffn"], np.float64)
    _rc(lib.oracle_ffn_dense(_KIND[L["kind"]], _DT[L["w_dtype"]], L["d"], L["d_ffn"], _p(wg),
                             _p(wu), _p(wd), _p(b), _p(x), _p(y), _p(act)), "ffn_dense")
    return y, act


def ffn_sparse(layer, x, idx):
    """FFN of one token over the listed neurons: (y [d], act [count])."""
    lib = _load()
    L = layer
    wg, wu, wd, b = _ffn_args(L)
    x = _x64(x)
    idx = _c(np.asarray(idx), np.int32)
    y = np.empty(L["d"], np.float64)
    act = np.empty(max(1, idx.size), np.float64)
    _rc(lib.oracle_ffn_sparse(_KIND[L["kind"]], _DT[L["w_dtype"]], L["d"], L["d_ffn"], _p(wg),
                              _p(wu), _p(wd), _p(b), _p(x), _p(idx), idx.size, _p(y),
                              _p(act)), "ffn_sparse")
    return y, act[:idx.size]


def ffn_masked(layer, x, mask):
    """FFN of one token over the neurons whose mask entry is set: y [d]."""
    lib = _load()
    L = layer
    wg, wu, wd, b = _ffn_args(L)
    x = _x64(x)
    m = _c(np.asarray(mask), np.uint8)
    y = np.empty(L["d"], np.float64)
    _rc(lib.oracle_ffn_masked(_KIND[L["kind"]], _DT[L["w_dtype"]], L["d"], L["d_ffn"], _p(wg),
                              _p(wu), _p(wd), _p(b), _p(x), _p(m), _p(y)), "ffn_masked")
    return y


def preact(layer, x):
    """(z [d_ffn], u [d_ffn], exact mask z > 0) of one token."""
    lib = _load()
    L = layer
    wg, wu, _, b = _ffn_args(L)
    x = _x64(x)
    z = np.empty(L["d_ffn"], np.float64)
    u = np.empty(L["d_ffn"], np.float64)
    m = np.empty(L["d_ffn"], np.uint8)
    _rc(lib.oracle_preact(_KIND[L["kind"]], _DT[L["w_dtype"]], L["d"], L["d_ffn"], _p(wg),
                          _p(wu), _p(b), _p(x), _p(z), _p(u), _p(m)), "preact")
    return z, u, m


# --------------------------------------------------------------------------- #
# profile and hot-first order
# --------------------------------------------------------------------------- #
def profile(layer, X):
    """Per-neuron count of the tokens X [N, d] with a positive pre-activation."""
    lib = _load()
    L = layer
    wg, wu, _, b = _ffn_args(L)
    X = _x64(np.atleast_2d(X))
    counts = np.empty(L["d_ffn"], np.int32)
    _rc(lib.oracle_profile(_KIND[L["kind"]], _DT[L["w_dtype"]], L["d"], L["d_ffn"], _p(wg),
                           _p(wu), _p(b), _p(X), X.shape[0], _p(counts)), "profile")
    return counts


def hot_first_perm(counts):
    """Stored-to-original neuron order, hottest first ([Guide] Step 1 sorts the
    neurons by descending activation count).  Ties keep ascending index, so
    the order is unique."""
    c = [int(v) for v in np.asarray(counts).ravel()]
    return np.array(sorted(range(len(c)), key=lambda i: (-c[i], i)), dtype=np.int32)


def hot_share(counts, beta):
    """Share of all activations that falls on the top int(beta * d_ffn) neurons
    ([Guide] Step 1 partition by budget ratio): (k_hot, share)."""
    c = np.asarray(counts, dtype=np.int64)
    k_hot = int(c.size * beta)
    perm = hot_first_perm(c)
    total = int(c.sum())
    return k_hot, int(c[perm[:k_hot]].sum()) / max(1, total)


def permute_layer(layer, perm):
    """Neuron i of the returned layer is neuron perm[i] of `layer`: rows of the
    gate, up and transposed-down weights, the activation bias and the
    predictor's second layer move together; the predictor's first layer and
    the threshold are unchanged."""
    L = dict(layer)
    perm = np.asarray(perm, dtype=np.int64)
    for k in ("w_gate", "w_up", "w_down_t", "b_act", "p_w2", "p_b2"):
        if L.get(k) is not None:
            L[k] = np.ascontiguousarray(np.asarray(layer[k])[perm])
    return L


# --------------------------------------------------------------------------- #
# decode glue
# --------------------------------------------------------------------------- #
def rmsnorm(x, eps):
    lib = _load()
    x = _x64(x)
    out = np.empty_like(x)
    lib.oracle_rmsnorm(_p(x), x.size, float(eps), _p(out))
    return out


def decode_layer(layer, h, eps, mask=None, thresholds=None):
    """One layer of the decode step for a batch h [B, d] (binary64):
    n_b = rmsnorm(h_b); M = union over the batch of the predicted masks (or
    the given `mask`); h_b + FFN over M of n_b.

    thresholds: optional per-token logit thresholds [B] (binary32 values)
    replacing the layer's t, token b's mask being logit > thresholds[b]
    ([Guide] "Production Engineering" section 2, adaptive dynamic
    thresholding: tau varies by token).

    Returns dict(h=h_next, n=[B,d], logits=[B,d_ffn], masks=[B,d_ffn],
    union=[d_ffn], y=[B,d])."""
    h = np.atleast_2d(_x64(h))
    B = h.shape[0]
    n = np.stack([rmsnorm(h[b], eps) for b in range(B)])
    if thresholds is None:
        preds = [predict(layer, n[b]) for b in range(B)]
    else:
        tv = np.asarray(thresholds, np.float32).reshape(B)
        preds = [predict(dict(layer, t=float(tv[b])), n[b]) for b in range(B)]
    logits = np.stack([p[1] for p in preds])
    masks = np.stack([p[2] for p in preds])
    U = union(masks) if mask is None else np.asarray(mask, np.uint8)
    y = np.stack([ffn_masked(layer, n[b], U) for b in range(B)])
    return dict(h=h + y, n=n, logits=logits, masks=masks, union=U, y=y)


def decode_step(layers, x, eps, thresholds=None):
    """The whole stack for one batch of tokens x [B, d]: returns h [B, d].
    thresholds: optional per-layer, per-token logit thresholds [L, B]."""
    h = np.atleast_2d(_x64(x))
    for l, L in enumerate(layers):
        h = decode_layer(L, h, eps, thresholds=None if thresholds is None
                         else np.asarray(thresholds)[l])["h"]
    return h
