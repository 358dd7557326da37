"""ctypes binding of libspffn (the C ABI in include/spffn.h).

Argument marshalling only: tensors are checked for device, dtype and layout,
their pointers and the current torch stream are passed to the C entry points,
and a negative status is raised as SpffnError.  Every step of the computation
runs in the library's HIP kernels; there is no CPU fallback, and importing
this module without the built library fails.
"""
import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspffn.so")

F32, F16, Q4_0 = 0, 1, 2
RELU, REGLU = 0, 1
MAX_BATCH = 16
DECODE_DENSE = 1
_DTYPES = {"f32": F32, "f16": F16, "q4_0": Q4_0}
_KINDS = {"relu": RELU, "reglu": REGLU}
_STATUS = {0: "OK", -1: "E_ARG", -2: "E_SHAPE", -3: "E_DTYPE", -4: "E_WORKSPACE", -5: "E_HIP"}


class SpffnError(RuntimeError):
    def __init__(self, status, where, text):
        super().__init__(f"{where}: {_STATUS.get(status, status)}: {text}")
        self.status = status


class LayerDesc(C.Structure):
    _fields_ = [("d", C.c_int32), ("d_ffn", C.c_int32), ("r", C.c_int32),
                ("kind", C.c_int32), ("w_dtype", C.c_int32), ("p_dtype", C.c_int32),
                ("tau", C.c_float), ("reserved", C.c_int32),
                ("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down_t", C.c_void_p),
                ("b_act", C.c_void_p), ("p_w1", C.c_void_p), ("p_b1", C.c_void_p),
                ("p_w2", C.c_void_p), ("p_b2", C.c_void_p)]


class Trace(C.Structure):
    _fields_ = [("h_in", C.c_void_p), ("union_mask", C.c_void_p), ("logits", C.c_void_p),
                ("events", C.c_void_p)]


# exported C symbols and their signatures (restype, argtypes)
_vp, _i32, _i64, _f32, _sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
SIGNATURES = {
    "spffn_layer_create": (_i32, [C.POINTER(LayerDesc), C.POINTER(_vp)]),
    "spffn_layer_destroy": (None, [_vp]),
    "spffn_layer_threshold": (_f32, [_vp]),
    "spffn_model_create": (_i32, [C.POINTER(_vp), _i32, _f32, C.POINTER(_vp)]),
    "spffn_model_destroy": (None, [_vp]),
    "spffn_layer_workspace_bytes": (_sz, [_vp, _i32]),
    "spffn_model_workspace_bytes": (_sz, [_vp, _i32]),
    "spffn_threshold": (_i32, [_vp, _i64, _f32, _vp, _vp]),
    "spffn_compact": (_i32, [_vp, _i32, _vp, _vp, _vp]),
    "spffn_predict": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spffn_forward": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spffn_decode_step": (_i32, [_vp, _vp, _vp, _i32, _i32, _vp, C.POINTER(Trace), _vp, _sz,
                                 _vp]),
    "spffn_decode_graph_create": (_i32, [_vp, _vp, _vp, _i32, _i32, _vp, _vp, _sz,
                                         C.POINTER(_vp)]),
    "spffn_graph_launch": (_i32, [_vp, _vp]),
    "spffn_graph_destroy": (None, [_vp]),
    "spffn_profile": (_i32, [_vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "spffn_hot_first_order": (_i32, [_vp, _i32, _vp, _vp]),
    "spffn_permute_rows": (_i32, [_vp, _vp, _vp, _i32, _i64, _vp]),
    "spffn_q4_0_repack": (_i32, [_vp, _vp, _i32, _i32, _vp]),
    "spffn_set_wait_limit": (_i32, [_i32]),
    "spffn_last_error": (C.c_char_p, []),
    "spffn_version": (C.c_char_p, []),
}

_lib = None


def load():
    """Load libspffn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status, where):
    if status != 0:
        raise SpffnError(status, where, load().spffn_last_error().decode())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _dev(t, dtype, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def version():
    return load().spffn_version().decode()


WAIT_LIMIT_DEFAULT = 1 << 18


def set_wait_limit(polls):
    """Test hook: polls before a down-projection workgroup of the single-token
    decode gives up on its chunk (NaN output instead of a hang); 0 makes it
    give up at once.  Applies to launches enqueued afterwards."""
    _check(load().spffn_set_wait_limit(int(polls)), "spffn_set_wait_limit")


class Layer:
    """One FFN layer + predictor on the GPU (a spffn_layer handle).

    `w` is a dict with kind, w_dtype, p_dtype, d, d_ffn, r, tau and device
    tensors w_gate (ReGLU) / w_up / w_down_t ([d_ffn, d], W_down transposed),
    b_act, p_w1, p_b1, p_w2, p_b2.  4-bit weights come in the 18-byte block
    layout and are split on the device (spffn_q4_0_repack); the handle keeps
    every tensor it points at alive."""

    def __init__(self, w):
        lib = load()
        self.kind, self.w_dtype, self.p_dtype = w["kind"], w["w_dtype"], w["p_dtype"]
        self.d, self.d_ffn, self.r = int(w["d"]), int(w["d_ffn"]), int(w["r"])
        self.tau = float(w["tau"])
        wd = {"f32": torch.float32, "f16": torch.float16, "q4_0": torch.uint8}[self.w_dtype]
        pd = {"f32": torch.float32, "f16": torch.float16}[self.p_dtype]
        t = {}
        for k in ("w_gate", "w_up", "w_down_t"):
            if w.get(k) is not None and (k != "w_gate" or self.kind == "reglu"):
                t[k] = _dev(w[k], wd, k)
                if self.w_dtype == "q4_0":
                    t[k] = q4_0_repack(t[k], self.d_ffn, self.d)
        t["b_act"] = _dev(w.get("b_act"), torch.float32, "b_act")
        for k in ("p_w1", "p_w2"):
            t[k] = _dev(w[k], pd, k)
        for k in ("p_b1", "p_b2"):
            t[k] = _dev(w[k], torch.float32, k)
        self.tensors = t
        desc = LayerDesc(d=self.d, d_ffn=self.d_ffn, r=self.r, kind=_KINDS[self.kind],
                         w_dtype=_DTYPES[self.w_dtype], p_dtype=_DTYPES[self.p_dtype],
                         tau=self.tau, reserved=0,
                         w_gate=_ptr(t.get("w_gate")), w_up=_ptr(t["w_up"]),
                         w_down_t=_ptr(t["w_down_t"]), b_act=_ptr(t["b_act"]),
                         p_w1=_ptr(t["p_w1"]), p_b1=_ptr(t["p_b1"]), p_w2=_ptr(t["p_w2"]),
                         p_b2=_ptr(t["p_b2"]))
        h = C.c_void_p()
        _check(lib.spffn_layer_create(C.byref(desc), C.byref(h)), "spffn_layer_create")
        self.handle = h
        self.t = float(lib.spffn_layer_threshold(h))

    def workspace_bytes(self, B):
        return int(load().spffn_layer_workspace_bytes(self.handle, B))

    def workspace(self, B, device=None):
        n = self.workspace_bytes(B)
        if n == 0:
            raise SpffnError(-2, "workspace_bytes", f"bad batch {B}")
        return torch.empty(n, dtype=torch.uint8, device=device or self.tensors["w_up"].device)

    def __del__(self):
        if getattr(self, "handle", None) is not None and _lib is not None:
            _lib.spffn_layer_destroy(self.handle)
            self.handle = None


class Model:
    """An ordered stack of Layer objects (a spffn_model handle)."""

    def __init__(self, layers, rms_eps=1e-5):
        lib = load()
        self.layers = list(layers)
        arr = (C.c_void_p * len(self.layers))(*[l.handle.value for l in self.layers])
        h = C.c_void_p()
        _check(lib.spffn_model_create(arr, len(self.layers), rms_eps, C.byref(h)),
               "spffn_model_create")
        self.handle = h
        self.rms_eps = rms_eps
        self.d = self.layers[0].d

    def workspace_bytes(self, B):
        return int(load().spffn_model_workspace_bytes(self.handle, B))

    def workspace(self, B):
        n = self.workspace_bytes(B)
        if n == 0:
            raise SpffnError(-2, "model_workspace_bytes", f"bad batch {B}")
        return torch.empty(n, dtype=torch.uint8, device=self.layers[0].tensors["w_up"].device)

    def __del__(self):
        if getattr(self, "handle", None) is not None and _lib is not None:
            _lib.spffn_model_destroy(self.handle)
            self.handle = None


# --------------------------------------------------------------------------- #
# entry points (same names as the C ABI, without the prefix)
# --------------------------------------------------------------------------- #
def threshold(logits, t, mask=None):
    logits = _dev(logits, torch.float32, "logits")
    if mask is None:
        mask = torch.empty(logits.shape, dtype=torch.uint8, device=logits.device)
    _dev(mask, torch.uint8, "mask")
    _check(load().spffn_threshold(_ptr(logits), logits.numel(), float(t), _ptr(mask), _stream()),
           "spffn_threshold")
    return mask


def compact(mask, idx=None, count=None):
    """(idx int32 [n], count int32 [1]) on the device; idx[:count] is valid."""
    mask = _dev(mask, None, "mask")
    if mask.dtype not in (torch.uint8, torch.bool):
        raise TypeError("mask must be uint8 or bool")
    n = mask.numel()
    if idx is None:
        idx = torch.empty(n, dtype=torch.int32, device=mask.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=mask.device)
    _dev(idx, torch.int32, "idx")
    _dev(count, torch.int32, "count")
    _check(load().spffn_compact(_ptr(mask), n, _ptr(idx), _ptr(count), _stream()),
           "spffn_compact")
    return idx, count


def _opt(v, shape, dtype, dev):
    if v is True:
        return torch.empty(shape, dtype=dtype, device=dev)
    if v is None or v is False:
        return None
    return v


def predict(layer, x, logits=True, mask=True, union=True, ws=None):
    """Returns dict(logits [B, d_ffn] f32, mask [B, d_ffn] u8, union [d_ffn] u8);
    pass False for an output that is not wanted, or a tensor to write into."""
    x = _dev(x, torch.float32, "x")
    B = x.shape[0] if x.dim() == 2 else 1
    dev = x.device
    lg = _dev(_opt(logits, (B, layer.d_ffn), torch.float32, dev), torch.float32, "logits")
    mk = _dev(_opt(mask, (B, layer.d_ffn), torch.uint8, dev), torch.uint8, "mask")
    un = _dev(_opt(union, (layer.d_ffn,), torch.uint8, dev), torch.uint8, "union")
    ws = layer.workspace(B) if ws is None else ws
    _check(load().spffn_predict(layer.handle, _ptr(x), B, _ptr(lg), _ptr(mk), _ptr(un), _ptr(ws),
                                ws.numel(), _stream()), "spffn_predict")
    out = {}
    for k, v in (("logits", lg), ("mask", mk), ("union", un)):
        if v is not None:
            out[k] = v
    return out


def forward(layer, x, mask=None, idx=None, count=None, y=None, ws=None):
    """y [B, d] of the FFN over the given neuron set (dense if none is given)."""
    x = _dev(x, torch.float32, "x")
    B = x.shape[0] if x.dim() == 2 else 1
    if y is None:
        y = torch.empty_like(x)
    _dev(y, torch.float32, "y")
    if mask is not None and mask.dtype not in (torch.uint8, torch.bool):
        raise TypeError("mask must be uint8 or bool")
    _dev(mask, None, "mask")
    _dev(idx, torch.int32, "idx")
    _dev(count, torch.int32, "count")
    ws = layer.workspace(B) if ws is None else ws
    _check(load().spffn_forward(layer.handle, _ptr(x), B, _ptr(mask), _ptr(idx), _ptr(count),
                                _ptr(y), _ptr(ws), ws.numel(), _stream()), "spffn_forward")
    return y


def decode_step(model, x, h=None, dense=False, layer_counts=None, trace=None, ws=None):
    """One pass of the whole stack: returns h [B, d].  `trace` is an optional
    dict with device tensors h_in [L, B, d] f32, union_mask [sum d_ffn] u8,
    logits [sum B*d_ffn] f32, and `events`, a ctypes array of 2L hipEvent_t
    handles recorded around each layer's largest kernel."""
    x = _dev(x, torch.float32, "x")
    B = x.shape[0] if x.dim() == 2 else 1
    if h is None:
        h = torch.empty_like(x)
    _dev(h, torch.float32, "h")
    _dev(layer_counts, torch.int32, "layer_counts")
    tr = None
    if trace is not None:
        ev = trace.get("events")
        tr = Trace(h_in=_ptr(trace.get("h_in")), union_mask=_ptr(trace.get("union_mask")),
                   logits=_ptr(trace.get("logits")),
                   events=None if ev is None else C.cast(ev, C.c_void_p))
    ws = model.workspace(B) if ws is None else ws
    _check(load().spffn_decode_step(model.handle, _ptr(x), _ptr(h), B,
                                    DECODE_DENSE if dense else 0, _ptr(layer_counts),
                                    C.byref(tr) if tr is not None else None, _ptr(ws), ws.numel(),
                                    _stream()), "spffn_decode_step")
    return h


class DecodeGraph:
    """One decode step captured into a HIP graph (a spffn_graph handle).

    The graph keeps the addresses of x, h, layer_counts and the workspace, so
    this object holds references to those tensors; write the next input into
    `x` and call launch() once per token."""

    def __init__(self, model, x, h=None, dense=False, layer_counts=None, ws=None):
        x = _dev(x, torch.float32, "x")
        B = x.shape[0] if x.dim() == 2 else 1
        if h is None:
            h = torch.empty_like(x)
        _dev(h, torch.float32, "h")
        _dev(layer_counts, torch.int32, "layer_counts")
        ws = model.workspace(B) if ws is None else ws
        self.model, self.x, self.h, self.layer_counts, self.ws = model, x, h, layer_counts, ws
        out = _vp()
        _check(load().spffn_decode_graph_create(model.handle, _ptr(x), _ptr(h), B,
                                                DECODE_DENSE if dense else 0, _ptr(layer_counts),
                                                _ptr(ws), ws.numel(), C.byref(out)),
               "spffn_decode_graph_create")
        self.handle = out.value

    def launch(self, stream=None):
        _check(load().spffn_graph_launch(self.handle, _stream(stream)), "spffn_graph_launch")
        return self.h

    def __del__(self):
        if getattr(self, "handle", None):
            _lib = load()
            _lib.spffn_graph_destroy(self.handle)
            self.handle = None


def profile(layer, x, counts=None):
    """counts int32 [d_ffn] += tokens of x [N, d] with a positive pre-activation."""
    x = _dev(x, torch.float32, "x")
    N = x.shape[0] if x.dim() == 2 else 1
    if counts is None:
        counts = torch.zeros(layer.d_ffn, dtype=torch.int32, device=x.device)
    _dev(counts, torch.int32, "counts")
    _check(load().spffn_profile(layer.handle, _ptr(x), N, _ptr(counts), None, 0, _stream()),
           "spffn_profile")
    return counts


def hot_first_order(counts, perm=None):
    counts = _dev(counts, torch.int32, "counts")
    if perm is None:
        perm = torch.empty_like(counts)
    _dev(perm, torch.int32, "perm")
    _check(load().spffn_hot_first_order(_ptr(counts), counts.numel(), _ptr(perm), _stream()),
           "spffn_hot_first_order")
    return perm


def permute_rows(src, perm, dst=None):
    """dst[k] = src[perm[k]] along dim 0 (any dtype, rows of a multiple of 4 bytes)."""
    src = _dev(src, None, "src")
    _dev(perm, torch.int32, "perm")
    if dst is None:
        dst = torch.empty_like(src)
    _dev(dst, src.dtype, "dst")
    rows = src.shape[0]
    row_bytes = src.numel() * src.element_size() // rows
    _check(load().spffn_permute_rows(_ptr(src), _ptr(dst), _ptr(perm), rows, row_bytes,
                                     _stream()), "spffn_permute_rows")
    return dst


def q4_0_repack(aos, rows, cols, soa=None):
    aos = _dev(aos, torch.uint8, "aos")
    if soa is None:
        soa = torch.empty(rows * (cols // 32) * 18, dtype=torch.uint8, device=aos.device)
    _dev(soa, torch.uint8, "soa")
    _check(load().spffn_q4_0_repack(_ptr(aos), _ptr(soa), rows, cols, _stream()),
           "spffn_q4_0_repack")
    return soa


# rows that move together under a neuron permutation
PERMUTED_KEYS = ("w_gate", "w_up", "w_down_t", "b_act", "p_w2", "p_b2")


def hot_first_permute(w, calib_x):
    """Load-time hot-first ordering of one layer dict (device tensors): profile
    the activated projection on calib_x [N, d], order neurons by descending
    count (ties by index), and permute every per-neuron row.  Returns
    (permuted dict, perm int32 [d_ffn], counts int32 [d_ffn]); stored neuron k
    of the result is neuron perm[k] of `w`."""
    layer = Layer(w)
    counts = profile(layer, calib_x)
    perm = hot_first_order(counts)
    out = dict(w)
    for k in PERMUTED_KEYS:
        if w.get(k) is not None and (k != "w_gate" or w["kind"] == "reglu"):
            src = w[k]
            if src.dim() == 1:
                out[k] = permute_rows(src.view(-1, 1), perm).view(-1)
            else:
                out[k] = permute_rows(src, perm)
    del layer
    return out, perm, counts
