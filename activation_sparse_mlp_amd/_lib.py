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

F32, F16, Q4_0, FP8_E4M3 = 0, 1, 2, 3
RELU, REGLU, SWIGLU = 0, 1, 2
MAX_BATCH = 16
DECODE_DENSE = 1
_DTYPES = {"f32": F32, "f16": F16, "q4_0": Q4_0, "fp8": FP8_E4M3}
_KINDS = {"relu": RELU, "reglu": REGLU, "swiglu": SWIGLU}
_STATUS = {0: "OK", -1: "E_ARG", -2: "E_SHAPE", -3: "E_DTYPE", -4: "E_WORKSPACE", -5: "E_HIP"}


class SpffnError(RuntimeError):
    def __init__(self, status, where, text):
        super().__init__(f"{where}: {_STATUS.get(status, status)}: {text}")
        self.status = status


class LayerDesc(C.Structure):
    _fields_ = [("d", C.c_int32), ("d_ffn", C.c_int32), ("r", C.c_int32),
                ("kind", C.c_int32), ("w_dtype", C.c_int32), ("p_dtype", C.c_int32),
                ("tau", C.c_float), ("dense_prefix", C.c_int32),
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
    "spffn_workspace_clear_status": (_i32, [_vp, _sz, _vp]),
    "spffn_workspace_status": (_i32, [_vp, _sz, _vp, _vp]),
    "spffn_threshold": (_i32, [_vp, _i64, _f32, _vp, _vp]),
    "spffn_compact": (_i32, [_vp, _i32, _vp, _vp, _vp]),
    "spffn_predict": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spffn_forward": (_i32, [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "spffn_decode_step": (_i32, [_vp, _vp, _vp, _i32, _i32, _vp, C.POINTER(Trace), _vp, _sz,
                                 _vp]),
    "spffn_decode_graph_create": (_i32, [_vp, _vp, _vp, _i32, _i32, _vp, _vp, _sz,
                                         C.POINTER(_vp)]),
    "spffn_decode_step_noalloc": (_i32, [_vp, _vp, _vp, _i32, _i32, _vp, _vp]),
    "spffn_tau_threshold": (_f32, [_f32]),
    "spffn_decode_step_adaptive": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, C.POINTER(Trace), _vp,
                                          _sz, _vp]),
    "spffn_graph_launch": (_i32, [_vp, _vp]),
    "spffn_graph_destroy": (None, [_vp]),
    "spffn_profile": (_i32, [_vp, _vp, _i32, _vp, _vp, _sz, _vp]),
    "spffn_profile_workspace_bytes": (_sz, [_vp]),
    "spffn_hot_first_order": (_i32, [_vp, _i32, _vp, _vp]),
    "spffn_permute_rows": (_i32, [_vp, _vp, _vp, _i32, _i64, _vp]),
    "spffn_q4_0_repack": (_i32, [_vp, _vp, _i32, _i32, _vp]),
    "spffn_stream_read": (_i32, [_vp, _i64, _vp, _vp]),
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


def _dev(t, dtype, name, n=None, at_least=False):
    """Check a tensor argument: its size first (n elements, or at least n), so
    that a wrongly sized buffer is rejected whatever its device, then that it
    is a contiguous HIP tensor of the given dtype."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if n is not None:
        _size(t, n, name, at_least)
    if not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _size(t, n, name, at_least=False):
    """Raise ValueError unless tensor t holds exactly n elements (at least n
    with at_least).  The C entry points receive bare pointers, so every length
    is checked here, before anything is enqueued."""
    if t is None:
        return
    k = t.numel()
    if (k < n) if at_least else (k != n):
        want = f">= {n}" if at_least else f"{n}"
        raise ValueError(f"{name} holds {k} elements, needs {want}")


def _tokens(x, d, name="x"):
    """Number of tokens B of an activation tensor x of shape [d] or [B, d]."""
    if x.dim() not in (1, 2) or x.shape[-1] != d:
        raise ValueError(f"{name} must have shape [d] or [B, d] with d={d}, got "
                         f"{tuple(x.shape)}")
    return x.shape[0] if x.dim() == 2 else 1


def _ws_bytes(ws, need, name="ws"):
    """Byte size of a caller workspace tensor (any dtype), checked against need."""
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise TypeError(f"{name} must be a contiguous CUDA (HIP) tensor")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"{name} has {nbytes} bytes, needs {need}")
    return nbytes


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
        self.dense_prefix = int(w.get("dense_prefix", 0) or 0)
        wd = {"f32": torch.float32, "f16": torch.float16, "q4_0": torch.uint8}[self.w_dtype]
        pd = {"f32": torch.float32, "f16": torch.float16, "fp8": torch.uint8}[self.p_dtype]
        if min(self.d, self.d_ffn, self.r) <= 0:
            raise ValueError(f"d={self.d}, d_ffn={self.d_ffn}, r={self.r} must be positive")
        if self.w_dtype == "q4_0" and self.d % 32:
            raise ValueError(f"4-bit rows need d % 32 == 0, got d={self.d}")
        n_w = self.d_ffn * (self.d // 32 * 18 if self.w_dtype == "q4_0" else self.d)
        # fp8 predictor matrices: the codes, then one fp32 scale per row
        ps = 4 if self.p_dtype == "fp8" else 0
        sizes = {"w_gate": n_w, "w_up": n_w, "w_down_t": n_w, "b_act": self.d_ffn,
                 "p_w1": self.r * (self.d + ps), "p_b1": self.r,
                 "p_w2": self.d_ffn * (self.r + ps), "p_b2": self.d_ffn}
        for k, n in sizes.items():  # every size before any device check
            if isinstance(w.get(k), torch.Tensor) and (k != "w_gate" or self.kind != "relu"):
                _size(w[k], n, k)
        t = {}
        for k in ("w_gate", "w_up", "w_down_t"):
            if w.get(k) is not None and (k != "w_gate" or self.kind != "relu"):
                t[k] = _dev(w[k], wd, k, n_w)
                if self.w_dtype == "q4_0":
                    t[k] = q4_0_repack(t[k], self.d_ffn, self.d)
        if "w_up" not in t or "w_down_t" not in t or (self.kind != "relu" and "w_gate" not in t):
            raise ValueError("missing FFN weight (w_up, w_down_t, and w_gate when gated)")
        t["b_act"] = _dev(w.get("b_act"), torch.float32, "b_act", self.d_ffn)
        for k in ("p_w1", "p_w2"):
            t[k] = _dev(w[k], pd, k, sizes[k])
        for k, n in (("p_b1", self.r), ("p_b2", self.d_ffn)):
            t[k] = _dev(w[k], torch.float32, k, n)
        self.tensors = t
        desc = LayerDesc(d=self.d, d_ffn=self.d_ffn, r=self.r, kind=_KINDS[self.kind],
                         w_dtype=_DTYPES[self.w_dtype], p_dtype=_DTYPES[self.p_dtype],
                         tau=self.tau, dense_prefix=self.dense_prefix,
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
        """A workspace for B tokens, its status word cleared."""
        n = self.workspace_bytes(B)
        if n == 0:
            raise SpffnError(-2, "workspace_bytes", f"bad batch {B}")
        ws = torch.empty(n, dtype=torch.uint8, device=device or self.tensors["w_up"].device)
        workspace_clear_status(ws)
        return ws

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
        self.n_layers = len(self.layers)
        self.sum_d_ffn = sum(l.d_ffn for l in self.layers)

    def workspace_bytes(self, B):
        return int(load().spffn_model_workspace_bytes(self.handle, B))

    def workspace(self, B):
        """A workspace for B tokens, its status word cleared."""
        n = self.workspace_bytes(B)
        if n == 0:
            raise SpffnError(-2, "model_workspace_bytes", f"bad batch {B}")
        ws = torch.empty(n, dtype=torch.uint8, device=self.layers[0].tensors["w_up"].device)
        workspace_clear_status(ws)
        return ws

    def __del__(self):
        if getattr(self, "handle", None) is not None and _lib is not None:
            _lib.spffn_model_destroy(self.handle)
            self.handle = None


# --------------------------------------------------------------------------- #
# entry points (same names as the C ABI, without the prefix)
# --------------------------------------------------------------------------- #
def workspace_clear_status(ws):
    """Zero the status block at the start of a workspace (on the current stream)."""
    nb = _ws_bytes(ws, 256)
    _check(load().spffn_workspace_clear_status(_ptr(ws), nb, _stream()),
           "spffn_workspace_clear_status")


def workspace_status(ws, out=None):
    """Device int32 [1]: the number of bounded in-launch waits that gave up
    since the workspace's status was last cleared (0 on a healthy run)."""
    nb = _ws_bytes(ws, 256)
    if out is None:
        out = torch.empty(1, dtype=torch.int32, device=ws.device)
    _dev(out, torch.int32, "out", 1, at_least=True)
    _check(load().spffn_workspace_status(_ptr(ws), nb, _ptr(out), _stream()),
           "spffn_workspace_status")
    return out


def threshold(logits, t, mask=None):
    if mask is not None:
        _size(mask, logits.numel(), "mask")
    logits = _dev(logits, torch.float32, "logits")
    if mask is None:
        mask = torch.empty(logits.shape, dtype=torch.uint8, device=logits.device)
    _dev(mask, torch.uint8, "mask", logits.numel())
    _check(load().spffn_threshold(_ptr(logits), logits.numel(), float(t), _ptr(mask), _stream()),
           "spffn_threshold")
    return mask


def compact(mask, idx=None, count=None):
    """(idx int32 [n], count int32 [1]) on the device; idx[:count] is valid."""
    n = mask.numel()
    _size(idx, n, "idx", at_least=True)
    _size(count, 1, "count", at_least=True)
    mask = _dev(mask, None, "mask")
    if mask.dtype not in (torch.uint8, torch.bool):
        raise TypeError("mask must be uint8 or bool")
    if idx is None:
        idx = torch.empty(n, dtype=torch.int32, device=mask.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=mask.device)
    _dev(idx, torch.int32, "idx", n, at_least=True)
    _dev(count, torch.int32, "count", 1, at_least=True)
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
    B = _tokens(x, layer.d)
    for v, n, name in ((logits, B * layer.d_ffn, "logits"), (mask, B * layer.d_ffn, "mask"),
                       (union, layer.d_ffn, "union")):
        if isinstance(v, torch.Tensor):
            _size(v, n, name)
    x = _dev(x, torch.float32, "x")
    dev = x.device
    lg = _dev(_opt(logits, (B, layer.d_ffn), torch.float32, dev), torch.float32, "logits",
              B * layer.d_ffn)
    mk = _dev(_opt(mask, (B, layer.d_ffn), torch.uint8, dev), torch.uint8, "mask",
              B * layer.d_ffn)
    un = _dev(_opt(union, (layer.d_ffn,), torch.uint8, dev), torch.uint8, "union", layer.d_ffn)
    ws = layer.workspace(B) if ws is None else ws
    nb = _ws_bytes(ws, layer.workspace_bytes(B))
    _check(load().spffn_predict(layer.handle, _ptr(x), B, _ptr(lg), _ptr(mk), _ptr(un), _ptr(ws),
                                nb, _stream()), "spffn_predict")
    out = {}
    for k, v in (("logits", lg), ("mask", mk), ("union", un)):
        if v is not None:
            out[k] = v
    return out


def forward(layer, x, mask=None, idx=None, count=None, y=None, ws=None):
    """y [B, d] of the FFN over the given neuron set (dense if none is given).

    idx must have room for d_ffn entries: the count lives on the device, so a
    shorter list could not be checked against it without a synchronisation."""
    B = _tokens(x, layer.d)
    if mask is None and (idx is None) != (count is None):
        raise ValueError("idx and count must be given together")
    _size(y, B * layer.d, "y")
    _size(mask, layer.d_ffn, "mask")
    _size(idx, layer.d_ffn, "idx", at_least=True)
    _size(count, 1, "count", at_least=True)
    x = _dev(x, torch.float32, "x")
    if y is None:
        y = torch.empty_like(x)
    _dev(y, torch.float32, "y", B * layer.d)
    if mask is not None and mask.dtype not in (torch.uint8, torch.bool):
        raise TypeError("mask must be uint8 or bool")
    _dev(mask, None, "mask", layer.d_ffn)
    _dev(idx, torch.int32, "idx", layer.d_ffn, at_least=True)
    _dev(count, torch.int32, "count", 1, at_least=True)
    ws = layer.workspace(B) if ws is None else ws
    nb = _ws_bytes(ws, layer.workspace_bytes(B))
    _check(load().spffn_forward(layer.handle, _ptr(x), B, _ptr(mask), _ptr(idx), _ptr(count),
                                _ptr(y), _ptr(ws), nb, _stream()), "spffn_forward")
    return y


def tau_threshold(tau):
    """The binary32 logit threshold ln(tau / (1 - tau)) a layer of this tau uses."""
    return float(load().spffn_tau_threshold(float(tau)))


def decode_step_adaptive(model, x, thresholds, h=None, layer_counts=None, trace=None, ws=None):
    """decode_step with a logit threshold per layer and token: thresholds is a
    device fp32 tensor [L, B] (tau_threshold of each per-token tau)."""
    B = _tokens(x, model.d)
    _size(thresholds, model.n_layers * B, "thresholds")
    thresholds = _dev(thresholds, torch.float32, "thresholds", model.n_layers * B)
    return decode_step(model, x, h=h, layer_counts=layer_counts, trace=trace, ws=ws,
                       _thresholds=thresholds)


def decode_step(model, x, h=None, dense=False, layer_counts=None, trace=None, ws=None,
                _thresholds=None):
    """One pass of the whole stack: returns h [B, d].  `trace` is an optional
    dict with device tensors h_in [L, B, d] f32, union_mask [sum d_ffn] u8,
    logits [sum B*d_ffn] f32, and `events`, a ctypes array of 2L hipEvent_t
    handles recorded around each layer's largest kernel."""
    B = _tokens(x, model.d)
    _size(h, B * model.d, "h")
    _size(layer_counts, model.n_layers, "layer_counts", at_least=True)
    tr = None
    if trace is not None:
        ev = trace.get("events")
        sizes = {"h_in": model.n_layers * B * model.d, "union_mask": model.sum_d_ffn,
                 "logits": B * model.sum_d_ffn}
        for k, n in sizes.items():
            _size(trace.get(k), n, f"trace {k}", at_least=True)
        if ev is not None and len(ev) < 2 * model.n_layers:
            raise ValueError(f"trace events holds {len(ev)} handles, needs "
                             f">= {2 * model.n_layers}")
    x = _dev(x, torch.float32, "x")
    if h is None:
        h = torch.empty_like(x)
    _dev(h, torch.float32, "h", B * model.d)
    _dev(layer_counts, torch.int32, "layer_counts", model.n_layers, at_least=True)
    if trace is not None:
        h_in = _dev(trace.get("h_in"), torch.float32, "trace h_in")
        um = _dev(trace.get("union_mask"), torch.uint8, "trace union_mask")
        lg = _dev(trace.get("logits"), torch.float32, "trace logits")
        tr = Trace(h_in=_ptr(h_in), union_mask=_ptr(um), logits=_ptr(lg),
                   events=None if ev is None else C.cast(ev, C.c_void_p))
    ws = model.workspace(B) if ws is None else ws
    nb = _ws_bytes(ws, model.workspace_bytes(B))
    trp = C.byref(tr) if tr is not None else None
    if _thresholds is not None:
        _check(load().spffn_decode_step_adaptive(model.handle, _ptr(x), _ptr(h), B,
                                                 _ptr(_thresholds), _ptr(layer_counts), trp,
                                                 _ptr(ws), nb, _stream()),
               "spffn_decode_step_adaptive")
        return h
    _check(load().spffn_decode_step(model.handle, _ptr(x), _ptr(h), B,
                                    DECODE_DENSE if dense else 0, _ptr(layer_counts), trp,
                                    _ptr(ws), nb, _stream()), "spffn_decode_step")
    return h


NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_step_noalloc(model, x, h=None, dense=False, layer_counts=None):
    """decode_step with the library's static scratch array as its workspace
    (no allocation in the library; h is allocated here only when not given)."""
    B = _tokens(x, model.d)
    _size(h, B * model.d, "h")
    _size(layer_counts, model.n_layers, "layer_counts", at_least=True)
    x = _dev(x, torch.float32, "x")
    if h is None:
        h = torch.empty_like(x)
    _dev(h, torch.float32, "h", B * model.d)
    _dev(layer_counts, torch.int32, "layer_counts", model.n_layers, at_least=True)
    _check(load().spffn_decode_step_noalloc(model.handle, _ptr(x), _ptr(h), B,
                                            DECODE_DENSE if dense else 0, _ptr(layer_counts),
                                            _stream()), "spffn_decode_step_noalloc")
    return h


class DecodeGraph:
    """One decode step captured into a HIP graph (a spffn_graph handle).

    The graph keeps the addresses of x, h, layer_counts and the workspace, so
    this object holds references to those tensors; write the next input into
    `x` and call launch() once per token."""

    def __init__(self, model, x, h=None, dense=False, layer_counts=None, ws=None):
        B = _tokens(x, model.d)
        _size(h, B * model.d, "h")
        _size(layer_counts, model.n_layers, "layer_counts", at_least=True)
        x = _dev(x, torch.float32, "x")
        if h is None:
            h = torch.empty_like(x)
        _dev(h, torch.float32, "h", B * model.d)
        _dev(layer_counts, torch.int32, "layer_counts", model.n_layers, at_least=True)
        ws = model.workspace(B) if ws is None else ws
        nb = _ws_bytes(ws, model.workspace_bytes(B))
        self.model, self.x, self.h, self.layer_counts, self.ws = model, x, h, layer_counts, ws
        out = _vp()
        _check(load().spffn_decode_graph_create(model.handle, _ptr(x), _ptr(h), B,
                                                DECODE_DENSE if dense else 0, _ptr(layer_counts),
                                                _ptr(ws), nb, C.byref(out)),
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


def profile(layer, x, counts=None, scratch=True):
    """counts int32 [d_ffn] += tokens of x [N, d] with a positive pre-activation.
    With scratch (the default) the library gets the workspace that lets fp16
    rows run on the matrix cores; scratch=False keeps the vector kernels."""
    N = _tokens(x, layer.d)
    _size(counts, layer.d_ffn, "counts")
    x = _dev(x, torch.float32, "x")
    if counts is None:
        counts = torch.zeros(layer.d_ffn, dtype=torch.int32, device=x.device)
    _dev(counts, torch.int32, "counts", layer.d_ffn)
    nb = int(load().spffn_profile_workspace_bytes(layer.handle)) if scratch else 0
    ws = torch.empty(nb, dtype=torch.uint8, device=x.device) if nb else None
    _check(load().spffn_profile(layer.handle, _ptr(x), N, _ptr(counts),
                                _ptr(ws) if ws is not None else None, nb, _stream()),
           "spffn_profile")
    return counts


def hot_first_order(counts, perm=None):
    _size(perm, counts.numel(), "perm")
    counts = _dev(counts, torch.int32, "counts")
    if perm is None:
        perm = torch.empty_like(counts)
    _dev(perm, torch.int32, "perm", counts.numel())
    _check(load().spffn_hot_first_order(_ptr(counts), counts.numel(), _ptr(perm), _stream()),
           "spffn_hot_first_order")
    return perm


def permute_rows(src, perm, dst=None):
    """dst[k] = src[perm[k]] along dim 0 (any dtype, rows of a multiple of 4 bytes)."""
    if src.dim() < 1 or src.shape[0] < 1:
        raise ValueError("src must have at least one row")
    rows = src.shape[0]
    _size(perm, rows, "perm")
    _size(dst, src.numel(), "dst")
    src = _dev(src, None, "src")
    _dev(perm, torch.int32, "perm", rows)
    if dst is None:
        dst = torch.empty_like(src)
    _dev(dst, src.dtype, "dst", src.numel())
    row_bytes = src.numel() * src.element_size() // rows
    _check(load().spffn_permute_rows(_ptr(src), _ptr(dst), _ptr(perm), rows, row_bytes,
                                     _stream()), "spffn_permute_rows")
    return dst


def q4_0_repack(aos, rows, cols, soa=None):
    if rows < 1 or cols < 32 or cols % 32:
        raise ValueError(f"rows={rows}, cols={cols}: need rows >= 1 and cols a multiple of 32")
    n = rows * (cols // 32) * 18
    _size(soa, n, "soa")
    aos = _dev(aos, torch.uint8, "aos", n)
    if soa is None:
        soa = torch.empty(n, dtype=torch.uint8, device=aos.device)
    _dev(soa, torch.uint8, "soa", n)
    _check(load().spffn_q4_0_repack(_ptr(aos), _ptr(soa), rows, cols, _stream()),
           "spffn_q4_0_repack")
    return soa


STREAM_SINK_WORDS = 4096


def stream_read(buf, sink=None):
    """Read every byte of a device tensor once (bandwidth probe); returns the
    device int32 [4096] sink the data is folded into (the XOR of its words is
    the XOR of all 32-bit words of buf)."""
    buf = _dev(buf, None, "buf")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.zeros(STREAM_SINK_WORDS, dtype=torch.int32, device=buf.device)
    _dev(sink, torch.int32, "sink", STREAM_SINK_WORDS, at_least=True)
    _check(load().spffn_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream()),
           "spffn_stream_read")
    return sink


# rows that move together under a neuron permutation
PERMUTED_KEYS = ("w_gate", "w_up", "w_down_t", "b_act", "p_w2", "p_b2")


def hot_first_permute(w, calib_x, dense_prefix=False):
    """Load-time hot-first ordering of one layer dict (device tensors): profile
    the activated projection on calib_x [N, d], order neurons by descending
    count (ties by index), and permute every per-neuron row.  Returns
    (permuted dict, perm int32 [d_ffn], counts int32 [d_ffn]); stored neuron k
    of the result is neuron perm[k] of `w`.

    dense_prefix: also mark the neurons that fired on every calibration token
    (the leading ones after the order) as the layer's always-active prefix."""
    layer = Layer(dict(w, dense_prefix=0))
    counts = profile(layer, calib_x)
    perm = hot_first_order(counts)
    out = dict(w)
    if dense_prefix:
        N = calib_x.shape[0] if calib_x.dim() == 2 else 1
        out["dense_prefix"] = int((counts == N).sum())  # one synchronisation, at load
    F = int(w["d_ffn"])
    for k in PERMUTED_KEYS:
        if w.get(k) is not None and (k != "w_gate" or w["kind"] != "relu"):
            src = w[k]
            if k == "p_w2" and w["p_dtype"] == "fp8":
                # the codes [d_ffn, r] and the per-row scales move together
                r = int(w["r"])
                codes = permute_rows(src[:F * r].view(F, r), perm)
                scales = permute_rows(src[F * r:].view(F, 4), perm)
                out[k] = torch.cat([codes.view(-1), scales.view(-1)])
            elif src.dim() == 1:
                out[k] = permute_rows(src.view(-1, 1), perm).view(-1)
            else:
                out[k] = permute_rows(src, perm)
    del layer
    return out, perm, counts
