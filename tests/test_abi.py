"""The C-ABI library loads and exports every symbol its header declares, and
its host-side argument checks return the documented status before anything
reaches the GPU (no kernels run here)."""
import ctypes as C
import os
import re

import pytest

import activation_sparse_mlp_amd as spffn
from activation_sparse_mlp_amd._lib import LayerDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spffn.h")

OK, E_ARG, E_SHAPE, E_DTYPE, E_WORKSPACE = 0, -1, -2, -3, -4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spffn_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    lib = spffn.load()
    names = declared_functions()
    assert len(names) >= 18
    for n in names:
        assert hasattr(lib, n), f"{n} declared in spffn.h but not exported"
    # the binding knows every declared function and nothing else
    assert sorted(spffn.SIGNATURES) == names


def test_version():
    assert "gfx950" in spffn.version()


FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced


def desc(**kw):
    base = dict(d=256, d_ffn=1024, r=64, kind=1, w_dtype=1, p_dtype=1, tau=0.5, dense_prefix=0,
                w_gate=FAKE, w_up=FAKE, w_down_t=FAKE, b_act=FAKE, p_w1=FAKE, p_b1=FAKE,
                p_w2=FAKE, p_b2=FAKE)
    base.update(kw)
    return LayerDesc(**base)


def create(**kw):
    lib = spffn.load()
    h = C.c_void_p()
    st = lib.spffn_layer_create(C.byref(desc(**kw)), C.byref(h))
    return st, h


@pytest.mark.parametrize("kw,status", [
    ({}, OK),
    ({"kind": 0, "w_gate": None}, OK),
    ({"d": 0}, E_SHAPE),
    ({"d_ffn": -1}, E_SHAPE),
    ({"r": 0}, E_SHAPE),
    ({"kind": 7}, E_ARG),
    ({"kind": 2}, OK),                      # SwiGLU
    ({"kind": 2, "w_gate": None}, E_ARG),   # gated: needs the gate
    ({"w_dtype": 9}, E_DTYPE),
    ({"p_dtype": 2}, E_DTYPE),
    ({"d": 260}, E_SHAPE),                  # fp16 rows need d % 8 == 0
    ({"w_dtype": 2, "d": 264}, E_SHAPE),    # 4-bit blocks need d % 32 == 0
    ({"w_dtype": 0, "p_dtype": 0, "d": 260, "r": 12}, OK),
    ({"r": 60}, E_SHAPE),                   # fp16 predictor needs r % 8 == 0
    ({"tau": 0.0}, E_ARG),
    ({"tau": 1.0}, E_ARG),
    ({"tau": float("nan")}, E_ARG),
    ({"dense_prefix": 1024}, OK),           # every neuron always active
    ({"dense_prefix": 1025}, E_SHAPE),
    ({"dense_prefix": -1}, E_SHAPE),
    ({"w_gate": None}, E_ARG),              # ReGLU needs the gate
    ({"w_up": None}, E_ARG),
    ({"p_b2": None}, E_ARG),
    ({"w_up": FAKE + 8}, E_ARG),            # weights must be 16-byte aligned
    ({"b_act": FAKE + 2}, E_ARG),
])
def test_layer_create_validation(kw, status):
    st, h = create(**kw)
    assert st == status, spffn.load().spffn_last_error()
    if st == OK:
        spffn.load().spffn_layer_destroy(h)
    else:
        assert spffn.load().spffn_last_error()


def test_threshold_value():
    lib = spffn.load()
    import math
    for tau in (0.5, 0.6, 0.45, 0.3, 0.999):
        st, h = create(tau=tau)
        assert st == OK
        t32 = C.c_float(tau).value  # the layer carries tau as binary32
        got = lib.spffn_layer_threshold(h)
        assert got == C.c_float(math.log(t32 / (1.0 - t32))).value
        lib.spffn_layer_destroy(h)
    assert lib.spffn_layer_threshold(None) != lib.spffn_layer_threshold(None)  # NaN


def test_workspace_and_entry_point_validation():
    lib = spffn.load()
    st, h = create()
    assert st == OK
    n1 = lib.spffn_layer_workspace_bytes(h, 1)
    n16 = lib.spffn_layer_workspace_bytes(h, 16)
    assert 0 < n1 < n16
    assert lib.spffn_layer_workspace_bytes(h, 0) == 0
    assert lib.spffn_layer_workspace_bytes(h, 17) == 0
    x = C.c_void_p(FAKE)
    ws = C.c_void_p(0x100000)
    # batch out of range
    assert lib.spffn_forward(h, x, 0, None, None, None, x, ws, n1, None) == E_SHAPE
    assert lib.spffn_forward(h, x, 17, None, None, None, x, ws, n16, None) == E_SHAPE
    # workspace missing, too small, misaligned
    assert lib.spffn_forward(h, x, 1, None, None, None, x, None, 0, None) == E_WORKSPACE
    assert lib.spffn_forward(h, x, 1, None, None, None, x, ws, n1 - 1, None) == E_WORKSPACE
    assert lib.spffn_forward(h, x, 1, None, None, None, x, C.c_void_p(0x100010), n1,
                             None) == E_ARG
    # idx without count
    assert lib.spffn_forward(h, x, 1, None, x, None, x, ws, n1, None) == E_ARG
    # predict with no outputs, NULL x
    assert lib.spffn_predict(h, x, 1, None, None, None, ws, n1, None) == E_ARG
    assert lib.spffn_predict(h, None, 1, x, None, None, ws, n1, None) == E_ARG
    # compact / threshold
    assert lib.spffn_compact(None, 10, x, x, None) == E_ARG
    assert lib.spffn_compact(x, 0, x, x, None) == E_SHAPE
    assert lib.spffn_threshold(x, -1, 0.0, x, None) == E_SHAPE
    assert lib.spffn_threshold(x, 0, 0.0, x, None) == OK  # nothing to do
    # load-time utilities
    assert lib.spffn_permute_rows(x, C.c_void_p(FAKE + 64), x, 4, 64, None) == E_ARG  # overlap
    assert lib.spffn_permute_rows(x, C.c_void_p(FAKE * 16), x, 4, 6, None) == E_SHAPE
    assert lib.spffn_q4_0_repack(x, x, 4, 48, None) == E_SHAPE
    assert lib.spffn_q4_0_repack(x, C.c_void_p(FAKE + 8), 4, 64, None) == E_ARG
    assert lib.spffn_hot_first_order(x, 0, x, None) == E_SHAPE
    assert lib.spffn_profile(h, x, 0, x, None, 0, None) == E_SHAPE
    lib.spffn_layer_destroy(h)


def test_model_validation():
    lib = spffn.load()
    st, a = create()
    st2, b = create(d=512)
    assert st == st2 == OK
    m = C.c_void_p()
    arr = (C.c_void_p * 2)(a.value, b.value)
    assert lib.spffn_model_create(arr, 2, 1e-5, C.byref(m)) == E_SHAPE  # mixed d
    assert lib.spffn_model_create(arr, 0, 1e-5, C.byref(m)) == E_ARG
    one = (C.c_void_p * 1)(a.value)
    assert lib.spffn_model_create(one, 1, -1.0, C.byref(m)) == E_ARG
    assert lib.spffn_model_create(one, 1, 1e-5, C.byref(m)) == OK
    nb = lib.spffn_model_workspace_bytes(m, 1)
    assert nb == lib.spffn_layer_workspace_bytes(a, 1)
    x = C.c_void_p(FAKE)
    ws = C.c_void_p(0x100000)
    assert lib.spffn_decode_step(m, x, x, 1, 4, None, None, ws, nb, None) == E_ARG  # bad flag
    assert lib.spffn_decode_step(m, x, x, 1, 0, None, None, ws, nb - 256, None) == E_WORKSPACE
    # graph capture validates like decode_step before touching the runtime
    g = C.c_void_p()
    assert lib.spffn_decode_graph_create(m, x, x, 1, 0, None, ws, nb, None) == E_ARG
    assert lib.spffn_decode_graph_create(m, x, x, 1, 4, None, ws, nb, C.byref(g)) == E_ARG
    assert lib.spffn_decode_graph_create(m, x, x, 0, 0, None, ws, nb, C.byref(g)) == E_SHAPE
    assert lib.spffn_decode_graph_create(m, x, x, 1, 0, None, ws, nb - 256,
                                         C.byref(g)) == E_WORKSPACE
    assert lib.spffn_decode_graph_create(None, x, x, 1, 0, None, ws, nb, C.byref(g)) == E_ARG
    assert g.value is None
    assert lib.spffn_graph_launch(None, None) == E_ARG
    lib.spffn_graph_destroy(None)  # no-op
    lib.spffn_model_destroy(m)
    lib.spffn_layer_destroy(a)
    lib.spffn_layer_destroy(b)


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(TypeError):
        spffn.threshold(torch.zeros(4), 0.0)


def test_set_wait_limit_range():
    # host-side check only (no kernel runs): the bounded-wait test hook takes
    # 0 .. 2^24 polls and rejects anything else before it takes effect
    lib = spffn.load()
    assert lib.spffn_set_wait_limit(-1) == E_ARG
    assert lib.spffn_set_wait_limit((1 << 24) + 1) == E_ARG
    assert lib.spffn_set_wait_limit(0) == OK
    assert lib.spffn_set_wait_limit(1 << 24) == OK
    assert lib.spffn_set_wait_limit(spffn.WAIT_LIMIT_DEFAULT) == OK


def test_workspace_status_validation():
    # host-side checks of the status calls (nothing is enqueued on failure)
    lib = spffn.load()
    ws = C.c_void_p(0x100000)
    out = C.c_void_p(FAKE)
    assert lib.spffn_workspace_clear_status(None, 4096, None) == E_ARG
    assert lib.spffn_workspace_clear_status(C.c_void_p(0x100010), 4096, None) == E_ARG
    assert lib.spffn_workspace_clear_status(ws, 255, None) == E_WORKSPACE
    assert lib.spffn_workspace_status(ws, 4096, None, None) == E_ARG
    assert lib.spffn_workspace_status(None, 4096, out, None) == E_ARG
    assert lib.spffn_workspace_status(ws, 4096, C.c_void_p(FAKE + 2), None) == E_ARG
    assert lib.spffn_workspace_status(ws, 100, out, None) == E_WORKSPACE


def test_stream_read_validation():
    lib = spffn.load()
    x = C.c_void_p(FAKE)
    assert lib.spffn_stream_read(None, 1024, x, None) == E_ARG
    assert lib.spffn_stream_read(x, 1024, None, None) == E_ARG
    assert lib.spffn_stream_read(x, 0, x, None) == E_SHAPE
    assert lib.spffn_stream_read(x, 1000, x, None) == E_SHAPE
    assert lib.spffn_stream_read(C.c_void_p(FAKE + 4), 1024, x, None) == E_ARG


def test_decode_noalloc_rejects_models_beyond_its_array():
    # host-side check, before any HIP call: a model whose workspace exceeds
    # the library's static scratch array is refused with a clear message
    lib = spffn.load()
    st, h = create(d=8192, d_ffn=1 << 22, r=1024)
    assert st == OK
    m = C.c_void_p()
    arr = (C.c_void_p * 1)(h.value)
    assert lib.spffn_model_create(arr, 1, 1e-5, C.byref(m)) == OK
    assert lib.spffn_model_workspace_bytes(m, 1) > spffn._lib.NOALLOC_SCRATCH_BYTES
    x = C.c_void_p(FAKE)
    assert lib.spffn_decode_step_noalloc(m, x, x, 1, 0, None, None) == E_WORKSPACE
    assert b"static" in lib.spffn_last_error()
    # argument checks come first, as in spffn_decode_step
    assert lib.spffn_decode_step_noalloc(m, x, x, 0, 0, None, None) == E_SHAPE
    assert lib.spffn_decode_step_noalloc(m, x, x, 1, 4, None, None) == E_ARG
    assert lib.spffn_decode_step_noalloc(None, x, x, 1, 0, None, None) == E_ARG
    lib.spffn_model_destroy(m)
    lib.spffn_layer_destroy(h)


def test_tau_threshold_and_adaptive_validation():
    import math
    lib = spffn.load()
    for tau in (0.5, 0.3, 0.75, 1e-6):
        t32 = C.c_float(tau).value
        assert lib.spffn_tau_threshold(tau) == C.c_float(math.log(t32 / (1.0 - t32))).value
    for bad in (0.0, 1.0, -0.5, float("nan")):
        assert math.isnan(lib.spffn_tau_threshold(bad))
    st, h = create()
    assert st == OK
    # a layer created with tau compares against spffn_tau_threshold(tau)
    assert lib.spffn_layer_threshold(h) == lib.spffn_tau_threshold(0.5)
    m = C.c_void_p()
    arr = (C.c_void_p * 1)(h.value)
    assert lib.spffn_model_create(arr, 1, 1e-5, C.byref(m)) == OK
    nb = lib.spffn_model_workspace_bytes(m, 2)
    x = C.c_void_p(FAKE)
    ws = C.c_void_p(0x100000)
    assert lib.spffn_decode_step_adaptive(m, x, x, 2, None, None, None, ws, nb, None) == E_ARG
    assert lib.spffn_decode_step_adaptive(m, x, x, 2, C.c_void_p(FAKE + 2), None, None, ws, nb,
                                          None) == E_ARG
    assert lib.spffn_decode_step_adaptive(m, x, x, 17, x, None, None, ws, nb, None) == E_SHAPE
    assert lib.spffn_decode_step_adaptive(m, x, x, 2, x, None, None, ws, nb - 256,
                                          None) == E_WORKSPACE
    lib.spffn_model_destroy(m)
    lib.spffn_layer_destroy(h)
