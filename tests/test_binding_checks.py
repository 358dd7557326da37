"""The Python binding rejects wrongly sized tensors before anything reaches the
C entry points (which receive bare pointers and could not notice).  The size
check comes before the device check, so these run on host tensors: a wrong
size raises ValueError, a right size on the host then fails the device check
(TypeError) -- either way nothing is enqueued."""
import types

import pytest
import torch

import activation_sparse_mlp_amd as spffn

D, F, R, L = 256, 1024, 64, 3


def _model():
    # only the attributes the wrappers read before they touch the library
    return types.SimpleNamespace(d=D, n_layers=L, sum_d_ffn=L * F, handle=None,
                                 workspace_bytes=lambda B: 1 << 20)


def _layer():
    return types.SimpleNamespace(d=D, d_ffn=F, r=R, handle=None,
                                 workspace_bytes=lambda B: 1 << 20)


def _f(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def _i(*shape):
    return torch.zeros(*shape, dtype=torch.int32)


def _u(*shape):
    return torch.zeros(*shape, dtype=torch.uint8)


@pytest.mark.parametrize("kw", [
    dict(x=_f(2, D + 8)),                                      # x wider than d
    dict(x=_f(2, 2, D)),                                       # x of rank 3
    dict(x=_f(2, D), h=_f(1, D)),                              # h for fewer tokens
    dict(x=_f(2, D), layer_counts=_i(L - 1)),                  # counts shorter than L
    dict(x=_f(1, D), trace={"h_in": _f(L - 1, 1, D)}),         # trace h_in short a layer
    dict(x=_f(1, D), trace={"union_mask": _u(L * F - 1)}),
    dict(x=_f(2, D), trace={"logits": _f(L * F)}),             # logits for one token of two
    dict(x=_f(1, D), trace={"events": (spffn._lib.C.c_void_p * (2 * L - 1))()}),
])
def test_decode_step_rejects_sizes(kw):
    x = kw.pop("x")
    with pytest.raises(ValueError):
        spffn.decode_step(_model(), x, **kw)


def test_decode_step_right_sizes_reach_device_check():
    with pytest.raises(TypeError, match="CUDA"):
        spffn.decode_step(_model(), _f(2, D), h=_f(2, D), layer_counts=_i(L),
                          trace={"h_in": _f(L, 2, D), "union_mask": _u(L * F),
                                 "logits": _f(2 * L * F)})


@pytest.mark.parametrize("kw", [
    dict(x=_f(1, D - 4)),
    dict(x=_f(1, D), h=_f(2, D)),
    dict(x=_f(1, D), layer_counts=_i(1)),
])
def test_decode_graph_rejects_sizes(kw):
    x = kw.pop("x")
    with pytest.raises(ValueError):
        spffn.DecodeGraph(_model(), x, **kw)


@pytest.mark.parametrize("kw", [
    dict(x=_f(3, D + 1)),
    dict(x=_f(3, D), y=_f(2, D)),
    dict(x=_f(1, D), mask=_u(F - 1)),
    dict(x=_f(1, D), idx=_i(F - 1), count=_i(1)),             # list shorter than d_ffn
    dict(x=_f(1, D), idx=_i(F), count=_i(0)),
])
def test_forward_rejects_sizes(kw):
    x = kw.pop("x")
    with pytest.raises(ValueError):
        spffn.forward(_layer(), x, **kw)


def test_forward_idx_without_count():
    with pytest.raises(ValueError, match="together"):
        spffn.forward(_layer(), _f(1, D), idx=_i(F))


@pytest.mark.parametrize("kw", [
    dict(x=_f(2, D), logits=_f(1, F)),
    dict(x=_f(2, D), mask=_u(2, F + 1)),
    dict(x=_f(2, D), union=_u(2 * F)),
    dict(x=_f(D * 2)),                                         # flat, not [B, d]
])
def test_predict_rejects_sizes(kw):
    x = kw.pop("x")
    with pytest.raises(ValueError):
        spffn.predict(_layer(), x, **kw)


def test_profile_and_order_reject_sizes():
    with pytest.raises(ValueError):
        spffn.profile(_layer(), _f(4, D), counts=_i(F - 1))
    with pytest.raises(ValueError):
        spffn.profile(_layer(), _f(4, D + 8))
    with pytest.raises(ValueError):
        spffn.hot_first_order(_i(F), perm=_i(F - 1))


def test_permute_and_repack_reject_sizes():
    with pytest.raises(ValueError):
        spffn.permute_rows(_f(8, 4), _i(7))
    with pytest.raises(ValueError):
        spffn.permute_rows(_f(8, 4), _i(8), dst=_f(8, 3))
    with pytest.raises(ValueError):
        spffn.q4_0_repack(_u(4 * 2 * 18 - 1), 4, 64)
    with pytest.raises(ValueError):
        spffn.q4_0_repack(_u(4 * 2 * 18), 4, 64, soa=_u(4 * 2 * 18 + 1))
    with pytest.raises(ValueError):
        spffn.q4_0_repack(_u(4 * 18), 4, 48)                   # cols not a multiple of 32


def test_threshold_and_compact_reject_sizes():
    with pytest.raises(ValueError):
        spffn.threshold(_f(F), 0.0, mask=_u(F - 1))
    with pytest.raises(ValueError):
        spffn.compact(_u(F), idx=_i(F - 1))
    with pytest.raises(ValueError):
        spffn.compact(_u(F), count=_i(0))


def _weights(**over):
    w = dict(kind="reglu", w_dtype="f16", p_dtype="f16", d=D, d_ffn=F, r=R, tau=0.5,
             w_gate=torch.zeros(F, D, dtype=torch.float16),
             w_up=torch.zeros(F, D, dtype=torch.float16),
             w_down_t=torch.zeros(F, D, dtype=torch.float16), b_act=_f(F),
             p_w1=torch.zeros(R, D, dtype=torch.float16), p_b1=_f(R),
             p_w2=torch.zeros(F, R, dtype=torch.float16), p_b2=_f(F))
    w.update(over)
    return w


@pytest.mark.parametrize("over", [
    dict(w_gate=torch.zeros(F - 1, D, dtype=torch.float16)),
    dict(w_up=torch.zeros(F, D + 8, dtype=torch.float16)),
    dict(w_down_t=torch.zeros(F // 2, D, dtype=torch.float16)),
    dict(b_act=_f(F + 1)),
    dict(p_w1=torch.zeros(R, D - 8, dtype=torch.float16)),
    dict(p_b1=_f(R - 1)),
    dict(p_w2=torch.zeros(F, R + 8, dtype=torch.float16)),
    dict(p_b2=_f(F - 1)),
    dict(w_dtype="q4_0", w_gate=_u(F * (D // 32) * 18 - 1), w_up=_u(F * (D // 32) * 18),
         w_down_t=_u(F * (D // 32) * 18)),
])
def test_layer_rejects_weight_sizes(over):
    with pytest.raises(ValueError):
        spffn.Layer(_weights(**over))


def test_layer_right_sizes_reach_device_check():
    with pytest.raises(TypeError, match="CUDA"):
        spffn.Layer(_weights())


def test_workspace_size_checked():
    from activation_sparse_mlp_amd._lib import _ws_bytes
    with pytest.raises(TypeError):
        _ws_bytes(_u(1 << 20), 1 << 10)  # host memory is not a workspace
