"""A decode step captured into a HIP graph replays exactly what the eager call
computes: every replay (with other eager work and synchronisation between
replays, and a new input written into the captured x each time) is compared
bit for bit with an eager decode_step on the same input, which the other GPU
tests check against the oracle."""
from dataclasses import replace

import pytest
import torch

import activation_sparse_mlp_amd as spffn
from tests.gpu_helpers import DEV, gpu_layer
from tests.test_gpu_mixed import CFGS as MIXED
from workloads import LLAMA2_7B, OPT_175B_Q4, TINY, make_layer, make_tokens

pytestmark = pytest.mark.gpu

# 4-bit rows at a small shape; 1530 neurons leave the last 20-row group ragged
_Q4 = replace(OPT_175B_Q4, d=512, d_ffn=1530, r=64)


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _model(cfg, layers):
    # 4-bit layers are generated on the host, as in the parity tests
    dev = "cpu" if cfg.w_dtype == "q4_0" else DEV
    gl = [gpu_layer(make_layer(cfg, l, seed=0, device=dev, n_cal=512)) for l in range(layers)]
    return spffn.Model(gl, rms_eps=1e-5)


@pytest.mark.parametrize("cfg,layers,B,dense", [
    (TINY, 2, 1, False),          # fp32 rows, single-token fused path
    (LLAMA2_7B, 2, 1, False),     # fp16 rows, single-token fused path
    (LLAMA2_7B, 2, 4, False),     # batched union path
    (LLAMA2_7B, 1, 12, False),    # batched, two row tiles per workgroup
    (LLAMA2_7B, 1, 1, True),      # dense baseline
    (_Q4, 2, 1, False),           # 4-bit rows, single-token fused path
    (_Q4, 2, 3, False),           # 4-bit rows, batched vector path
])
def test_graph_replays_match_eager(cfg, layers, B, dense):
    print(f"graph {cfg.name} layers={layers} B={B} dense={dense}", flush=True)
    _replays_match_eager(_model(cfg, layers), cfg.d, layers, B, dense, cfg.d_ffn)


@pytest.mark.parametrize("B", [1, 3])
def test_graph_mixed_stack(B):
    """Layers of different kinds, formats and shapes (per-kernel path at one
    token; matrix-core and vector layers in turn at three)."""
    print(f"graph mixed stack B={B}", flush=True)
    gl = [gpu_layer(make_layer(c, l, seed=3, n_cal=512)) for l, c in enumerate(MIXED)]
    _replays_match_eager(spffn.Model(gl, rms_eps=1e-5), MIXED[0].d, len(MIXED), B, False, None)


def _replays_match_eager(model, d, layers, B, dense, d_ffn):
    xs = make_tokens(d, 4, B, seed=9, device=DEV)
    xbuf = torch.empty(B, d, device=DEV)
    hbuf = torch.empty(B, d, device=DEV)
    cnt = torch.full((layers,), -1, dtype=torch.int32, device=DEV)
    g = spffn.DecodeGraph(model, xbuf, hbuf, dense=dense, layer_counts=cnt)
    torch.cuda.synchronize()
    # capturing enqueues nothing
    assert torch.all(cnt == -1)
    for rep in range(4):
        xbuf.copy_(xs[rep])
        g.launch()
        torch.cuda.synchronize()
        got_h, got_c = hbuf.clone(), cnt.clone()
        # eager reference with its own workspace, plus unrelated work on the stream
        ref_c = torch.empty_like(cnt)
        ref_h = spffn.decode_step(model, xs[rep], dense=dense, layer_counts=ref_c)
        junk = torch.randn(1 << 16, device=DEV).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(got_h, ref_h), f"replay {rep}: h differs"
        assert torch.equal(got_c, ref_c), f"replay {rep}: layer counts differ"
        if dense:
            assert all(int(c) == d_ffn for c in got_c)
    del g


def test_graph_inputs_are_captured_by_address():
    """Writing a new token into the captured input changes the output; the
    caller's other buffers are untouched."""
    model = _model(TINY, 1)
    xbuf = torch.empty(1, TINY.d, device=DEV)
    hbuf = torch.empty(1, TINY.d, device=DEV)
    g = spffn.DecodeGraph(model, xbuf, hbuf)
    xs = make_tokens(TINY.d, 2, 1, seed=4, device=DEV)
    outs = []
    for k in range(2):
        xbuf.copy_(xs[k])
        outs.append(g.launch().clone())
    torch.cuda.synchronize()
    assert not torch.equal(outs[0], outs[1])
    assert torch.equal(outs[1], spffn.decode_step(model, xs[1]))
