"""GPU parity of the batched matrix-core path (fp16 weights, 2 <= B <= 16)
against the CPU oracle: predictor, forward over a mask / an index list /
every neuron / an empty set, and the decode step, at shapes with a ragged row
tail (d_ffn not a multiple of the 16-row tiles or of the 32-row down steps)
and with both ways of carrying the fp16 halves (B <= 8 shares one instruction,
B > 8 takes two); the wide shape (d = 8192, r = 1024) runs the predictor
products with eight waves per workgroup."""
from dataclasses import replace

import pytest
import torch

from tests.gpu_helpers import DEV
from tests.test_gpu_kernels import _decode_checks, _forward_checks, _predict_case
from workloads import LLAMA2_7B

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cfg(kind):
    # d a multiple of 4096 and r of 512 select the matrix-core kernels
    return replace(LLAMA2_7B, kind=kind, d=4096, d_ffn=1000, r=512, layers=2, tau=0.45)


def _cfg_wide(kind):
    # d = 8192 and r = 1024: the predictor products split K over 8 waves
    return replace(LLAMA2_7B, kind=kind, d=8192, d_ffn=1000, r=1024, layers=1, tau=0.45)


@pytest.mark.parametrize("B", [2, 8, 9, 16])
def test_mfma_predict(B):
    print(f"mfma predict B={B}", flush=True)
    _predict_case(_cfg("reglu"), B, seed=21)


@pytest.mark.parametrize("kind", ["reglu", "relu"])
@pytest.mark.parametrize("B", [2, 5, 9, 16])
def test_mfma_forward(kind, B):
    _forward_checks(_cfg(kind), B, seed=31)


@pytest.mark.parametrize("B", [3, 12])
def test_mfma_decode(B):
    print(f"mfma decode B={B}", flush=True)
    _decode_checks(_cfg("reglu"), B, 2, seed=41)


@pytest.mark.parametrize("B", [4, 12])
def test_mfma_predict_wide(B):
    print(f"mfma predict wide B={B}", flush=True)
    _predict_case(_cfg_wide("reglu"), B, seed=23)


@pytest.mark.parametrize("B", [5, 16])
def test_mfma_decode_wide(B):
    print(f"mfma decode wide B={B}", flush=True)
    _decode_checks(_cfg_wide("relu"), B, 1, seed=47)


def test_mfma_decode_dense():
    _decode_checks(_cfg("relu"), 4, 1, seed=43, dense=True)


def test_mfma_list_longer_than_tiles():
    """A list covering every row of a layer whose row count is not a multiple
    of 16 or 32 (last tile and last down step partly empty) equals dense."""
    import activation_sparse_mlp_amd as spffn
    from tests.gpu_helpers import gpu_layer
    from workloads import make_layer, make_tokens
    cfg = replace(_cfg("reglu"), d_ffn=1000 + 17)
    G = gpu_layer(make_layer(cfg, 0, seed=5, n_cal=512))
    x = make_tokens(cfg.d, 1, 6, seed=6)[0].to(DEV)
    idx = torch.arange(cfg.d_ffn, dtype=torch.int32, device=DEV)
    cnt = torch.tensor([cfg.d_ffn], dtype=torch.int32, device=DEV)
    assert torch.equal(spffn.forward(G, x, idx=idx, count=cnt), spffn.forward(G, x))


def _forced_model(cfg, b2, layers=2):
    """Layers whose predictor bias is the constant b2: every logit is then
    far on one side of the threshold (all neurons active or none)."""
    import activation_sparse_mlp_amd as spffn
    from tests.gpu_helpers import gpu_layer
    from workloads import make_layer
    ws = [make_layer(cfg, l, seed=7, n_cal=512) for l in range(layers)]
    for w in ws:
        w["p_b2"] = torch.full_like(w["p_b2"], b2)
    return spffn.Model([gpu_layer(w) for w in ws], rms_eps=1e-5)


@pytest.mark.parametrize("B", [3, 12])
def test_mfma_no_neuron_active_keeps_residual(B):
    """Empty union: the on-device list is empty, the residual passes through."""
    import activation_sparse_mlp_amd as spffn
    from workloads import make_tokens
    cfg = _cfg("relu")
    model = _forced_model(cfg, -1e4)
    x = make_tokens(cfg.d, 1, B, seed=4, device=DEV)[0]
    counts = torch.full((2,), -1, dtype=torch.int32, device=DEV)
    h = spffn.decode_step(model, x, layer_counts=counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0, 0]
    assert torch.equal(h, x)


@pytest.mark.parametrize("d_ffn,B", [(1000, 4), (8320, 4), (8320, 10)])
def test_mfma_every_neuron_active_equals_dense(d_ffn, B):
    """Every row in the union: the list built from tile masks is 0..d_ffn-1,
    so the step equals the dense step.  8320 rows are 520 tiles, more than one
    pass of the gather's workgroups, which then loop."""
    import activation_sparse_mlp_amd as spffn
    from workloads import make_tokens
    cfg = replace(_cfg("reglu"), d_ffn=d_ffn)
    model = _forced_model(cfg, 1e4, layers=1)
    x = make_tokens(cfg.d, 1, B, seed=3, device=DEV)[0]
    counts = torch.empty(1, dtype=torch.int32, device=DEV)
    h = spffn.decode_step(model, x, layer_counts=counts)
    hd = spffn.decode_step(model, x, dense=True)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [d_ffn]
    rel = float((h - hd).norm() / hd.norm())
    assert rel < 1e-6, rel
