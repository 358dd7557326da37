"""GPU parity of the batched matrix-core path (fp16 weights, 2 <= B <= 16)
against the CPU oracle: predictor, forward over a mask / an index list /
every neuron / an empty set, and the decode step, at shapes with a ragged row
tail (d_ffn not a multiple of the 16-row tiles or of the 32-row down steps)
and with both ways of carrying the fp16 halves (B <= 8 shares one instruction,
B > 8 takes two)."""
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
