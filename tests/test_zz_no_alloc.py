"""The decode step without a caller workspace (spffn_decode_step_noalloc,
called through the C ABI's binding) gives bit for bit what spffn_decode_step
gives with a workspace of its own, on two calls in a row of which the second
has a smaller input (fewer tokens, then a smaller model), so leftovers of the
first call in the shared static array cannot leak into the second; the
single-token layer kernel (whose counters must start at zero) and the batched
path both run on it."""
from dataclasses import replace

import pytest
import torch

import activation_sparse_mlp_amd as spffn
from tests.gpu_helpers import DEV, gpu_layer
from workloads import LLAMA2_7B, TINY, make_layer, make_tokens

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _model(cfg, layers, seed):
    return spffn.Model([gpu_layer(make_layer(cfg, l, seed=seed, n_cal=512))
                        for l in range(layers)], rms_eps=1e-5)


def _pair(model, x):
    counts_ref = torch.empty(model.n_layers, dtype=torch.int32, device=DEV)
    counts = torch.full((model.n_layers,), -7, dtype=torch.int32, device=DEV)
    ref = spffn.decode_step(model, x, layer_counts=counts_ref)
    got = spffn.decode_step_noalloc(model, x, layer_counts=counts)
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    assert torch.equal(got, ref)
    assert torch.equal(counts, counts_ref)
    return got


def test_noalloc_equals_workspace_step_twice_second_smaller():
    cfg = replace(LLAMA2_7B, d=4096, d_ffn=2816, r=512)  # fp16 ReGLU rows: matrix cores at B=4
    big = _model(cfg, 3, seed=81)
    xb = make_tokens(cfg.d, 1, 4, seed=82, device=DEV)[0]
    print("noalloc: 3 fp16 layers, B=4 (matrix cores)", flush=True)
    _pair(big, xb)                       # batched path, B = 4
    print("noalloc: same model, B=1", flush=True)
    _pair(big, xb[:1].contiguous())      # smaller input: one token
    small = _model(TINY, 2, seed=83)
    print("noalloc: tiny model, B=1", flush=True)
    _pair(small, make_tokens(TINY.d, 1, 1, seed=84, device=DEV)[0])
    print("noalloc: big model again, B=1, dense", flush=True)
    ref = spffn.decode_step(big, xb[:1].contiguous(), dense=True)
    got = spffn.decode_step_noalloc(big, xb[:1].contiguous(), dense=True)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
