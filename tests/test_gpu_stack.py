"""End-to-end decode through a three-layer stack, not teacher forced: the GPU
step's final h against the oracle's whole-stack decode from the same input.
The seeds are ones whose every logit (in the oracle's binary64 run) stays at
least 1e-4 away from the threshold, far beyond the ~1e-6 logit error of the
GPU path, so both sides take the same masks and the outputs must agree to the
FFN tolerance; the margin is asserted so that the comparison stays meaningful."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import activation_sparse_mlp_amd as spffn
import oracle
from tests.gpu_helpers import DEV, REL_L2, gpu_layer, np_layer, rel_l2
from workloads import LLAMA2_7B, TINY, make_layer, make_tokens

pytestmark = pytest.mark.gpu

_F16 = replace(LLAMA2_7B, d=512, d_ffn=1536, r=64)


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("cfg,B,seed", [
    (TINY, 1, 71),    # fp32 rows, single-token layer kernel
    (TINY, 3, 71),    # fp32 rows, batched vector path
    (_F16, 1, 72),    # fp16 ReGLU rows, single-token layer kernel
    (_F16, 3, 72),    # fp16 ReGLU rows, batched vector path
])
def test_stack_decode_matches_oracle_stack(cfg, B, seed):
    print(f"stack decode {cfg.name} B={B} seed={seed}", flush=True)
    layers = 3
    hosts = [make_layer(cfg, l, seed=seed, n_cal=512) for l in range(layers)]
    Ls = [np_layer(w) for w in hosts]
    x = make_tokens(cfg.d, 1, B, seed=seed + 4)[0]
    # the oracle's stack, layer by layer for the margin, then as one call
    h = np.atleast_2d(x.numpy().astype(np.float64))
    margin = np.inf
    for L in Ls:
        out = oracle.decode_layer(L, h, 1e-5)
        margin = min(margin, float(np.min(np.abs(out["logits"] - L["t"]))))
        h = out["h"]
    assert margin >= 1e-4, margin
    ref = oracle.decode_step(Ls, x.numpy(), 1e-5)
    assert np.array_equal(ref, h)
    model = spffn.Model([gpu_layer(w) for w in hosts], rms_eps=1e-5)
    got = spffn.decode_step(model, x.to(DEV))
    torch.cuda.synchronize()
    got = np.atleast_2d(got.cpu().numpy().astype(np.float64))
    x64 = np.atleast_2d(x.numpy().astype(np.float64))
    for b in range(B):
        # compare what the stack added to the input
        assert rel_l2(got[b] - x64[b], ref[b] - x64[b]) <= REL_L2, b
