"""Decode steps through a stack whose layers differ in kind, weight format,
neuron count and predictor width (only d is shared).  Such a stack leaves the
single-token layer kernel (it needs every layer alike) for the per-kernel path
at batch 1.  At batch 3 it alternates between matrix-core layers (fp16 rows
and predictor) and vector layers, so the residual stream passes between the
two batched paths in both directions, and two adjacent matrix-core layers of
different shapes hand the split input of the next layer from one to the
other.  Every layer is checked against the oracle on the input the GPU
actually gave it."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import activation_sparse_mlp_amd as spffn
import oracle
from tests.gpu_helpers import (DEV, REL_L2, check_mask_agreement, gpu_layer, np_layer, rel_l2)
from workloads import LLAMA2_7B, make_layer, make_tokens

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


D = 4096  # the matrix-core path needs d % 4096 == 0 and r % 512 == 0
_BASE = replace(LLAMA2_7B, d=D, tau=0.45)
CFGS = [
    replace(_BASE, kind="relu", w_dtype="f32", p_dtype="f32", d_ffn=768, r=64),
    replace(_BASE, kind="reglu", w_dtype="f16", p_dtype="f16", d_ffn=1003, r=512),
    # next to the layer above with another shape: the split input is handed over
    replace(_BASE, kind="relu", w_dtype="f16", p_dtype="f16", d_ffn=1200, r=512),
    replace(_BASE, kind="relu", w_dtype="q4_0", p_dtype="f16", d_ffn=640, r=64),
    replace(_BASE, kind="reglu", w_dtype="f16", p_dtype="f16", d_ffn=1536, r=512),
]


@pytest.mark.parametrize("B", [1, 3])
def test_decode_mixed_layers(B):
    print(f"mixed-layer decode B={B}", flush=True)
    seed = 61
    hosts = [make_layer(c, l, seed=seed, n_cal=1024) for l, c in enumerate(CFGS)]
    Ls = [np_layer(w) for w in hosts]
    model = spffn.Model([gpu_layer(w) for w in hosts], rms_eps=1e-5)
    n = len(CFGS)
    Fs = [c.d_ffn for c in CFGS]
    x = make_tokens(D, 1, B, seed=seed + 4)[0].to(DEV)
    trace = dict(h_in=torch.empty(n, B, D, device=DEV),
                 union_mask=torch.empty(sum(Fs), dtype=torch.uint8, device=DEV),
                 logits=torch.empty(B * sum(Fs), device=DEV))
    counts = torch.empty(n, dtype=torch.int32, device=DEV)
    h = spffn.decode_step(model, x, layer_counts=counts, trace=trace)
    torch.cuda.synchronize()
    h_in = trace["h_in"].cpu().numpy().astype(np.float64)
    assert np.array_equal(h_in[0], x.cpu().numpy())
    outs = np.concatenate([h_in[1:], h.cpu().numpy()[None].astype(np.float64)])
    um = trace["union_mask"].cpu().numpy()
    lg_all = trace["logits"].cpu().numpy()
    cnts = counts.cpu().numpy()
    m_off = l_off = 0
    for l, F in enumerate(Fs):
        U = um[m_off:m_off + F]
        lg = lg_all[l_off:l_off + B * F].reshape(B, F)
        m_off += F
        l_off += B * F
        assert cnts[l] == U.sum(), l
        ref = oracle.decode_layer(Ls[l], h_in[l], 1e-5, mask=U)
        for b in range(B):
            check_mask_agreement(oracle.threshold(lg[b], Ls[l]["t"]), ref["logits"][b],
                                 Ls[l]["t"])
        assert np.array_equal(U, oracle.union(oracle.threshold(lg, Ls[l]["t"])))
        for b in range(B):
            assert rel_l2(outs[l][b] - h_in[l][b], ref["y"][b]) <= REL_L2, (l, b)
    # fixed summation order: a second step gives the same bits
    h2 = spffn.decode_step(model, x)
    assert torch.equal(h, h2)
