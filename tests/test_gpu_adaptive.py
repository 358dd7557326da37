"""GPU parity of the decode step with a logit threshold per token and per
layer (spffn_decode_step_adaptive; the Guide's adaptive dynamic thresholding)
against the oracle's decode layer with the same thresholds, teacher forced,
on every path that thresholds: the single-token layer kernel, the per-kernel
single-token path (a stack of unlike layers), the batched vector kernels and
the matrix cores.  Thresholds equal to each layer's own give the plain decode
step bit for bit."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import activation_sparse_mlp_amd as spffn
import oracle
from tests.gpu_helpers import DEV, REL_L2, check_mask_agreement, gpu_layer, np_layer, rel_l2
from tests.test_gpu_mixed import CFGS as MIXED
from workloads import LLAMA2_7B, OPT_175B_Q4, TINY, make_layer, make_tokens

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_F16 = replace(LLAMA2_7B, d=512, d_ffn=1536, r=64)        # fp16 rows, vector path at B > 1
_MF = replace(LLAMA2_7B, d=4096, d_ffn=1000, r=512)       # matrix cores at B > 1
# single-token layer kernels whose row groups read their predictor rows in
# four passes (16-row groups, about 1024 of them) and gather in pairs
_F16_PASSES = replace(LLAMA2_7B, d=512, d_ffn=16384, r=64)
_Q4_PASSES = replace(OPT_175B_Q4, d=512, d_ffn=16390, r=64, layers=2)


def _check(cfgs, B, seed):
    layers = len(cfgs)
    hosts = [make_layer(c, l, seed=seed, n_cal=512) for l, c in enumerate(cfgs)]
    G = [gpu_layer(w) for w in hosts]
    Ls = [np_layer(w) for w in hosts]
    model = spffn.Model(G, rms_eps=1e-5)
    d = cfgs[0].d
    x = make_tokens(d, 1, B, seed=seed + 1, device=DEV)[0]
    # per-token thresholds around each layer's own: tau from 0.2 to 0.8
    rng = np.random.default_rng(seed)
    taus = rng.uniform(0.2, 0.8, size=(layers, B)).astype(np.float32)
    T = np.array([[spffn.tau_threshold(t) for t in row] for row in taus], np.float32)
    for l in range(layers):
        for b in range(B):
            assert T[l, b] == np.float32(oracle.logit_threshold(float(taus[l, b])))
    Td = torch.from_numpy(T).to(DEV)
    F = [c.d_ffn for c in cfgs]
    trace = dict(h_in=torch.empty(layers, B, d, device=DEV),
                 union_mask=torch.empty(sum(F), dtype=torch.uint8, device=DEV),
                 logits=torch.empty(B * sum(F), device=DEV))
    counts = torch.empty(layers, dtype=torch.int32, device=DEV)
    print(f"adaptive decode {[c.name for c in cfgs][0]} x{layers} B={B}", flush=True)
    h = spffn.decode_step_adaptive(model, x, Td, layer_counts=counts, trace=trace)
    torch.cuda.synchronize()
    h_in = trace["h_in"].cpu().numpy().astype(np.float64)
    outs = np.concatenate([h_in[1:], h.cpu().numpy()[None].astype(np.float64)])
    um = trace["union_mask"].cpu().numpy()
    lg = trace["logits"].cpu().numpy()
    cnts = counts.cpu().numpy()
    mo = lo = 0
    for l in range(layers):
        U = um[mo:mo + F[l]]
        lgl = lg[lo:lo + B * F[l]].reshape(B, F[l])
        mo += F[l]
        lo += B * F[l]
        assert cnts[l] == U.sum()
        # the union is the OR of each token's decision against its own threshold
        own = np.stack([oracle.threshold(lgl[b], T[l, b]) for b in range(B)])
        assert np.array_equal(U, oracle.union(own))
        ref = oracle.decode_layer(Ls[l], h_in[l], 1e-5, mask=U, thresholds=T[l])
        for b in range(B):
            check_mask_agreement(own[b], ref["logits"][b], T[l, b])
            assert np.array_equal(ref["masks"][b], ref["logits"][b] > T[l, b])
            assert rel_l2(outs[l][b] - h_in[l][b], ref["y"][b]) <= REL_L2, (l, b)
    # each layer's own threshold everywhere: the plain step, bit for bit
    T0 = torch.tensor([[G[l].t] * B for l in range(layers)], dtype=torch.float32, device=DEV)
    assert torch.equal(spffn.decode_step_adaptive(model, x, T0), spffn.decode_step(model, x))


@pytest.mark.parametrize("cfg,B", [
    (TINY, 1),      # fp32 rows, single-token layer kernel
    (_F16, 1),      # fp16 rows, single-token layer kernel
    (_F16_PASSES, 1),  # fp16 rows, row groups in four passes
    (_Q4_PASSES, 1),   # 4-bit rows, row groups in four passes
    (_F16, 3),      # batched vector path
    (_MF, 4),       # matrix cores, tokens sharing one instruction
    (_MF, 11),      # matrix cores, two instructions per tile
])
def test_adaptive_thresholds_match_oracle(cfg, B):
    _check([cfg, cfg], B, seed=91)


@pytest.mark.parametrize("B", [1, 3])
def test_adaptive_thresholds_mixed_stack(B):
    """Unlike layers: the per-kernel single-token path, or matrix-core and
    vector layers in turn."""
    _check(MIXED, B, seed=93)
