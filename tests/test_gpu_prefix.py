"""GPU parity of the always-active prefix (the first k stored neurons run for
every token, unscored): against the oracle's decode layer with the same
prefix, teacher forced, on the single-token layer kernel, the per-kernel
single-token path (a stack of unlike layers), the batched vector kernels and
the matrix cores; and the load-time choice of the prefix (neurons that fired
on every profiling token) at the full 70B shape."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import activation_sparse_mlp_amd as spffn
import oracle
from tests.gpu_helpers import DEV, REL_L2, check_mask_agreement, gpu_layer, np_layer, rel_l2
from tests.test_gpu_fullsize import _decode_check
from tests.test_gpu_mixed import CFGS as MIXED
from workloads import LLAMA2_7B, LLAMA2_70B_PREFIX, TINY, make_layer, make_tokens

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_F16 = replace(LLAMA2_7B, d=512, d_ffn=1536, r=64)
_MF = replace(LLAMA2_7B, d=4096, d_ffn=1000, r=512)


def _check(cfgs, prefixes, B, seed):
    layers = len(cfgs)
    hosts = []
    for l, (c, k) in enumerate(zip(cfgs, prefixes)):
        w = make_layer(c, l, seed=seed, n_cal=512)
        w["dense_prefix"] = k
        hosts.append(w)
    model = spffn.Model([gpu_layer(w) for w in hosts], rms_eps=1e-5)
    Ls = [np_layer(w) for w in hosts]
    d = cfgs[0].d
    x = make_tokens(d, 1, B, seed=seed + 1, device=DEV)[0]
    F = [c.d_ffn for c in cfgs]
    trace = dict(h_in=torch.empty(layers, B, d, device=DEV),
                 union_mask=torch.empty(sum(F), dtype=torch.uint8, device=DEV),
                 logits=torch.empty(B * sum(F), device=DEV))
    counts = torch.empty(layers, dtype=torch.int32, device=DEV)
    print(f"prefix decode {cfgs[0].name} x{layers} B={B} k={prefixes}", flush=True)
    h = spffn.decode_step(model, x, layer_counts=counts, trace=trace)
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
        k = prefixes[l]
        assert cnts[l] == U.sum() and np.all(U[:k] == 1)
        assert np.all(np.isposinf(lgl[:, :k]))  # prefix neurons are not scored
        assert np.array_equal(U, oracle.union(oracle.threshold(lgl, Ls[l]["t"])))
        ref = oracle.decode_layer(Ls[l], h_in[l], 1e-5, mask=U)
        for b in range(B):
            check_mask_agreement(oracle.threshold(lgl[b], Ls[l]["t"]), ref["logits"][b],
                                 Ls[l]["t"])
            assert rel_l2(outs[l][b] - h_in[l][b], ref["y"][b]) <= REL_L2, (l, b)


@pytest.mark.parametrize("cfg,B", [(TINY, 1), (_F16, 1), (_F16, 3), (_MF, 4), (_MF, 11)])
def test_prefix_matches_oracle(cfg, B):
    _check([cfg, cfg], [cfg.d_ffn // 7, 3], B, seed=101)


@pytest.mark.parametrize("B", [1, 3])
def test_prefix_mixed_stack(B):
    _check(MIXED, [c.d_ffn // 5 for c in MIXED], B, seed=103)


def test_prefix_every_neuron_equals_dense():
    cfg = _F16
    w = make_layer(cfg, 0, seed=105, n_cal=512)
    dense = spffn.Model([gpu_layer(w)])
    full = spffn.Model([gpu_layer(dict(w, dense_prefix=cfg.d_ffn))])
    x = make_tokens(cfg.d, 1, 1, seed=106, device=DEV)[0]
    a = spffn.decode_step(full, x)
    b = spffn.decode_step(dense, x, dense=True)
    torch.cuda.synchronize()
    assert float((a - b).norm() / b.norm()) < 1e-5


def test_prefix_70b_shape_as_benchmarked():
    """Two 70B-shaped layers with the prefix chosen at load (neurons active on
    every one of the 256 profiling tokens: the saturated ones and more)."""
    _decode_check(LLAMA2_70B_PREFIX, 1, 2, hot_first=True)
