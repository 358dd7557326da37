"""GPU parity of the 8-bit (OCP E4M3, one fp32 scale per row) predictor.

The kernels' E4M3 decode is checked on every finite code: a predictor whose
first layer passes one input through unchanged (E4M3 1.0 on the diagonal) and
whose second layer holds code i in row i turns the logits into the decoded
codes, which must equal the oracle's decode (from the format's definition)
bit for bit, on the single-token kernels and on the batched vector kernels.
Then predictor and decode steps with fp8 predictors are compared with the
oracle on the same fp8 weights: the single-token layer kernel, the batched
vector path and a full 70B-shaped layer pair."""
from dataclasses import replace

import numpy as np
import pytest
import torch

import activation_sparse_mlp_amd as spffn
import oracle
from tests.gpu_helpers import DEV, gpu_layer, np_layer
from tests.test_gpu_fullsize import _decode_check
from tests.test_gpu_kernels import _decode_checks, _predict_case
from workloads import LLAMA2_7B, LLAMA2_70B_FP8P, OPT_175B_Q4, TINY

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _fp8_buf(codes, scales):
    return torch.cat([torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).reshape(-1),
                      torch.from_numpy(np.asarray(scales, np.float32)).view(torch.uint8)])


@pytest.mark.parametrize("B", [1, 2])
def test_fp8_decode_every_code(B):
    d = r = 16
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)  # 254 finite
    F = codes.size
    w1 = np.zeros((r, d), np.uint8)
    np.fill_diagonal(w1, 0x38)                      # E4M3 1.0
    w2 = np.zeros((F, r), np.uint8)
    w2[:, 0] = codes                                 # row i reads hid[0] with code i
    f32 = lambda a: torch.tensor(a, dtype=torch.float32)  # noqa: E731
    w = dict(kind="relu", w_dtype="f32", p_dtype="fp8", d=d, d_ffn=F, r=r, tau=0.5,
             w_gate=None, w_up=torch.zeros(F, d), w_down_t=torch.zeros(F, d),
             b_act=torch.zeros(F), p_w1=_fp8_buf(w1, np.ones(r)), p_b1=torch.zeros(r),
             p_w2=_fp8_buf(w2, np.ones(F)), p_b2=torch.zeros(F))
    G = gpu_layer(w)
    x = torch.zeros(B, d)
    x[:, 0] = 1.0                                    # hid = e_0, so logit i = e4m3(code i)
    out = spffn.predict(G, x.to(DEV))
    torch.cuda.synchronize()
    want = oracle.e4m3_to_f64(codes)
    for b in range(B):
        got = out["logits"][b].cpu().numpy().astype(np.float64)
        assert np.array_equal(got, want)
        assert np.array_equal(out["mask"][b].cpu().numpy(), (want > 0).astype(np.uint8))
    L = np_layer(w)
    _, ref_logits, _ = oracle.predict(L, x[0].numpy())
    assert np.array_equal(ref_logits, want)


_F16_FP8 = replace(LLAMA2_7B, d=512, d_ffn=1536, r=64, p_dtype="fp8")
_F32_FP8 = replace(TINY, p_dtype="fp8")
_Q4_FP8 = replace(OPT_175B_Q4, d=512, d_ffn=1530, r=64, layers=2, p_dtype="fp8")


@pytest.mark.parametrize("cfg", [_F32_FP8, _F16_FP8, _Q4_FP8])
@pytest.mark.parametrize("B", [1, 3])
def test_fp8_predict(cfg, B):
    print(f"fp8 predict {cfg.name} B={B}", flush=True)
    _predict_case(cfg, B, seed=61)


@pytest.mark.parametrize("cfg", [_F32_FP8, _F16_FP8, _Q4_FP8])
@pytest.mark.parametrize("B", [1, 3])
def test_fp8_decode(cfg, B):
    print(f"fp8 decode {cfg.name} B={B}", flush=True)
    _decode_checks(cfg, B, 2, seed=63, n_cal=512)


def test_fp8_llama2_70b_decode_b1():
    """The full 70B shape with the fp8 predictor, two layers as the
    benchmark builds them (hot-first rows)."""
    _decode_check(LLAMA2_70B_FP8P, 1, 2, hot_first=True)
