"""GPU parity of SwiGLU layers (SiLU on the gate) against the oracle on the
same masks: the single-token layer kernel, the batched vector kernels, the
matrix cores and a mixed stack, and the 7B-shaped SwiGLU workload at full
shape.  SiLU is evaluated with the hardware exponential in fp32; the bound is
the FFN tolerance."""
from dataclasses import replace

import pytest
import torch

from tests.test_gpu_fullsize import _decode_check
from tests.test_gpu_kernels import _decode_checks, _forward_checks
from workloads import LLAMA2_7B, LLAMA2_7B_SWIGLU, OPT_175B_Q4, TINY

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_SW16 = replace(LLAMA2_7B_SWIGLU, d=512, d_ffn=1536, r=64, gate_std=0.1 * 8 ** 0.5)
_SW32 = replace(TINY, kind="swiglu")
_SWQ4 = replace(OPT_175B_Q4, kind="swiglu", d=512, d_ffn=1530, r=64, layers=2)
_SWMF = replace(LLAMA2_7B, kind="swiglu", d=4096, d_ffn=1000, r=512, tau=0.45, gate_std=0.1)


@pytest.mark.parametrize("cfg,B", [(_SW32, 1), (_SW16, 1), (_SW16, 3), (_SWQ4, 1), (_SWQ4, 3),
                                   (_SWMF, 4), (_SWMF, 12)])
def test_swiglu_decode(cfg, B):
    print(f"swiglu decode {cfg.name} d={cfg.d} B={B}", flush=True)
    _decode_checks(cfg, B, 2, seed=111, n_cal=512)


@pytest.mark.parametrize("cfg,B", [(_SW16, 1), (_SW16, 5), (_SWMF, 9)])
def test_swiglu_forward(cfg, B):
    _forward_checks(cfg, B, seed=113, n_cal=512)


def test_swiglu_7b_full_shape():
    _decode_check(LLAMA2_7B_SWIGLU, 1, 2, hot_first=False)
