"""The five synthetic FFN-stack workloads (shapes of real model families).

Each entry fixes the FFN shape, the weight storage, the power-law firing
statistics and the predictor size.  Firing follows [Guide] section 1: the
activation frequency of the rank-k neuron falls off as k^-gamma, gamma > 1
("PowerInfer Guide: Exploiting Activation Sparsity for LLM AI", section 1
"Empirical Power-Law Distribution and Skewness").  Mean activities of 5-10%
sit in that page's "80% to 90% of neurons are exactly zero" band
("The Hidden Inefficiency").
"""
from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Config:
    name: str
    kind: str            # "relu" (non-gated up/down), "reglu" or "swiglu" (gated)
    d: int
    d_ffn: int
    layers: int
    w_dtype: str         # "f32" | "f16" | "q4_0"
    p_dtype: str         # predictor weights: "f32" | "f16" | "fp8" (E4M3, a scale per row)
    r: int               # predictor hidden width
    gamma: float         # power-law exponent of firing probability vs rank
    mean_activity: float
    tokens: int
    batches: Tuple[int, ...] = (1,)
    w_std: float = 0.02  # std of fp weights (fp32 / fp16 configs)
    gate_std: float = 0.0  # std of the gate matrix when set (else w_std)
    q4_scale_std: float = 0.003  # std of the |N(0, s^2)| block scales (q4_0)
    tau: float = 0.5
    hot_first: bool = False
    dense_prefix: bool = False  # neurons active on every profiling token run unscored
    description: str = field(default="", compare=False)


TINY = Config(
    name="tiny_relu", kind="relu", d=256, d_ffn=1024, layers=2, w_dtype="f32", p_dtype="f32",
    r=64, gamma=1.2, mean_activity=0.10, tokens=16, w_std=256 ** -0.5,
    description="Tiny ReLU FFN (OPT-style, non-gated), fp32 weights ~N(0, 1/d)")

LLAMA2_7B = Config(
    name="llama2_7b_reglu", kind="reglu", d=4096, d_ffn=11008, layers=32, w_dtype="f16",
    p_dtype="f16", r=1024, gamma=1.2, mean_activity=0.10, tokens=128,
    description="Llama2-7B-shaped ReGLU FFN (ProSparse-like), fp16")

# SwiGLU: SiLU is never exactly zero, so the gate weights are wider (std 0.1,
# ||w_gate|| ~ 6.4) to make the activation magnitude-sparse: a neuron whose
# gate pre-activation sits a typical distance below zero has |silu(z)| of
# about 1e-3 and below ([Guide] "The Hidden Inefficiency": SwiGLU
# activations are near-zero magnitudes rather than exact zeros).
LLAMA2_7B_SWIGLU = Config(
    name="llama2_7b_swiglu", kind="swiglu", d=4096, d_ffn=11008, layers=32, w_dtype="f16",
    p_dtype="f16", r=1024, gamma=1.2, mean_activity=0.10, tokens=128, gate_std=0.1,
    description="Llama2-7B-shaped SwiGLU FFN (magnitude-sparse gate), fp16")

FALCON_40B = Config(
    name="falcon_40b_relu", kind="relu", d=8192, d_ffn=32768, layers=60, w_dtype="f16",
    p_dtype="f16", r=1024, gamma=1.1, mean_activity=0.08, tokens=128, batches=(1, 8),
    description="Falcon-40B-shaped ReLU FFN (non-gated up/down), fp16")

LLAMA2_70B = Config(
    name="llama2_70b_reglu", kind="reglu", d=8192, d_ffn=28672, layers=80, w_dtype="f16",
    p_dtype="f16", r=1024, gamma=1.2, mean_activity=0.10, tokens=256, batches=(1, 4, 16),
    hot_first=True,
    description="Llama2-70B-shaped ReGLU FFN, fp16, hot-first permuted rows")

# The same stack with an 8-bit predictor (OCP E4M3 codes, one fp32 scale per
# row): half the predictor bytes ([x64] list item 2 and [Guide] section 3
# describe a small, low-rank predictor; its bytes are a third of a step here).
LLAMA2_70B_FP8P = Config(
    name="llama2_70b_reglu_fp8pred", kind="reglu", d=8192, d_ffn=28672, layers=80, w_dtype="f16",
    p_dtype="fp8", r=1024, gamma=1.2, mean_activity=0.10, tokens=256, batches=(1, 4, 16),
    hot_first=True,
    description="Llama2-70B-shaped ReGLU FFN, fp16, hot-first rows, fp8 (E4M3) predictor")

# Hot-first rows with the always-active prefix: the neurons that fire on every
# profiling token are computed for every token without predictor rows
# ([Guide] section 2: hot neurons always at hand; section 4: neuron blocks).
LLAMA2_70B_PREFIX = Config(
    name="llama2_70b_reglu_prefix", kind="reglu", d=8192, d_ffn=28672, layers=80,
    w_dtype="f16", p_dtype="f16", r=1024, gamma=1.2, mean_activity=0.10, tokens=256,
    batches=(1, 4, 16), hot_first=True, dense_prefix=True,
    description="Llama2-70B-shaped ReGLU FFN, fp16, hot-first rows, always-active prefix")

OPT_175B_Q4 = Config(
    name="opt_175b_relu_q4_0", kind="relu", d=12288, d_ffn=49152, layers=96, w_dtype="q4_0",
    p_dtype="f16", r=1024, gamma=1.3, mean_activity=0.05, tokens=128,
    description="OPT-175B-shaped ReLU FFN with 4-bit (Q4_0 block) weights, fp16 predictor")

ALL = {c.name: c for c in (TINY, LLAMA2_7B, LLAMA2_7B_SWIGLU, FALCON_40B, LLAMA2_70B,
                           LLAMA2_70B_FP8P, LLAMA2_70B_PREFIX, OPT_175B_Q4)}
