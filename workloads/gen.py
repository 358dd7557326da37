"""Seeded synthetic inputs for the neuron-sparse FFN: weights, biases, predictor
parameters and tokens.

This module only *constructs* inputs; both the CPU oracle and the GPU path
consume what it returns, and neither imports the other.  Everything is drawn
from torch generators seeded by (seed, layer, tensor tag), so a given call
reproduces bit-identical tensors on a given device type.

Construction (one layer):
  * firing probability of the rank-k neuron p_k = min(1 - 1e-6, c * k^-gamma),
    c chosen by bisection so that mean(p) equals the configured activity
    ([Guide] section 1 power law P(k) ~ k^-gamma); ranks are dealt to neurons
    by a seeded random permutation, so the stored order is not hot-first;
  * fp weights ~ N(0, std^2), rounded to the storage type; 4-bit weights are
    blocks of 32 codes uniform on 0..15 with an fp16 scale |N(0, s^2)|;
  * bias of the activated projection b_i = ||w_i|| * Phi^-1(p_i), so that
    P(w_i . x + b_i > 0) = p_i for x ~ N(0, I);
  * predictor: W1 ~ N(0, 1/d), b1 = 0; [W2 | b2] by ridge least squares of
    the true pre-activations on the hidden features over calibration tokens,
    then b2_i shifted so that the calibration firing rate of neuron i is p_i;
  * in a stack (make_stack) every layer after the first is calibrated on the
    normalised residual stream of the calibration tokens as the layers before
    it leave it, with the bias from a normal fit of each pre-activation there.
"""
import math

import numpy as np
import torch

from .configs import Config

# tensor tags mixed into the per-tensor seed
TAG_RANK, TAG_GATE, TAG_UP, TAG_DOWN, TAG_W1, TAG_CAL = 1, 2, 3, 4, 5, 6
TAG_Q4_CODES, TAG_Q4_SCALES, TAG_SHIFT = 7, 8, 9
TAG_TOKENS, TAG_PROFILE = 20, 21

Q4_0_BLOCK, Q4_0_BYTES = 32, 18


def _gen(device, seed, layer, tag):
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + (layer + 1) * 10_007 + tag * 101) % (2 ** 63 - 1))
    return g


def firing_probs(d_ffn, gamma, mean, cap=1.0 - 1e-6):
    """p_k for ranks k = 1..d_ffn (descending), mean(p) == mean."""
    k = np.arange(1, d_ffn + 1, dtype=np.float64)
    base = k ** -gamma
    lo, hi = 0.0, 1.0
    while np.minimum(cap, hi * base).mean() < mean:
        hi *= 2.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(cap, mid * base).mean() < mean:
            lo = mid
        else:
            hi = mid
    return np.minimum(cap, hi * base)


def q4_0_pack(codes, scales):
    """codes uint8 [rows, cols] in 0..15, scales fp16 [rows, cols/32] -> uint8
    [rows, cols/32*18] blocks: 2 scale bytes (little-endian), then 16 bytes whose
    byte k holds code k (low nibble) and code k+16 (high nibble)."""
    rows, cols = codes.shape
    nb = cols // Q4_0_BLOCK
    c = codes.reshape(rows, nb, Q4_0_BLOCK).to(torch.int32)
    packed = (c[:, :, :16] | (c[:, :, 16:] << 4)).to(torch.uint8)
    sb = scales.contiguous().view(torch.int16).to(torch.int32) & 0xFFFF
    lo = (sb & 0xFF).to(torch.uint8).unsqueeze(-1)
    hi = (sb >> 8).to(torch.uint8).unsqueeze(-1)
    return torch.cat([lo, hi, packed], dim=-1).reshape(rows, nb * Q4_0_BYTES).contiguous()


def q4_0_values(codes, scales):
    """Exact fp32 values (code - 8) * scale of unpacked 4-bit weights."""
    rows, cols = codes.shape
    s = scales.float().repeat_interleave(Q4_0_BLOCK, dim=1)
    return (codes.float() - 8.0) * s


FP8_E4M3_MAX = 448.0


def fp8_pack(w):
    """Predictor weights w fp32 [rows, cols] as OCP E4M3 codes with one fp32
    scale per row (max |w_i| / 448, so the largest weight of a row maps to the
    largest finite code), rounded to nearest even.  Returns (uint8 buffer of
    the rows*cols codes followed by the rows' fp32 scales, the fp32 values
    code * scale the buffer stands for)."""
    amax = w.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / FP8_E4M3_MAX, torch.ones_like(amax)).float()
    q = (w / scale[:, None]).clamp(-FP8_E4M3_MAX, FP8_E4M3_MAX).cpu().to(torch.float8_e4m3fn)
    codes = q.view(torch.uint8).to(w.device)
    vals = q.to(torch.float32).to(w.device) * scale[:, None]
    buf = torch.cat([codes.reshape(-1), scale.contiguous().view(torch.uint8)])
    return buf, vals


def _pred_store(w, p_dtype):
    """(stored tensor, fp32 values) of one predictor matrix."""
    if p_dtype == "fp8":
        return fp8_pack(w)
    if p_dtype == "f16":
        w = w.half()
        return w, w.float()
    return w, w


def _weights(cfg, g_codes_or_normal, g_scales, shape, device, std=None):
    """(stored tensor, fp32 values) of one weight matrix (fp: std, default
    the config's w_std)."""
    rows, cols = shape
    if cfg.w_dtype == "q4_0":
        codes = torch.randint(0, 16, shape, generator=g_codes_or_normal, device=device,
                              dtype=torch.uint8)
        scales = (torch.randn(rows, cols // Q4_0_BLOCK, generator=g_scales, device=device)
                  * cfg.q4_scale_std).abs().half()
        vals = q4_0_values(codes, scales)
        return q4_0_pack(codes, scales), vals
    w = torch.randn(shape, generator=g_codes_or_normal, device=device) * (std or cfg.w_std)
    if cfg.w_dtype == "f16":
        w = w.half()
        return w, w.float()
    return w, w


def make_layer(cfg: Config, layer: int, seed: int = 0, device="cpu", n_cal: int = 4096,
               return_values: bool = False, cal_inputs=None):
    """One layer of `cfg` as a dict of torch tensors on `device`.

    Keys: kind, w_dtype, p_dtype, d, d_ffn, r, tau, w_gate (ReGLU) / None,
    w_up, w_down_t ([d_ffn, d], W_down transposed), b_act fp32 [d_ffn],
    p_w1 [r, d], p_b1 fp32 [r], p_w2 [d_ffn, r], p_b2 fp32 [d_ffn],
    p_fire float64 numpy [d_ffn] (target firing probability per neuron).

    cal_inputs: None calibrates on fresh x ~ N(0, I) tokens (the input of a
    first layer); or a pair (fit, shift) of [n_cal, d] fp32 tensors, the
    normalised inputs this layer receives inside a stack (make_stack), on
    which the bias, the predictor fit and its shift are then taken."""
    dev = torch.device(device)
    d, F, r = cfg.d, cfg.d_ffn, cfg.r
    if cfg.w_dtype == "q4_0" and d % Q4_0_BLOCK:
        raise ValueError("4-bit blocks need d % 32 == 0")

    p_rank = firing_probs(F, cfg.gamma, cfg.mean_activity)
    order = torch.randperm(F, generator=_gen(dev, seed, layer, TAG_RANK), device=dev).cpu()
    p = p_rank[order.numpy()]

    def w(tag):
        std = cfg.gate_std if tag == TAG_GATE and cfg.gate_std else None
        return _weights(cfg, _gen(dev, seed, layer, tag), _gen(dev, seed, layer, tag + 40),
                        (F, d), dev, std)

    up_vals = None
    if cfg.kind != "relu":
        w_gate, act_vals = w(TAG_GATE)
        w_up, up_vals = w(TAG_UP)
    else:
        w_gate = None
        w_up, act_vals = w(TAG_UP)
    w_down_t, down_vals = w(TAG_DOWN)

    ppf = torch.special.ndtri(torch.from_numpy(p).to(dev))
    zfit = None
    if cal_inputs is None:
        # exact for x ~ N(0, I): w_i . x ~ N(0, ||w_i||^2)
        norms = act_vals.double().norm(dim=1)
        b_act = (norms * ppf).float()
    else:
        # inside a stack the inputs are not N(0, I) (the residual stream picks
        # up a common direction); take each pre-activation's mean and spread
        # over the inputs this layer actually receives, as a normal fit
        zfit = cal_inputs[0] @ act_vals.t()
        zd = zfit.double()
        b_act = (-zd.mean(dim=0) + zd.std(dim=0) * ppf).float()
        del zd

    # predictor first layer
    w1, w1v = _pred_store(torch.randn(r, d, generator=_gen(dev, seed, layer, TAG_W1), device=dev)
                          * d ** -0.5, cfg.p_dtype)
    b1 = torch.zeros(r, device=dev)

    # second layer fitted on calibration tokens
    if cal_inputs is None:
        xc = torch.randn(n_cal, d, generator=_gen(dev, seed, layer, TAG_CAL), device=dev)
    else:
        xc = cal_inputs[0]
    hcal = torch.relu(xc @ w1v.t() + b1)
    zcal = (xc @ act_vals.t() if zfit is None else zfit) + b_act
    del xc, zfit
    ha = torch.cat([hcal, torch.ones(n_cal, 1, device=dev)], dim=1).double()
    A = ha.t() @ ha
    lam = 1e-3 * float(torch.trace(A[:r, :r])) / r
    A[:r, :r] += lam * torch.eye(r, device=dev, dtype=torch.float64)
    Ainv = torch.from_numpy(np.linalg.inv(A.cpu().numpy())).to(dev)
    sol = Ainv @ (ha.t() @ zcal.double())          # [r+1, F]
    del zcal
    w2, w2v = _pred_store(sol[:r].t().float().contiguous(), cfg.p_dtype)
    b2 = sol[r].float()
    # the per-neuron shift is taken on held-out tokens: the fit's own tokens have
    # less residual variance than new ones, which would bias every rate upward
    del hcal
    if cal_inputs is None:
        xq = torch.randn(n_cal, d, generator=_gen(dev, seed, layer, TAG_SHIFT), device=dev)
    else:
        xq = cal_inputs[1]
    hq = torch.relu(xq @ w1v.t() + b1)
    del xq
    lcal = hq @ w2v.t() + b2                         # [n_cal, F]
    del hq
    srt = torch.sort(lcal, dim=0, descending=True).values
    del lcal
    k = torch.from_numpy(np.clip(np.rint(p * n_cal), 0, n_cal).astype(np.int64)).to(dev)
    cols = torch.arange(F, device=dev)
    top = srt[0]
    upper = srt[(k - 1).clamp(min=0), cols]
    lower = srt[k.clamp(max=n_cal - 1), cols]
    q = torch.where(k == 0, top, torch.where(k == n_cal, srt[n_cal - 1] - 1.0,
                                                0.5 * (upper + lower)))
    b2 = (b2 - q).float()
    del srt

    out = dict(kind=cfg.kind, w_dtype=cfg.w_dtype, p_dtype=cfg.p_dtype, d=d, d_ffn=F, r=r,
               tau=cfg.tau, w_gate=w_gate, w_up=w_up, w_down_t=w_down_t,
               b_act=b_act.contiguous(), p_w1=w1.contiguous(), p_b1=b1.contiguous(),
               p_w2=w2.contiguous(), p_b2=b2.contiguous(), p_fire=p)
    if return_values:
        out["act_values"] = act_vals
        out["up_values"] = up_vals
        out["down_values"] = down_vals
        out["p_w1_values"] = w1v
        out["p_w2_values"] = w2v
    return out


def _rms(h, eps=1e-5):
    return h * torch.rsqrt((h * h).mean(dim=1, keepdim=True) + eps)


def _carry(w, n):
    """What a layer adds to the residual stream of calibration inputs n
    [N, d]: its FFN over the neurons its own predictor selects (fp32; the
    generator's propagation only, never an expected value)."""
    z = n @ w["act_values"].t() + w["b_act"]
    a = torch.nn.functional.silu(z) if w["kind"] == "swiglu" else torch.relu(z)
    del z
    if w["kind"] != "relu":
        a = a * (n @ w["up_values"].t())
    hid = torch.relu(n @ w["p_w1_values"].t() + w["p_b1"])
    logit = hid @ w["p_w2_values"].t() + w["p_b2"]
    del hid
    t = math.log(w["tau"] / (1.0 - w["tau"]))
    a = torch.where(logit > t, a, torch.zeros((), device=a.device))
    del logit
    return a @ w["down_values"]


def make_stack(cfg: Config, seed: int = 0, device="cpu", n_cal: int = 4096, n_layers=None):
    """Layers 0 .. n_layers-1 of `cfg`, yielded in order, each calibrated on
    the inputs it receives in the stack: two sets of n_cal calibration tokens
    (x ~ N(0, I), the same draws the first layer calibrates on) are carried
    through every layer before it -- gainless RMS norm, the layer's FFN over
    its predicted neurons, residual add -- and their normalised values are that
    layer's calibration inputs.  The first layer is make_layer(cfg, 0)."""
    dev = torch.device(device)
    n_layers = cfg.layers if n_layers is None else n_layers
    hs = [torch.randn(n_cal, cfg.d, generator=_gen(dev, seed, 0, tag), device=dev)
          for tag in (TAG_CAL, TAG_SHIFT)]
    for l in range(n_layers):
        ns = [_rms(h) for h in hs]
        w = make_layer(cfg, l, seed=seed, device=dev, n_cal=n_cal, return_values=True,
                       cal_inputs=None if l == 0 else ns)
        if l + 1 < n_layers:
            for h, n in zip(hs, ns):
                h += _carry(w, n)
        del ns
        for k in ("act_values", "up_values", "down_values", "p_w1_values", "p_w2_values"):
            w.pop(k)
        yield w


def make_tokens(d: int, T: int, B: int, seed: int = 0, device="cpu", tag: int = TAG_TOKENS):
    """Decode inputs x ~ N(0, I): [T, B, d] fp32 (one fresh batch per step)."""
    dev = torch.device(device)
    return torch.randn(T, B, d, generator=_gen(dev, seed, -1, tag), device=dev)


def make_profile_tokens(d: int, N: int, seed: int = 0, device="cpu"):
    """Calibration tokens for the hot-first activation profile: [N, d] fp32."""
    return make_tokens(d, N, 1, seed, device, tag=TAG_PROFILE)[:, 0, :].contiguous()


def layer_to_numpy(layer):
    """The layer dict with every tensor moved to host numpy (for the oracle)."""
    out = {}
    for k, v in layer.items():
        if isinstance(v, torch.Tensor):
            out[k] = v.detach().cpu().numpy()
        else:
            out[k] = v
    return out
