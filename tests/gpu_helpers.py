"""Shared helpers of the GPU parity tests (marshalling only)."""
import numpy as np
import torch

import activation_sparse_mlp_amd as spffn
import oracle
from workloads import layer_to_numpy

DEV = torch.device("cuda:0")

# FFN output bound: relative L2 error against the oracle on identical masks
# and identically decoded weights (fp32 accumulation of fp16/4-bit rows).
REL_L2 = 1e-3
# predictor: a mask entry may differ from the oracle's only where the oracle's
# logit is this close to the threshold, and on at most this share of entries.
FLIP_BAND = 1e-3
MIN_AGREEMENT = 0.9999


def to_dev(w):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in w.items()}


def gpu_layer(w):
    return spffn.Layer(to_dev(w))


def np_layer(w):
    L = layer_to_numpy(w)
    L["t"] = oracle.logit_threshold(L["tau"])
    return L


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0.0:
        return 0.0 if np.all(got == 0) else float("inf")
    return float(np.linalg.norm(got - ref) / nr)


def check_mask_agreement(gpu_mask, ref_logits, t):
    """gpu_mask vs the oracle's fp64 logits: flips only inside the band."""
    gpu_mask = np.asarray(gpu_mask).astype(bool)
    ref_mask = np.asarray(ref_logits) > t
    flips = gpu_mask != ref_mask
    agree = 1.0 - flips.mean()
    assert agree >= MIN_AGREEMENT, f"mask agreement {agree}"
    assert np.all(np.abs(np.asarray(ref_logits)[flips] - t) < FLIP_BAND), \
        "mask flip outside the threshold band"
    return int(flips.sum())
