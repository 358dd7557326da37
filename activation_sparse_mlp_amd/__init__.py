"""Neuron-sparse FFN on AMD Instinct MI355X (gfx950): Python binding of libspffn.

The C ABI (include/spffn.h) exposes the per-token hot path -- predictor,
threshold, mask compaction, row-gather up/gate GEMV with the activation,
column-gather down projection -- and a multi-layer decode step, all as
hand-written HIP kernels.  This package only marshals torch tensors into it.
"""
from ._lib import (DECODE_DENSE, F16, F32, MAX_BATCH, PERMUTED_KEYS, Q4_0, RELU, REGLU,  # noqa
                   SIGNATURES, DecodeGraph, Layer, Model, SpffnError, compact, decode_step, forward,
                   hot_first_order, hot_first_permute, load, permute_rows, predict, profile,
                   q4_0_repack, threshold, version, set_wait_limit, WAIT_LIMIT_DEFAULT,
                   stream_read, workspace_clear_status, workspace_status,
                   decode_step_noalloc, decode_step_adaptive, tau_threshold)

LIB_PATH = __import__("os").path.join(__import__("os").path.dirname(__file__), "libspffn.so")
