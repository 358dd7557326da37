"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the
benchmark.  Inputs only: no predictor, compaction or FFN evaluation lives here
beyond what constructing the weights needs (fitting the synthetic predictor,
and carrying calibration tokens through a stack so that every layer is
calibrated on the inputs it receives); nothing here is ever an expected
value."""
from .configs import (ALL, FALCON_40B, LLAMA2_7B, LLAMA2_7B_SWIGLU, LLAMA2_70B,  # noqa
                      LLAMA2_70B_FP8P, LLAMA2_70B_PREFIX, OPT_175B_Q4, TINY, Config)
from .gen import (firing_probs, fp8_pack, layer_to_numpy, make_layer,  # noqa
                  make_profile_tokens, make_stack, make_tokens, q4_0_pack, q4_0_values)
