"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the
benchmark.  Inputs only: no predictor, compaction or FFN evaluation lives here
beyond what fitting the synthetic predictor's weights needs."""
from .configs import ALL, FALCON_40B, LLAMA2_7B, LLAMA2_70B, OPT_175B_Q4, TINY, Config  # noqa
from .gen import (firing_probs, layer_to_numpy, make_layer, make_profile_tokens,  # noqa
                  make_tokens, q4_0_pack, q4_0_values)
