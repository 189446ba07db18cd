"""fp64 CPU oracle (test infrastructure only; see rankmixer_oracle)."""
from .rankmixer_oracle import *  # noqa: F401,F403
from .rankmixer_oracle import (as_f64, block_fwd, gelu, layer_norm, mean_pool, model_fwd,  # noqa: F401
                               moe_gates, moe_relu_pffn, pffn, round_to_bf16, run_config,
                               subset_inputs, token_mix, tokenize_padsplit, LN_EPS)
