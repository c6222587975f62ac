"""CPU fp64 oracle for stabilised softmax attention (forward, backward, repeat counts).

TEST INFRASTRUCTURE: imported only by the test suite, the package smoke check and the
CPU-baseline leg of the benchmark.  It shares no code with the HIP library and never imports it.
"""
from .attention import (MODE_STANDARD, MODE_TIE_RULE, MODE_TIE_ANTICIPATE, bf16_round, fp16_round, e4m3_round,
                        fp8_p_hat_round, P_HAT_FP8_LOG2_SCALE, visible,
                        scaled_scores, row_max_and_repeats, stable_shift, forward, forward_rows,
                        backward, dq_rows, integer_repeat_counts,
                        probabilities,
                        exact_causal_pairs, visible_pairs, CAUSAL_NONE, CAUSAL_TOP_LEFT,
                        CAUSAL_BOTTOM_RIGHT, ForwardResult, BackwardResult)
from .tiled import tiled_forward, tiled_ones, fp8_v_block

__all__ = [
    "MODE_STANDARD", "MODE_TIE_RULE", "MODE_TIE_ANTICIPATE", "bf16_round", "fp16_round", "e4m3_round",
    "fp8_p_hat_round", "P_HAT_FP8_LOG2_SCALE", "fp8_v_block", "visible",
    "scaled_scores", "row_max_and_repeats", "stable_shift", "forward", "forward_rows",
    "backward", "dq_rows", "integer_repeat_counts",
    "probabilities", "exact_causal_pairs",
    "visible_pairs", "CAUSAL_NONE", "CAUSAL_TOP_LEFT", "CAUSAL_BOTTOM_RIGHT",
    "ForwardResult", "BackwardResult", "tiled_forward", "tiled_ones",
]
