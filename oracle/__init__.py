"""fp64 CPU reference for pair-biased attention (test infrastructure only).

Imported by the test suite, the smoke check and the benchmark's CPU-baseline
leg.  The product library never imports or calls anything in this package.
"""
from .pairattn_oracle import *  # noqa: F401,F403
from .pairattn_oracle import (START, END, layer_norm, sigmoid, pair_bias, attention_bias,
                              masked_softmax_weights, gated_output, tri_start, tri_end,
                              tri_fwd, tri_points, tri_rows, tri_partial, tri_partial_finish,
                              msa_row, max_abs_err, mean_rel_err)
