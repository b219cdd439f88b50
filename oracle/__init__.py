"""fp64 CPU oracle for SANTA / S²ANTA decode attention.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP path (the package
``stochastic_sparse_attention_split_amd``) and never imports it; the product path never imports this.
"""

from .santa import (IID, STRAT, SYS, TERNARY_Q, MODE_NAMES, DecodeResult, bytes_touched, cdf, decode, dense,
                    estimate, inverse_cdf, round_to_bf16, round_to_f32, sample_points, scale, scores_exact,
                    scores_ternary, softmax, stratum_weights, ternary_query, var_trace_iid, var_trace_strat)
from . import philox
from . import prop
from . import flash
from . import group_bernoulli

MODES = {"iid": IID, "strat": STRAT, "sys": SYS}
