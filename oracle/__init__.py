"""fp64 CPU oracle of the SPLA decode step -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  See ``spla_oracle`` for the definitions, the
passages they follow and the readings taken where the pages are silent.
"""
from .spla_oracle import (  # noqa: F401
    RLA_NORMALIZED,
    RLA_PLAIN,
    RLA_RMSNORM,
    SCORE_MEAN,
    SCORE_TAYLOR,
    SplaOracle,
    block_stats,
    exact_block_log_mass,
    group_log_score,
    linear_attention_numerator,
    mean_pool_log_score,
    phi,
    rla_branch,
    select_blocks,
    softmax_attention,
    taylor_log_score,
)
