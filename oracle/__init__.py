"""CPU oracle of the AB-Attention hot path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It shares no code with the GPU library.
"""
from .abatt_oracle import *  # noqa: F401,F403
from .abatt_oracle import (Problem, Plan, attend, attend_row, dense, dense_rows,  # noqa: F401
                           ht_estimates, ibcs_scores, inclusion_probabilities,
                           key_block_means, kmeans, philox4x32_10, plan,
                           plan_from_scores, query_clusters, sample_row,
                           block_scores, block_words, unflatten_row)
