"""CPU oracle for SSA attention: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It shares no code with the HIP path and never imports it.
"""
from .ssa_oracle import *  # noqa: F401,F403
from .ssa_oracle import (DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE, FULL_ONLY, SPARSE_ONLY,
                         alignment_loss, attend_rows, backward, block_means, dkdv_tail,
                         dq_rows, forward, full_stats, select_blocks, select_rows, stats_rows,
                         stream_grads)
