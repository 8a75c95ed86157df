"""SSA (Sparse Sparse Attention) dual-stream attention for MI355X (gfx950).

The computation lives in libssa.so (HIP kernels behind a C interface,
include/ssa.h); this package only binds it to torch tensors.
"""
from ._lib import (DUAL_ACTIVE_FULL, DUAL_ACTIVE_SPARSE, FULL_ONLY, SPARSE_ONLY,  # noqa: F401
                   SSAError)
from .ops import (kernel_names, ssa_attn_bwd, ssa_attn_fwd, ssa_attn_fwd_noalloc, ssa_cache_block_means, ssa_decode,  # noqa: F401
                  ssa_prefill, ssa_probe_atomic, ssa_probe_copy, ssa_probe_lds, ssa_probe_mfma, ssa_select_blocks, timing_enable, timing_query)
from .autograd import SSAFunction, SSAOutput, ssa_attention  # noqa: F401,E402
