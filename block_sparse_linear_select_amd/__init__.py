"""MI355X (gfx950) block-sparse + rotary low-rank linear hybrid attention.

The computation lives in libhsa_attn.so (hand-written HIP kernels behind a C
ABI, declared in include/hsa_attn.h); this package is its thin Python binding.
"""
from .binding import (Config, HsaError, HybridPlan, block_select, hybrid_attn, linear_attn,  # noqa: F401
                      sparse_attn, version, workspace_size)
