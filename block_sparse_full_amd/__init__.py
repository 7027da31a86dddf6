"""SSA dual-stream block-sparse attention (forward and backward) for AMD MI355X (gfx950).

The computation lives in libssa.so (HIP kernels behind the C ABI declared in
include/ssa.h); `block_sparse_full_amd.ssa` is the thin ctypes binding.
"""
from .ssa import (SSA_BF16, SSA_F32, SSA_SELECT_GROUP, SSA_SELECT_PER_HEAD, SSA_SELECT_TOKEN,
                  Problem, SsaError,
                  align_loss, align_loss_noalloc, alloc_bwd_workspace, alloc_workspace,
                  attn_bwd, attn_fwd,
                  bwd_workspace_bytes, dual_attention, load_library, pool_blocks, problem_for,
                  select_blocks, set_attn_timing_events, workspace_bytes)
