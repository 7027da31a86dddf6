"""fp64 CPU oracle (test infrastructure only; see ssa_oracle)."""
from .ssa_oracle import (align_loss, block_score_matrix, dual_attention,
                         dual_attention_rows, forced_blocks, pool_blocks,
                         row_block_diag, select_blocks, select_row,
                         selected_mask, ssa_forward)
