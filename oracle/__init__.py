"""CPU oracle for the PSA path, forward and backward (test infrastructure only; see psa_oracle)."""
from .psa_oracle import *  # noqa: F401,F403
from .psa_oracle import (Problem, AssignParams, as_f64, pool, pyramid, pack_pyramid,
                         packed_level_offset, mask_scores_sampling, mask_scores_antidiag,
                         block_cossim, assign_row, assign_levels, build_index, attention_head,
                         attention, attention_backward_head, attention_backward, mask,
                         e4m3_round, bf16_round, fp8_scale, fp8_quantize, attention_fp8qk_head, attention_fp8_head, sample_offsets, kb_diag, SKIP, NUM_LEVELS)
