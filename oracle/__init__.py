"""fp64 CPU oracle for block-sparse attention.

TEST INFRASTRUCTURE: only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package. It shares no code with
the GPU path, which never calls it.
"""
from .sparge_oracle import *  # noqa: F401,F403
from .sparge_oracle import (Q_BLOCK, K_BLOCK, num_blocks, default_scale, topk_count, pool_blocks,  # noqa: F401
                            block_logits, row_softmax, select_topk, predict_mask, selected_keys,
                            attend_rows, masked_attention, masked_attention_rows, compact_mask,
                            mask_parity)
