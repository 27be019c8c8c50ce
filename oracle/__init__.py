"""CPU oracle of the block-sparse attention path: test infrastructure only.

Imported only by tests/, __graft_entry__.smoke() and the bench's CPU-baseline
leg.  It shares no code with the HIP library.
"""
from .spade_oracle import *  # noqa: F401,F403
from .spade_oracle import (  # noqa: F401
    Geometry, Selection, block_extents, block_tokens, token_block_ids, summarize, sics,
    default_scale, estimate, keep_count, select, window_blocks, attention, attention_block_row,
    attention_full, dense_attention, spade_attn, MODE_COUNT, MODE_RATIO, MODE_MASS, SUMMARIZERS,
    scheme_aggregate, choose_scheme, spade_attn_schemes,
)
