"""fp64 CPU oracles of the ReLU linear-attention token mixer and the block-causal
temporal convolution beside it (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  It imports nothing from the HIP library and the library imports
nothing from it.
"""
from .linattn_oracle import (  # noqa: F401
    ROPE_BASE, phi, rope_axis_pairs, grid_positions, rope_angles, rope,
    state, apply, bidirectional_head, block_causal_head, weights_form_head,
    bidirectional, block_causal, rel_row_error,
    cross_attention_head, cross_attention, token_causal_head, token_causal,
)
from .temporal_conv_oracle import (  # noqa: F401
    temporal_conv_block, temporal_conv, temporal_conv_blocks,
)
