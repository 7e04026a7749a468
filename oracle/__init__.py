"""CPU oracle for the packed text-embedding encoder (test infrastructure only).

Only tests, the smoke check and the bench's CPU-baseline leg may import this
package.  The HIP library never calls it, and it imports nothing from the HIP
side; both read the same seeded inputs.
"""
from .encoder import (  # noqa: F401
    attention,
    block_matmul_int8,
    block_matmul_q4,
    cosine_matrix,
    decode_matrix,
    encode,
    encode_layers,
    encode_tokens,
    encoder_layer,
    gelu,
    geglu,
    layer_norm,
    mean_pool_l2,
    positions,
    q4_block_params,
    q4_codes,
    quantize_rows_7bit,
    rope,
    rope_inverse_frequencies,
    text_index,
    validate_offsets,
)
