"""Plain CPU oracle for FFD decode attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use it;
the library's product path never does.
"""

from . import ffd_oracle  # noqa: F401
from .ffd_oracle import (  # noqa: F401
    attend,
    bf16_bits_to_f32,
    block_scores,
    decode,
    decode_multi,
    pack_int4,
    quantize_cache,
    quantize_keys,
    quantize_query,
    select_blocks,
    select_head,
    token_scores,
    unpack_int4,
)
