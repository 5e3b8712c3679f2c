"""CPU float64 oracle for decode-step attention over a paged KV cache,
(``oracle.kv_quant``) for appending to an fp8 cache with quantisation, and
(``oracle.block_manager``) for the block allocator with copy-on-write, and
(``oracle.mla``) for absorbed multi-head latent attention decode.

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``; never by the library.

Every function here is pinned by ``tests/test_oracle.py``; none is "parity
unpinned".
"""

from .paged_attention import (  # noqa: F401
    LN2,
    attend,
    decode_attention,
    decode_bf16,
    decode_e4m3fn,
    decode_partials,
    decode_step,
    gather_sequence,
    kv_append,
    kv_append_tokens,
    merge_partials,
    multi_query_attention,
    partition_partials,
    slot_of,
    to_float64,
    visible_tokens,
)
from .kv_quant import (  # noqa: F401
    SCALE_FIXED,
    SCALE_RUNNING_AMAX,
    encode_e4m3fn,
    kv_append_quant,
    quantize,
)
from .block_manager import BlockManager, OutOfBlocks, copy_blocks  # noqa: F401
from .mla import absorb_query, mla_decode_absorbed, mla_decode_expanded, project_out  # noqa: F401
