"""CPU oracle for paged decode attention -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  It shares no code with the HIP path
and imports nothing from it.
"""
from .paged_attention import (  # noqa: F401
    attention,
    gather_kv,
    gather_sequence,
    gather_sequence_fast,
    key_vector,
    kv_head_of,
    lse_merge,
    num_partitions,
    online_block_attention,
    paged_decode,
    paged_prefill,
    partition_partials,
    poison_unused,
    reshape_and_cache,
    used_fill,
    value_vector,
)
from .block_manager import BlockManager, BlockManagerError, copy_blocks  # noqa: F401
from . import fp8  # noqa: F401
