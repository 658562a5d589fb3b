"""CPU oracle for paged decode attention and the paged KV write.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link or
execute anything under ``oracle/``; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table
or helper with the HIP library.

Everything is plain numpy in float64: the stored bfloat16 / float32 values are
widened exactly to float64 and every sum, max, exp and division is done there.
See ``oracle.paged_attention`` for the definitions and their citations.
"""
from .paged_attention import (  # noqa: F401
    widen,
    reshape_and_cache,
    copy_blocks,
    gather_kv,
    decode,
    decode_one,
    prefill,
    decode_partials,
    merge_partials,
)
