"""Oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Plain fp64 CPU definition of decode attention (``attention``), of multi-query (chunked-prefill)
attention over the same cache (``multiquery``), a 40-digit ``decimal`` brute force (``brute``)
and the cache writer that stores new tokens (``encode``).
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package; the GPU library never does, and the two share no code.
"""
from .attention import (  # noqa: F401
    E4M3FN_TABLE,
    alibi_bias,
    attend,
    attended_range,
    bf16_to_f64,
    decode_attention,
    dequant_gather,
    e4m3fn_value,
    gather_kv,
    gather_stored,
    lse_merge,
    partition_partials,
    partitions,
    sylvester_hadamard,
    unpack_le,
    unrotate,
)
from . import encode  # noqa: F401,E402
from .multiquery import multi_query_attention, multi_query_partials  # noqa: F401,E402
