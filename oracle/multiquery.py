"""Oracle: multi-query (chunked-prefill) attention over the paged KV cache -- TEST INFRASTRUCTURE
ONLY (same import rule as ``oracle/attention.py``; shares no code with the GPU library).

What it follows (page titles and sections of the source pages):
  * attention.rs README: the feature list's "Chunked Prefill", the "Features" line ("causal
    masking", paged block tables, sliding window, softcapping, GQA/MQA), the paged-attention
    bullet list ("ALiBi slopes") and the "KV Cache Formats" table, whose Kernels column lists a
    prefill kernel for every format (TQ4 / TQ3 for the Turbo formats): prefill reads the same
    paged, possibly compressed cache.

Reading taken where the pages are silent: a chunk of n_q query tokens per sequence occupies the
last n_q positions of its context (their K and V are already in the cache).  Query i of a
sequence with context length L sits at position p = L - n_q + i and sees exactly the keys its own
decode step would see, causally: [p + 1 - W, p] with a window W, else [0, p]; the cap and the
ALiBi term (slope * (j - p)) are those of that decode step.  So a chunk of n_q queries equals n_q
decode steps at context lengths L - n_q + 1, ..., L, which is how it is written below.  L = 0
gives zero rows; 0 < L < n_q has no reading (the query positions would be negative).
"""
from __future__ import annotations

import math

import numpy as np

from .attention import (_q_rows, alibi_bias, attend, decode_attention, gather_kv, partitions,
                        sylvester_hadamard)


def query_position(L: int, n_q: int, i: int) -> int:
    """Position of query i of a chunk of n_q in a context of L tokens."""
    return L - n_q + i


def row_range(L: int, n_q: int, i: int, W: int) -> tuple[int, int]:
    """Keys [lo, hi) query i attends to: causal up to its own position, windowed."""
    hi = query_position(L, n_q, i) + 1
    return (max(0, hi - W) if W > 0 else 0), hi


def multi_query_attention(q, k_cache, v_cache, block_table, context_lens, fmt, scales, codebook,
                          sign, softmax_scale, window, softcap, num_kv_heads, head_dim,
                          alibi=None, seqs=None, kv_heads=None):
    """out[b, i, h] for q bf16 bits [B, n_q, Hq, D]: query i is the decode query of the context
    prefix that ends at its own position (fp64 [B, n_q, Hq, D]; ``seqs`` / ``kv_heads`` restrict
    the work to a sample, other rows are NaN)."""
    q = np.asarray(q)
    B, n_q, Hq, D = q.shape
    L = np.asarray(context_lens).astype(np.int64)
    assert ((L == 0) | (L >= n_q)).all(), "context lengths must be 0 or >= the query count"
    out = np.full((B, n_q, Hq, D), np.nan)
    for i in range(n_q):
        ctx_i = np.where(L > 0, L - n_q + i + 1, 0)
        out[:, i] = decode_attention(q[:, i], k_cache, v_cache, block_table, ctx_i, fmt, scales,
                                     codebook, sign, softmax_scale, window, softcap,
                                     num_kv_heads, head_dim, seqs=seqs, kv_heads=kv_heads,
                                     alibi=alibi)
    return out


def multi_query_partials(q, k_cache, v_cache, block_table, context_lens, fmt, scales, codebook,
                         sign, softmax_scale, window, softcap, num_kv_heads, head_dim,
                         partition_size, b, hk, rotated=False, alibi=None):
    """Per-partition triples of one (sequence, KV head) for a chunk of queries.

    Partitions cover the keys any query of the chunk sees, [lo of query 0, L), by the split
    rule on that span.  Rows are (query i, head h of the group), i-major.  A row that sees no
    key of a partition has m = -inf, l = 0 and o = 0.  Returns a list of
    (lo, hi, m [n_q g], l [n_q g], o [n_q g, D]); o rotated for the codebook V formats when
    rotated=True (the GPU's partial buffers hold that).
    """
    q = np.asarray(q)
    _, n_q, Hq, D = q.shape
    g = Hq // num_kv_heads
    L = int(context_lens[b])
    W = 0 if window is None else int(window[b])
    res = []
    for lo, hi in partitions(L, W + n_q - 1 if W > 0 else 0, partition_size):
        m = np.full(n_q * g, -np.inf)
        l = np.zeros(n_q * g)
        o = np.zeros((n_q * g, D))
        for i in range(n_q):
            a, c = row_range(L, n_q, i, W)
            a, c = max(a, lo), min(c, hi)
            if c <= a:
                continue
            kk = gather_kv(fmt, "k", k_cache, block_table[b], hk, a, c, head_dim, scales=scales,
                           codebook=codebook, sign=sign)
            vv = gather_kv(fmt, "v", v_cache, block_table[b], hk, a, c, head_dim, scales=scales,
                           codebook=codebook, sign=sign)
            bias = None
            if alibi is not None:
                bias = alibi_bias(np.asarray(alibi)[hk * g: hk * g + g],
                                  query_position(L, n_q, i) + 1, a, c)
            rows = slice(i * g, i * g + g)
            m[rows], l[rows], o[rows] = attend(_q_rows(q[:, i], b, hk * g, g), kk, vv,
                                               softmax_scale, softcap, bias)
        if rotated and fmt.startswith("turbo"):
            h = sylvester_hadamard(D).astype(np.float64)
            o = ((o * np.asarray(sign, np.float64)) @ h.T) / math.sqrt(D)
        res.append((lo, hi, m, l, o))
    return res
