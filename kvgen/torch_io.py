"""Move a generated batch into torch tensors (device memory plumbing; no arithmetic)."""
from __future__ import annotations

import numpy as np


def dims_kwargs(inp, partition_size: int | None = None, partitions_per_wave: int = 0,
                mean_hint: bool = True) -> dict:
    """Field values of the C ABI's kvd_dims for a batch (mean_hint: pass the batch's mean
    attended span, which the host knows, as the launch hint)."""
    s = inp.spec
    mean = int(round(float(inp.spans().mean()))) if mean_hint and s.num_seqs else 0
    return dict(num_seqs=s.num_seqs, num_q_heads=s.num_q_heads, num_kv_heads=s.num_kv_heads,
                head_dim=s.head_dim, block_size=16, max_blocks_per_seq=inp.max_blocks_per_seq,
                num_pool_blocks=inp.num_pool_blocks, max_context_len=inp.max_context_len,
                partition_size=s.partition_size if partition_size is None else partition_size,
                partitions_per_wave=partitions_per_wave, queries_per_seq=s.queries_per_seq,
                mean_context_len=mean)


def to_torch(inp, device) -> dict:
    """Tensors for every array argument of the decode call (None where unused)."""
    import torch

    def t(a, dtype=None):
        if a is None:
            return None
        x = torch.from_numpy(np.ascontiguousarray(a))
        if dtype is not None:
            x = x.view(dtype)
        return x.to(device)

    return dict(q=t(inp.q.view(np.int16), torch.bfloat16), k_cache=t(inp.k_cache),
                v_cache=t(inp.v_cache), block_table=t(inp.block_table),
                context_lens=t(inp.context_lens), scales=t(inp.scales), codebook=t(inp.codebook),
                sign_pattern=t(inp.sign), window=t(inp.window))
