"""How sensitive the GPU parity gate is (CPU only, oracle arithmetic).

The GPU parity tests bound the row RMS-relative error ||gpu - oracle||_2 / ||oracle||_2 per
format (tests/gpu_harness.py, ROW_RMS_TOL).  Here the oracle itself shows that one key lost
from a 32K-token context -- the effect of a gathering or masking bug that skips one token --
moves the output rows far more than that bound, so such a bug cannot pass at full size.  The
key dropped is the one of median softmax weight (a typical key, not the largest).
"""
import numpy as np
import pytest

import kvgen
import oracle
from gpu_harness import ROW_RMS_TOL


def _row_rms_rel(a, b):
    return float((np.linalg.norm(a - b, axis=-1) / np.linalg.norm(b, axis=-1)).max())


@pytest.mark.parametrize("fmt,hq", [("fp8", 8), ("bf16", 8), ("turbo4", 4), ("turbo3", 4),
                                    ("turbo8", 4)])
def test_one_dropped_key_at_32k_exceeds_the_gate(fmt, hq):
    L = 32768
    inp = kvgen.make_inputs(kvgen.spec("c4", fmt=fmt, num_seqs=1, num_q_heads=hq,
                                       num_kv_heads=1, context=L, pool_spare=4))
    kw = dict(scales=inp.scales, codebook=inp.codebook, sign=inp.sign)
    k = oracle.gather_kv(fmt, "k", inp.k_cache, inp.block_table[0], 0, 0, L, 128, **kw)
    v = oracle.gather_kv(fmt, "v", inp.v_cache, inp.block_table[0], 0, 0, L, 128, **kw)
    q = oracle.bf16_to_f64(inp.q[0])
    _, _, full = oracle.attend(q, k, v, inp.softmax_scale, 0.0)
    z = float(np.float32(inp.softmax_scale)) * (q[0] @ k.T)
    for quartile in (1, 2, 3):
        j = int(np.argsort(z)[quartile * L // 4])
        keep = np.arange(L) != j
        _, _, dropped = oracle.attend(q, k[keep], v[keep], inp.softmax_scale, 0.0)
        moved = _row_rms_rel(dropped, full)
        # one typical key moves a row by a few 1e-3 of its norm (about 1 / sqrt(L))
        assert moved > 2 * ROW_RMS_TOL[fmt], (quartile, moved, ROW_RMS_TOL[fmt])
    # the same full result, computed blockwise as the oracle does beyond 64K keys, stays far
    # inside the gate
    blocked = oracle.decode_attention(*(inp.q, inp.k_cache, inp.v_cache, inp.block_table,
                                        inp.context_lens, fmt, inp.scales, inp.codebook, inp.sign,
                                        inp.softmax_scale, None, 0.0, 1, 128), chunk=4096)[0]
    assert _row_rms_rel(blocked, full) < 1e-12
