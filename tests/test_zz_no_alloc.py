"""The allocation-free entry point (kvd_decode_attn_paged_noalloc) against kvd_decode_attn_paged.

Both run the same kernels; the no-alloc call takes its partition workspace from the library's
static device array.  Two calls in a row, the second on a smaller batch (the array then still
holds the first call's triples beyond the second's), must each give the bits of the entry
point with a caller workspace, and match the oracle to the parity gate.
"""
import numpy as np
import pytest

import kvgen
import oracle
from conftest import oracle_args
from gpu_harness import GpuBatch, assert_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(inp, ps=0):
    import torch
    gb = GpuBatch(inp, partition_size=ps)
    ref = gb.run()
    args = gb._args()
    out = torch.full_like(gb.out, float("nan"))
    gb.kvd.decode_attn_paged_noalloc(*args[:13], out)
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), ref


@pytest.mark.parametrize("fmt", ["fp8", "bf16", "turbo4", "turbo8"])
def test_noalloc_matches_workspace_entry_point_twice(fmt):
    big = kvgen.make_inputs(kvgen.spec("c3", fmt=fmt, num_seqs=6, num_q_heads=16, num_kv_heads=2,
                                       ctx_range=(1, 9000), window=3000, softcap=0.0, seed=3))
    small = kvgen.make_inputs(kvgen.spec("c3", fmt=fmt, num_seqs=2, num_q_heads=8, num_kv_heads=2,
                                         ctx_range=(1100, 2600), window=0, softcap=0.0, seed=4))
    for what, inp, ps in (("large", big, 0), ("smaller", small, 128)):
        got, ref = _both(inp, ps)
        assert (got.view(np.uint64) == ref.view(np.uint64)).all(), what
        assert_close(got, oracle.decode_attention(*oracle_args(inp)), f"{fmt} no-alloc {what}")


def test_noalloc_too_large_is_refused():
    import torch
    import quantized_kv_cache_split_amd as kvd
    d = kvd.Dims(num_seqs=64, num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                 max_blocks_per_seq=8192, num_pool_blocks=1, max_context_len=131072,
                 partition_size=0)
    assert kvd.workspace_bytes(d) > kvd.NOALLOC_WORKSPACE_BYTES
    x = torch.zeros(16, device="cuda:0")
    with pytest.raises(kvd.KvdError) as e:
        kvd.decode_attn_paged_noalloc(d, x, x, x, x, x, "bf16", None, None, None, 0.1, None, 0.0, x)
    assert e.value.status == -5
