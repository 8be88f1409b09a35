"""GPU: the decode call captured in a HIP graph (torch.cuda.CUDAGraph, on the stream the binding
launches on) replays bit-identically to the eager call.

The partition and reduce launches need no memset and no host round trip, so a serving loop can
capture them.  Each graph is replayed three times with eager library calls on another batch and
synchronisations between the replays, and every replay is compared with the eager result, bit
for bit.  The allocation-free entry point is captured the same way after one eager call (its
first call on a device looks up the library's workspace array).
"""
import numpy as np
import pytest

import kvgen
from gpu_harness import GpuBatch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _batch(fmt, seed):
    # split and unsplit rows, windows on half of the sequences
    return kvgen.make_inputs(kvgen.spec("c3", fmt=fmt, num_seqs=5, num_q_heads=16,
                                        num_kv_heads=2, ctx_range=(1, 6000), window=1500,
                                        softcap=0.0, seed=seed))


def _replays_match(gb, capture, eager):
    import torch
    other = GpuBatch(_batch(gb.inp.spec.fmt, 99))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture()
    for i in range(3):
        gb.out.fill_(float("nan"))
        other.run()                      # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = gb.out.double().cpu().numpy()
        assert (got.view(np.uint64) == eager.view(np.uint64)).all(), i


@pytest.mark.parametrize("fmt", ["fp8", "bf16", "turbo4", "turbo8"])
def test_graph_replays_match_eager(fmt):
    gb = GpuBatch(_batch(fmt, 7))
    eager = gb.run()
    assert np.isfinite(eager).all()
    args = gb._args()
    _replays_match(gb, lambda: gb.kvd.decode_attn_paged(*args), eager)


@pytest.mark.parametrize("fmt", ["fp8", "turbo4"])
def test_graph_replays_noalloc_entry_point(fmt):
    import torch
    gb = GpuBatch(_batch(fmt, 11))
    eager = gb.run()
    args = gb._args()[:13] + (gb.out,)
    gb.out.fill_(float("nan"))
    gb.kvd.decode_attn_paged_noalloc(*args)      # first call on the device: outside the graph
    torch.cuda.synchronize()
    assert (gb.out.double().cpu().numpy().view(np.uint64) == eager.view(np.uint64)).all()
    _replays_match(gb, lambda: gb.kvd.decode_attn_paged_noalloc(*args), eager)
