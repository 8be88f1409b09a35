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


def _replays_match(gb, capture, eager, before=None):
    import torch
    other = GpuBatch(_batch(gb.inp.spec.fmt, 99))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture()
    for i in range(3):
        gb.out.fill_(float("nan"))
        if before is not None:
            before()
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


@pytest.mark.parametrize("fmt", ["fp8", "bf16", "turbo4", "turbo8"])
def test_graph_replays_append_then_decode(fmt):
    """One serving step -- quantize each sequence's newest token into the paged cache, then
    decode over the cache -- captured as one graph.  Before every replay the caches are put
    back as they were before the eager step, so the replay's own append must write the token
    the decode then attends to; each replay matches the eager step bit for bit."""
    import torch
    from kvgen.torch_io import dims_kwargs
    inp = _batch(fmt, 13)
    gb = GpuBatch(inp)
    s = inp.spec
    rng = np.random.default_rng(17)
    kn = torch.from_numpy(rng.standard_normal((s.num_seqs, 1, s.num_kv_heads, s.head_dim))
                          .astype(np.float32)).to("cuda:0")
    vn = torch.from_numpy(rng.standard_normal((s.num_seqs, 1, s.num_kv_heads, s.head_dim))
                          .astype(np.float32)).to("cuda:0")
    assert (inp.context_lens >= 1).all()
    pos = torch.from_numpy((inp.context_lens - 1).astype(np.int32)).to("cuda:0")
    adims = gb.kvd.Dims(**dims_kwargs(inp, 0))
    t = gb.t
    args = gb._args()

    def step():
        gb.kvd.append_kv(adims, fmt, kn, vn, t["block_table"], pos, 1, t["k_cache"],
                         t["v_cache"], t["scales"], t["codebook"], t["sign_pattern"])
        gb.kvd.decode_attn_paged(*args)

    k0, v0 = t["k_cache"].clone(), t["v_cache"].clone()
    before_step = gb.run()
    step()
    torch.cuda.synchronize()
    eager = gb.out.double().cpu().numpy()
    assert np.isfinite(eager).all()
    assert not np.array_equal(eager, before_step)      # the appended token changes the output

    def restore():
        t["k_cache"].copy_(k0)
        t["v_cache"].copy_(v0)

    _replays_match(gb, step, eager, before=restore)
