"""GPU parity at the full workload sizes, in the launch configuration bench.py times (automatic
partitions and partitions-per-wave, phase 1 then phase 2), on sampled outputs: every output row
of a few seeded (sequence, KV head) pairs is compared with the oracle, which computes just those
pairs.  Same bar as the small cases: max abs <= 2e-3, row-normwise relative <= 1e-2.

The ragged configuration samples a windowed and an unwindowed sequence and its shortest and
longest ones; the others sample sequences and KV heads by a seeded draw.
"""
import numpy as np
import pytest

import kvgen
import oracle
from conftest import oracle_args
from gpu_harness import assert_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bench_like_run(inp, mean_hint=True):
    """The two calls bench.py times, with its dims (automatic partitioning and runs)."""
    import torch
    import quantized_kv_cache_split_amd as kvd
    from kvgen.torch_io import dims_kwargs, to_torch

    t = to_torch(inp, "cuda:0")
    dims = kvd.Dims(**dims_kwargs(inp, inp.spec.partition_size, 0, mean_hint=mean_hint))
    out = torch.full(tuple(inp.q.shape), float("nan"), dtype=torch.float32, device="cuda:0")
    nws = kvd.workspace_bytes(dims)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device="cuda:0") if nws else None
    args = (dims, t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["context_lens"],
            inp.spec.fmt, t["scales"], t["codebook"], t["sign_pattern"], float(inp.softmax_scale),
            t["window"], float(inp.softcap), out, ws)
    kvd.decode_partitions(*args)
    kvd.reduce_partitions(*args)
    torch.cuda.synchronize()
    res = out.double().cpu().numpy()
    del t, out, ws
    torch.cuda.empty_cache()
    return res


def _pairs(inp, n_seq, n_head, seed):
    s = inp.spec
    r = np.random.default_rng(seed)
    seqs = r.choice(s.num_seqs, size=min(n_seq, s.num_seqs), replace=False)
    heads = r.choice(s.num_kv_heads, size=min(n_head, s.num_kv_heads), replace=False)
    return [(int(b), int(h)) for b in seqs for h in heads]


def _check(inp, gpu, pairs, what):
    s = inp.spec
    g = s.group
    mq = s.queries_per_seq > 1
    fn = oracle.multi_query_attention if mq else oracle.decode_attention
    for b, hk in pairs:
        ref = fn(*oracle_args(inp), seqs=[b], kv_heads=[hk])
        rows = slice(hk * g, (hk + 1) * g)
        if mq:
            assert_close(gpu[b, :, rows], ref[b, :, rows], f"{what} seq {b} kv head {hk}")
        else:
            assert_close(gpu[b, rows], ref[b, rows], f"{what} seq {b} kv head {hk}")


@pytest.mark.parametrize("name", ["c4", "m-bf16", "m-t4", "m-t3", "m-t8", "c2", "c5-t4", "c5-t3",
                                  "c5-t8", "mq-fp8", "mq8-fp8", "mq-t4", "mq-t3", "mqa-fp8", "mqa-bf16",
                                  "mqa-t4", "mqa-t8"])
def test_full_size_sampled(name):
    inp = kvgen.make_inputs(kvgen.SPECS[name])
    gpu = _bench_like_run(inp)
    assert np.isfinite(gpu).all()
    _check(inp, gpu, _pairs(inp, 2, 2, seed=len(name)), name)


def test_full_size_ragged_window_cap():
    """The ragged batch: lengths U{1..32768}, window 4096 on half the sequences, cap 50."""
    inp = kvgen.make_inputs(kvgen.SPECS["c3"])
    gpu = _bench_like_run(inp)
    assert np.isfinite(gpu).all()
    L, W = inp.context_lens, inp.window
    win = np.flatnonzero(W > 0)
    nowin = np.flatnonzero(W == 0)
    picks = {int(win[np.argmax(L[win])]), int(nowin[np.argmax(L[nowin])]),
             int(np.argmin(L)), int(np.argsort(L)[len(L) // 2])}
    pairs = [(b, hk) for b in sorted(picks) for hk in (0, inp.spec.num_kv_heads - 1)]
    _check(inp, gpu, pairs, "c3")


@pytest.mark.parametrize("fmt,nq", [("fp8", 1), ("bf16", 1), ("fp8", 2), ("bf16", 2)])
def test_skewed_runs_ragged_without_hint(fmt, nq):
    """The FP8 / BF16 32K batch shape (16 sequences, 64 query / 8 KV heads) without a mean-length
    hint takes the uniform-batch run choice, whose runs alternate between longer (even run
    blocks) and shorter (odd) ones; here the sequences have unequal lengths and windows, so
    blocks end inside a sequence, exactly at its end, one token past it, and start from a
    window's first partition.  FP8 on MI355X: runs of 2048 +- 64 tokens, blocks of 8448 and
    7936 tokens, ends at 8448, 16384, 24832 and 32768.  With 2 queries per sequence (16 rows per
    KV head, one tile) the chunk path takes the same runs.  Every sequence's first and last KV
    head is checked against the oracle."""
    lengths = [32768, 8448, 8449, 16385, 24833, 1000, 30000, 20000, 32767, 24832, 16384, 9000,
               5000, 31000, 12000, 32768]
    windows = [0, 0, 0, 0, 0, 0, 5000, 12000, 0, 0, 0, 0, 0, 4096, 0, 1]
    inp = kvgen.make_inputs(kvgen.spec("c4", fmt=fmt, queries_per_seq=nq), lengths=lengths,
                            windows=windows, poison_before_window=True)
    gpu = _bench_like_run(inp, mean_hint=False)
    assert np.isfinite(gpu).all()
    pairs = [(b, hk) for b in range(len(lengths)) for hk in (0, inp.spec.num_kv_heads - 1)]
    _check(inp, gpu, pairs, f"{fmt} nq={nq} skewed runs")


@pytest.mark.parametrize("fmt,L", [("fp8", 1 << 20), ("turbo4", 1 << 18), ("bf16", 3 * (1 << 17) + 5)])
def test_very_long_context(fmt, L):
    """One sequence far longer than the configs: 512 to 2048 partitions, i.e. up to 32 blocks of
    64 partitions in the reduce, and a ragged last page -- against the oracle on every row."""
    inp = kvgen.make_inputs(kvgen.spec("c4", fmt=fmt, num_seqs=1, num_q_heads=8, num_kv_heads=1,
                                       context=L))
    gpu = _bench_like_run(inp)
    assert_close(gpu, oracle.decode_attention(*oracle_args(inp)), f"{fmt} L={L}")
