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
from gpu_harness import GpuBatch, assert_close, merge_blocks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bench_like_run(inp, mean_hint=True):
    """The call bench.py times (kvd_decode_attn_paged), with its dims (automatic partitioning
    and runs)."""
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
    kvd.decode_attn_paged(*args)
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
                                  "mqa-t4", "mqa-t8", "s-t4", "s-t3", "b6-fp8", "b6-bf16", "b6-t4",
                                  "b1-fp8", "b1-t4", "b64-fp8"])
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
    window's first partition.  FP8 on MI355X: runs of 2048 +- 64 tokens, and since the grid is
    two workgroups per CU, the block pair dispatched first has runs 64 tokens longer and the
    other pair 64 shorter: blocks of 8192, 7680, 8704 and 8192 tokens, ends at 8192, 15872,
    24576 and 32768 (lengths 8448, 16384 and 24832 were ends of the layout without the early
    pair's extra tokens).  With 2 queries per sequence (16 rows per KV head, one tile) the chunk
    path takes the same runs, for BF16 too.  Every sequence's first and last KV head is checked
    against the oracle."""
    lengths = [32768, 8192, 8193, 15873, 24577, 1000, 30000, 20000, 32767, 24576, 15872, 8448,
               16384, 31000, 24832, 32768]
    windows = [0, 0, 0, 0, 0, 0, 5000, 12000, 0, 0, 0, 0, 0, 4096, 0, 1]
    inp = kvgen.make_inputs(kvgen.spec("c4", fmt=fmt, queries_per_seq=nq), lengths=lengths,
                            windows=windows, poison_before_window=True)
    gpu = _bench_like_run(inp, mean_hint=False)
    assert np.isfinite(gpu).all()
    pairs = [(b, hk) for b in range(len(lengths)) for hk in (0, inp.spec.num_kv_heads - 1)]
    _check(inp, gpu, pairs, f"{fmt} nq={nq} skewed runs")


def _header_block_starts(T, s, a, W, Y):
    """Token starts of the workgroup blocks of a full sequence in the skewed automatic run
    layout kvd_decode_partitions documents -- W runs of T + s tokens in even workgroups and of
    T - s in odd ones; with an early skew a > 0, Y (even) workgroup pairs of which pairs
    y >= Y/2 take runs a longer and the others a shorter -- followed by the last block's end."""
    st = []
    for y in range(Y):
        p = 2 * W * y * (T - a) if y <= Y // 2 else W * Y * (T - a) + 2 * W * (y - Y // 2) * (T + a)
        st += [p, p + W * (T + s + (a if y >= Y // 2 else -a))]
    return st + [st[-1] + W * (T - s + (a if Y - 1 >= Y // 2 else -a))]


@pytest.mark.parametrize("fmt,layout", [("fp8", (2048, 64, 64, 2)), ("bf16", (4096, 288, 0, 1))])
def test_skewed_partials_follow_header_layout(fmt, layout):
    """Phase 1 alone on the 16 x 32K batch shape (64 query / 8 KV heads) with the automatic run
    choice: each workgroup's triple in the workspace holds exactly the keys of the token range
    the documented skewed layout gives that workgroup.  On MI355X (256 CUs) FP8 takes runs of
    2048 +- 64 tokens in a grid of two workgroups per CU, the pair dispatched first 64 tokens
    longer per run (blocks start at 0, 8192, 15872, 24576); BF16 takes the one-workgroup-per-CU
    layout with runs of 4096 +- 288 (blocks at 0 and 17536, inside a partition).  The oracle's
    triples over 32-token ranges are merged per block; the slots past the last block stay
    unwritten."""
    import torch
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the run choice asserted here is the one for 256 CUs")
    T, s, a, Y = layout
    starts = _header_block_starts(T, s, a, 4, Y)
    assert starts[-1] == 32768
    inp = kvgen.make_inputs(kvgen.spec("c4", fmt=fmt))
    assert (inp.window == 0).all() and (inp.context_lens == 32768).all()
    gb = GpuBatch(inp)
    gb.run_phase1()
    m, l, o = gb.partials()
    g = inp.spec.group
    for b, hk in _pairs(inp, 2, 2, 5):
        rows = slice(hk * g, hk * g + g)
        blocks = merge_blocks(oracle.partition_partials(*oracle_args(inp), 32, b, hk), starts)
        assert [x for x, *_ in blocks] == list(range(len(starts) - 1))
        for x, lo, hi, pm, pl, po in blocks:
            m_nat = m[b, rows, x].astype(np.float64) * np.log(2.0)
            assert (np.abs(m_nat - pm) <= 1e-4).all(), (x, np.abs(m_nat - pm))
            lse = m_nat + np.log(l[b, rows, x].astype(np.float64))
            assert (np.abs(lse - (pm + np.log(pl))) <= 3e-4).all(), (x, lse, pm + np.log(pl))
            assert_close(o[b, rows, x].astype(np.float64), po, f"{fmt} block {x} b{b} h{hk}")
        assert np.isnan(m[b, rows, len(starts) - 1:]).all()
    del gb
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt,L", [("fp8", 1 << 20), ("turbo4", 1 << 18), ("bf16", 3 * (1 << 17) + 5)])
def test_very_long_context(fmt, L):
    """One sequence far longer than the configs: 512 to 2048 partitions, i.e. up to 32 blocks of
    64 partitions in the reduce, and a ragged last page -- against the oracle on every row."""
    inp = kvgen.make_inputs(kvgen.spec("c4", fmt=fmt, num_seqs=1, num_q_heads=8, num_kv_heads=1,
                                       context=L))
    gpu = _bench_like_run(inp)
    assert_close(gpu, oracle.decode_attention(*oracle_args(inp)), f"{fmt} L={L}")
