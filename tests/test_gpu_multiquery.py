"""GPU parity of multi-query (chunked-prefill) decode: a chunk of n_q queries per sequence at
its last positions, each attending causally (its own window and ALiBi position), through the
C ABI against the oracle (oracle/multiquery.py).  Same bar as single-query decode: max abs error
<= 2e-3 and row-normwise relative error <= 1e-2; bit-identity where the arithmetic is fixed."""
import numpy as np
import pytest

import kvgen
import oracle
from conftest import oracle_args
from gpu_harness import GpuBatch, assert_close, merge_runs, runs_per_triple

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _mq(fmt, n_q, **kw):
    base = dict(fmt=fmt, head_dim=128, num_q_heads=8, num_kv_heads=2, pool_total=None,
                queries_per_seq=n_q)
    base.update(kw)
    return kvgen.make_inputs(kvgen.spec("c1", **base))


def _oracle(inp, alibi=None):
    return oracle.multi_query_attention(*oracle_args(inp), alibi=alibi)


def _slopes(h, base=8.0):
    return (2.0 ** (-base * (np.arange(h) + 1) / h)).astype(np.float32)


@pytest.mark.parametrize("fmt", kvgen.FORMATS)
@pytest.mark.parametrize("n_q,L", [(2, 2), (4, 17), (4, 300), (5, 1030), (16, 1500), (3, 4000)])
def test_multi_query_lengths(fmt, n_q, L):
    inp = _mq(fmt, n_q, context=L, num_seqs=2, seed=L + n_q)
    gpu = GpuBatch(inp).run()
    assert gpu.shape == inp.q.shape
    assert_close(gpu, _oracle(inp), f"{fmt} n_q={n_q} L={L}")


@pytest.mark.parametrize("fmt", kvgen.FORMATS)
@pytest.mark.parametrize("hq,hkv,n_q", [(4, 1, 4), (32, 8, 4), (8, 1, 8), (2, 2, 7), (64, 8, 3)])
def test_multi_query_groups(fmt, hq, hkv, n_q):
    """Rows per KV head n_q * g from 4 to 64 (one to four tiles of 16, ragged last tile)."""
    inp = _mq(fmt, n_q, num_q_heads=hq, num_kv_heads=hkv, context=None, ctx_range=(n_q, 2600),
              num_seqs=3)
    assert_close(GpuBatch(inp).run(), _oracle(inp), f"{fmt} hq={hq} hkv={hkv} n_q={n_q}")


@pytest.mark.parametrize("ps", [0, 128, -1, 32])
@pytest.mark.parametrize("fmt", kvgen.FORMATS)
def test_multi_query_window_alibi_cap(fmt, ps):
    """Ragged lengths, windows on half the sequences (each query its own window), ALiBi from
    each query's position, softcap (BF16), pages before the windows poisoned."""
    inp = kvgen.make_inputs(kvgen.spec("c3", fmt=fmt, num_seqs=6, num_q_heads=8, num_kv_heads=2,
                                       ctx_range=(16, 3000), window=700, queries_per_seq=6,
                                       softcap=50.0 if fmt == "bf16" else 0.0),
                            poison_before_window=True)
    sl = _slopes(8)
    gpu = GpuBatch(inp, partition_size=ps, alibi=sl).run()
    assert_close(gpu, _oracle(inp, sl), f"{fmt} mq window alibi ps={ps}")


@pytest.mark.parametrize("cap", [0.0, 30.0])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_multi_query_tile_pairs(fmt, D, cap):
    """Chunks with more than 16 rows per KV head run two query tiles per wave for BF16 / FP8
    (3 queries x 8 heads = 24 rows here): both head dims, with and without a softcap, ragged
    lengths, windows on half the sequences (each query its own window), split and unsplit
    rows, with and without ALiBi."""
    inp = kvgen.make_inputs(kvgen.spec("c3", fmt=fmt, head_dim=D, num_seqs=4, num_q_heads=16,
                                       num_kv_heads=2, ctx_range=(8, 3000), window=900,
                                       queries_per_seq=3, softcap=cap),
                            poison_before_window=True)
    for sl in (None, _slopes(16)):
        gpu = GpuBatch(inp, alibi=sl).run()
        assert_close(gpu, _oracle(inp, sl), f"{fmt} D={D} cap={cap} mq tile pairs alibi={sl is not None}")


@pytest.mark.parametrize("fmt,hq", [("bf16", 8), ("fp8", 8), ("turbo4", 8), ("turbo8", 8),
                                    ("bf16", 16), ("fp8", 16)])
def test_multi_query_runs_agree(fmt, hq):
    """Partitions per wave change the launch and the grouping of the sums (one triple per
    workgroup and query row), not the result.  With 16 query heads on 2 KV heads the 4 x 8
    rows of a KV head are two tiles, which BF16 / FP8 compute in one wave."""
    lengths, windows = [5000, 1100, 2600, 40], [1100, 0, 333, 0]
    inp = kvgen.make_inputs(kvgen.spec("c3", fmt=fmt, num_seqs=4, num_q_heads=hq, num_kv_heads=2,
                                       softcap=0.0, queries_per_seq=4),
                            lengths=lengths, windows=windows, poison_before_window=True)
    ref = _oracle(inp)
    outs = {}
    for run in (1, 2, 3):
        outs[run] = GpuBatch(inp, partition_size=128, partitions_per_wave=run).run()
        assert_close(outs[run], ref, f"{fmt} mq run={run}")
    tol = 1e-5 if fmt in ("bf16", "fp8") else 5e-4
    for run in (2, 3):
        assert np.abs(outs[run] - outs[1]).max() <= tol, run


@pytest.mark.parametrize("fmt", ["bf16", "turbo4"])
def test_multi_query_partials(fmt):
    """Workspace triples per (query, head) row, including rows that see no key of a triple:
    m = -inf, l = 0, o = 0 there."""
    # lengths 32k + 3 and 32k + 4: the last 32-token partition holds only the chunk's last 3 / 4
    # tokens, which its first queries do not see.  One-partition runs, and a workgroup of W
    # runs gives one triple, so the window makes the attended range W + 1 partitions long: the
    # last triple then holds that last partition alone.
    W = runs_per_triple(fmt)
    win = {4: 100, 8: 230}[W]
    inp = kvgen.make_inputs(kvgen.spec("c1", fmt=fmt, head_dim=128, num_q_heads=8, num_kv_heads=2,
                                       pool_total=None, queries_per_seq=8, num_seqs=2),
                            lengths=[355, 612], windows=[win, win])
    for L in (355, 612):   # first attended partition .. last: W + 1 of them
        assert (L - 1) // 32 - (L - 8 + 1 - win) // 32 == W
    gb = GpuBatch(inp, partition_size=32, partitions_per_wave=1)
    gb.run_phase1()
    m, l, o = gb.partials()          # [B, n_q, Hq, P]
    s = inp.spec
    g = s.group
    empty = 0
    for b in range(s.num_seqs):
        for hk in range(s.num_kv_heads):
            parts = merge_runs(oracle.multi_query_partials(*oracle_args(inp), 32, b, hk,
                                                           rotated=True), 32, runs_per_triple(fmt))
            for p, lo_, hi_, pm, pl, po in parts:
                gm = m[b, :, hk * g:(hk + 1) * g, p].reshape(-1).astype(np.float64)
                gl = l[b, :, hk * g:(hk + 1) * g, p].reshape(-1).astype(np.float64)
                go = o[b, :, hk * g:(hk + 1) * g, p].reshape(-1, s.head_dim).astype(np.float64)
                none = pl == 0
                empty += int(none.sum())
                assert (np.isneginf(gm[none])).all() and (gl[none] == 0).all() and (go[none] == 0).all()
                lse = gm[~none] * np.log(2.0) + np.log(gl[~none])
                assert np.abs(lse - (pm[~none] + np.log(pl[~none]))).max() < 5e-3
                assert_close(go[~none], po[~none], f"{fmt} mq partial b{b} p{p}")
    assert empty > 0


def test_multi_query_zero_and_short_rows():
    """L = 0: zero rows; 0 < L < n_q: NaN rows (no position exists for the first queries); the
    sequence next to them matches the oracle."""
    inp = _mq("fp8", 4, num_seqs=3, context=None, ctx_range=(4, 50))
    inp.context_lens[:] = [0, 3, 50]
    gpu = GpuBatch(inp).run()
    assert (gpu[0] == 0).all()
    assert np.isnan(gpu[1]).all()
    ok = inp.context_lens.copy()
    ok[1] = 4                      # the oracle's domain; sequences are independent
    import dataclasses
    ref = oracle.multi_query_attention(*oracle_args(dataclasses.replace(inp, context_lens=ok)),
                                       seqs=[2])
    assert_close(gpu[2:3], ref[2:3], "fp8 mq next to short rows")


def test_one_query_chunk_equals_decode_bits():
    """queries_per_seq = 1 runs the single-query kernels: bit-identical to leaving it 0."""
    inp = _mq("turbo4", 1, context=None, ctx_range=(1, 3000), num_seqs=3)
    a = GpuBatch(inp).run()
    gb = GpuBatch(inp)
    gb.dims.queries_per_seq = 0
    b = gb.run()
    assert (a.view(np.uint64) == b.view(np.uint64)).all()


@pytest.mark.parametrize("fmt", kvgen.FORMATS)
def test_chunked_prefill_step(fmt):
    """One chunked-prefill step end to end: append a chunk of 24 tokens per sequence to the cache
    (kvd_append_kv), then attend with those 24 queries (queries_per_seq = 24) -- against the
    oracle's cache writer followed by its multi-query attention."""
    import dataclasses
    import torch
    import quantized_kv_cache_split_amd as kvd
    from kvgen.torch_io import dims_kwargs, to_torch
    from oracle import encode as enc

    n_q, old = 24, [40, 1100, 7]
    s = kvgen.spec("c1", fmt=fmt, head_dim=128, num_q_heads=8, num_kv_heads=2, pool_total=None,
                   num_seqs=3, queries_per_seq=n_q, seed=21)
    inp = kvgen.make_inputs(s, lengths=[L + n_q for L in old])
    rng = np.random.default_rng(22)
    kn = rng.standard_normal((3, n_q, 2, 128)).astype(np.float32)
    vn = rng.standard_normal((3, n_q, 2, 128)).astype(np.float32)
    pos = np.array(old, dtype=np.int32)
    t = to_torch(inp, "cuda:0")
    dims = kvd.Dims(**dims_kwargs(inp, 0))
    kvd.append_kv(dims, fmt, torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(),
                  t["block_table"], torch.from_numpy(pos).cuda(), n_q, t["k_cache"], t["v_cache"],
                  t["scales"], t["codebook"], t["sign_pattern"])
    out = torch.full(tuple(inp.q.shape), float("nan"), dtype=torch.float32, device="cuda:0")
    nws = kvd.workspace_bytes(dims)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device="cuda:0")
    kvd.decode_attn_paged(dims, t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                          t["context_lens"], fmt, t["scales"], t["codebook"], t["sign_pattern"],
                          float(inp.softmax_scale), t["window"], float(inp.softcap), out,
                          ws if nws else None)
    torch.cuda.synchronize()
    kc, vc, sc = enc.append_tokens(fmt, kn, vn, inp.block_table, pos, inp.k_cache, inp.v_cache,
                                   inp.scales, inp.codebook, inp.sign)
    ref = oracle.multi_query_attention(*oracle_args(dataclasses.replace(
        inp, k_cache=kc, v_cache=vc, scales=sc)))
    assert_close(out.double().cpu().numpy(), ref, f"{fmt} chunked prefill step")
