"""Seeded random sweep of the decode parameters against the oracle (GPU): format, query group
and KV head counts, head dim, ragged lengths, windows, softcap, ALiBi, partition size, partitions
per wave and chunks of queries are drawn together, so combinations the hand-written cases do not
name are covered too.  Same bar: max abs <= 2e-3, row-normwise relative <= 1e-2."""
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


def _draw(case):
    r = np.random.default_rng(np.random.SeedSequence([case, 0x5EED]))
    fmt = kvgen.FORMATS[r.integers(len(kvgen.FORMATS))]
    d = 128 if fmt.startswith("turbo") else int(r.choice([64, 128]))
    hkv = int(r.choice([1, 2, 3, 8]))
    g = int(r.choice([1, 2, 4, 5, 8, 16, 24]))
    nq = int(r.choice([1, 1, 1, 2, 3, 8]))
    B = int(r.integers(1, 6))
    hi = int(r.choice([40, 700, 2100, 5000]))
    lengths = r.integers(nq, hi + 1, size=B)
    lengths[r.integers(B)] = hi                       # one sequence at the maximum
    windows = np.where(r.random(B) < 0.4, r.integers(1, hi + 1, size=B), 0)
    spec = kvgen.spec("c1", fmt=fmt, head_dim=d, num_q_heads=g * hkv, num_kv_heads=hkv,
                      num_seqs=B, pool_total=None, queries_per_seq=nq, seed=case,
                      softcap=float(r.choice([0.0, 0.0, 20.0])),
                      softmax_scale=float(r.choice([d ** -0.5, 0.3])))
    inp = kvgen.make_inputs(spec, lengths=lengths, windows=windows,
                            poison_before_window=bool(r.integers(2)))
    ps = int(r.choice([0, 0, 16, 64, 128, 512, -1]))
    ppw = int(r.choice([0, 0, 1, 2, 3]))
    alibi = (2.0 ** (-r.uniform(0.5, 8.0, size=g * hkv))).astype(np.float32) if r.random() < 0.4 else None
    return inp, ps, ppw, alibi


@pytest.mark.parametrize("case", range(48))
def test_random_configuration(case):
    inp, ps, ppw, alibi = _draw(case)
    s = inp.spec
    fn = oracle.multi_query_attention if s.queries_per_seq > 1 else oracle.decode_attention
    ref = fn(*oracle_args(inp), alibi=alibi)
    gpu = GpuBatch(inp, partition_size=ps, partitions_per_wave=ppw, alibi=alibi).run()
    what = (f"case {case}: {s.fmt} D={s.head_dim} B={s.num_seqs} hq={s.num_q_heads} "
            f"hkv={s.num_kv_heads} nq={s.queries_per_seq} L={list(inp.context_lens)} "
            f"W={list(inp.window)} cap={s.softcap} ps={ps} ppw={ppw} alibi={alibi is not None}")
    assert_close(gpu, ref, what)


def _draw_single_query(case):
    """Single-query decode at head_dim 128 in the formats whose launch shapes differ most
    (BF16 picks between its one- and two-workgroup-per-CU layouts; FP8 and Turbo8 walk with one
    page pair in flight): automatic or explicit partitioning, contexts up to 12K."""
    r = np.random.default_rng(np.random.SeedSequence([case, 0xD128]))
    fmt = ["bf16", "fp8", "turbo8"][r.integers(3)]
    hkv = int(r.choice([1, 2, 4, 8]))
    g = int(r.choice([1, 4, 8, 16]))
    B = int(r.integers(1, 9))
    hi = int(r.choice([1500, 4100, 12000]))
    lengths = r.integers(1, hi + 1, size=B)
    lengths[r.integers(B)] = hi
    windows = np.where(r.random(B) < 0.3, r.integers(1, hi + 1, size=B), 0)
    spec = kvgen.spec("c1", fmt=fmt, head_dim=128, num_q_heads=g * hkv, num_kv_heads=hkv,
                      num_seqs=B, pool_total=None, seed=1000 + case,
                      softcap=float(r.choice([0.0, 0.0, 30.0])))
    inp = kvgen.make_inputs(spec, lengths=lengths, windows=windows,
                            poison_before_window=bool(r.integers(2)))
    ps = int(r.choice([0, 0, 0, 256, 512]))
    ppw = int(r.choice([0, 0, 0, 2, 4]))
    return inp, ps, ppw


@pytest.mark.parametrize("case", range(32))
def test_random_single_query_d128(case):
    inp, ps, ppw = _draw_single_query(case)
    s = inp.spec
    ref = oracle.decode_attention(*oracle_args(inp))
    gpu = GpuBatch(inp, partition_size=ps, partitions_per_wave=ppw).run()
    what = (f"single-query case {case}: {s.fmt} B={s.num_seqs} hq={s.num_q_heads} "
            f"hkv={s.num_kv_heads} L={list(inp.context_lens)} W={list(inp.window)} "
            f"cap={s.softcap} ps={ps} ppw={ppw}")
    assert_close(gpu, ref, what)
