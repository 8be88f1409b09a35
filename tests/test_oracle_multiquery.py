"""Pins of the multi-query (chunked-prefill) oracle, CPU only: the 40-digit brute force with
explicit causal bounds, the reduction to decode for one query, a closed form, causality (keys
after a query's position never change its row), the partition triples merging to the full
result (rows without keys in a partition included), and planted mistakes."""
import numpy as np
import pytest

import kvgen
import oracle
import oracle.multiquery as omq
from oracle.brute import brute_multi_query
from conftest import brute_as_array, oracle_args


def _mq(fmt, n_q, **kw):
    base = dict(fmt=fmt, head_dim=64 if fmt in ("bf16", "fp8") else 128, queries_per_seq=n_q)
    base.update(kw)
    return kvgen.make_inputs(kvgen.spec("c1", **base))


def _brute(inp, alibi=None):
    rows = brute_multi_query(*oracle_args(inp), alibi=alibi)
    return np.array([[[[float(x) for x in r] for r in h] for h in s] for s in rows])


@pytest.mark.parametrize("fmt", kvgen.FORMATS)
def test_brute_multi_query(fmt):
    inp = _mq(fmt, 3, num_seqs=2, num_q_heads=4, num_kv_heads=2, context=None, ctx_range=(3, 21),
              window=5, window_frac=0.5, softcap=2.0 if fmt == "bf16" else 0.0)
    assert inp.q.shape == (2, 3, 4, inp.spec.head_dim)
    sl = (2.0 ** (-np.arange(1, 5))).astype(np.float32) if fmt != "fp8" else None
    o = oracle.multi_query_attention(*oracle_args(inp), alibi=sl)
    assert np.isfinite(o).all()
    assert np.abs(o - _brute(inp, sl)).max() <= 1e-12


def test_one_query_is_decode():
    inp = _mq("bf16", 1, num_seqs=3, context=None, ctx_range=(1, 300), window=40, window_frac=0.67)
    q4 = inp.q[:, None]
    a = oracle.multi_query_attention(q4, *oracle_args(inp)[1:])[:, 0]
    b = oracle.decode_attention(*oracle_args(inp))
    assert np.array_equal(a, b)


def _count_bit_set(a, b, d):
    def f(n):
        period = 1 << (d + 1)
        return (n // period) * (1 << d) + max(0, n % period - (1 << d))
    return f(b) - f(a)


@pytest.mark.parametrize("L,W,n_q", [(300, 0, 4), (300, 37, 7), (40, 5, 16), (16, 0, 16), (1100, 513, 3)])
def test_position_coded_v_closed_form(L, W, n_q):
    """K = 0 and V[j][d] = bit d of j: query i averages the bits over its own causal window."""
    D = 64

    def kv(seq, n):
        j = np.arange(n)
        v = ((j[None, :, None] >> np.arange(D)[None, None, :]) & 1).astype(np.float32)
        return np.zeros((1, n, D), np.float32), v

    inp = kvgen.make_inputs(kvgen.spec("c1", pool_total=None, queries_per_seq=n_q), lengths=[L],
                            windows=[W], kv_override=kv)
    o = oracle.multi_query_attention(*oracle_args(inp))[0]
    for i in range(n_q):
        pos = L - n_q + i
        lo = max(0, pos + 1 - W) if W else 0
        want = np.array([_count_bit_set(lo, pos + 1, d) for d in range(D)]) / (pos + 1 - lo)
        assert np.abs(o[i] - want[None, :]).max() < 1e-15, i


def test_causality_later_keys_do_not_matter():
    """Changing the K and V of the chunk's last tokens leaves the earlier queries' rows exactly
    as they were and changes the last query's row."""
    D = 64
    rng = np.random.default_rng(5)
    base = rng.standard_normal((2, 1, 60, D)).astype(np.float32)

    def kv_a(seq, n):
        return base[0, :, :n], base[1, :, :n]

    def kv_b(seq, n):
        k, v = base[0, :, :n].copy(), base[1, :, :n].copy()
        k[:, -2:] += 3.0
        v[:, -2:] -= 5.0
        return k, v

    sp = kvgen.spec("c1", pool_total=None, queries_per_seq=6)
    a = oracle.multi_query_attention(*oracle_args(kvgen.make_inputs(sp, lengths=[60], kv_override=kv_a)))
    b = oracle.multi_query_attention(*oracle_args(kvgen.make_inputs(sp, lengths=[60], kv_override=kv_b)))
    assert np.array_equal(a[0, :4], b[0, :4])
    assert np.abs(a[0, 4:] - b[0, 4:]).min(axis=-1).max() > 1e-3


@pytest.mark.parametrize("ps,W", [(16, 20), (32, 0), (0, 0), (128, 300)])
def test_partials_merge_to_full(ps, W):
    inp = _mq("bf16", 8, num_q_heads=4, num_kv_heads=2, context=None, ctx_range=(40, 1500),
              num_seqs=2, window=W, window_frac=1.0 if W else 0.0, pool_total=None)
    full = oracle.multi_query_attention(*oracle_args(inp))
    empty_rows = 0
    for b in range(2):
        for hk in range(2):
            parts = oracle.multi_query_partials(*oracle_args(inp), ps, b, hk)
            empty_rows += sum(int((p[3] == 0).sum()) for p in parts)
            for _, _, m, l, o in parts:
                assert (np.isinf(m) == (l == 0)).all() and (o[l == 0] == 0).all()
            merged = oracle.lse_merge([p[2] for p in parts], [p[3] for p in parts],
                                      [p[4] for p in parts])
            want = full[b, :, hk * 2: hk * 2 + 2].reshape(16, -1)
            assert np.abs(merged - want).max() < 1e-13
    if ps == 16 and W:
        assert empty_rows > 0     # some queries see no key of some partition


def test_planted_future_leak(monkeypatch):
    """Every query attending to the whole context (no causal bound) breaks the closed form."""
    monkeypatch.setattr(omq, "decode_attention",
                        lambda q, *a, **k: oracle.decode_attention(q, *a[:3], _L_full[0], *a[4:], **k))
    D, L, n_q = 64, 300, 4

    def kv(seq, n):
        j = np.arange(n)
        return (np.zeros((1, n, D), np.float32),
                ((j[None, :, None] >> np.arange(D)[None, None, :]) & 1).astype(np.float32))

    inp = kvgen.make_inputs(kvgen.spec("c1", pool_total=None, queries_per_seq=n_q), lengths=[L],
                            kv_override=kv)
    _L_full[0] = inp.context_lens
    o = oracle.multi_query_attention(*oracle_args(inp))[0]
    want0 = np.array([_count_bit_set(0, L - n_q + 1, d) for d in range(D)]) / (L - n_q + 1)
    assert np.abs(o[0] - want0[None, :]).max() > 1e-3


_L_full = [None]


def test_planted_window_from_last_position(monkeypatch):
    """Windows measured from the chunk's last position instead of each query's own position
    are caught by the brute force."""
    inp = _mq("bf16", 4, context=30, window=6, window_frac=1.0)
    good = omq.multi_query_attention(*oracle_args(inp))
    want = _brute(inp)
    assert np.abs(good - want).max() <= 1e-12
    # the plausible mistake: every query keeps the keys [L - W, ...) of the last position
    W = int(inp.window[0])
    bad = np.empty_like(good)
    L = int(inp.context_lens[0])
    q4 = inp.q
    for i in range(4):
        pos = L - 4 + i
        wide = oracle.decode_attention(q4[:, i], inp.k_cache, inp.v_cache, inp.block_table,
                                       np.array([pos + 1]), "bf16", None, None, None,
                                       inp.softmax_scale, np.array([W + (3 - i)]), inp.softcap, 1, 64)
        bad[0, i] = wide[0]
    assert np.abs(bad - want).max() > 1e-6
