"""Pins of the fp64 oracle against things other than itself (CPU only).

* a 40-digit ``decimal`` brute force that reads the cache by byte offsets (oracle/brute.py);
* closed forms: Hadamard orthogonality, E4M3FN special values, the position-coded V count;
* identities: one token, uniform V, zero K, split = unsplit;
* library routines: torch's float8_e4m3fn decode, scipy's normal quadrature.
A final block plants plausible mistakes in the oracle and checks that a pin catches each.
"""
import json
import math
import os

import numpy as np
import pytest

import kvgen
import oracle
import oracle.attention as oa
from oracle.brute import brute_decode_attention
from conftest import brute_as_array, oracle_args

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(fmt, **kw):
    base = dict(fmt=fmt, head_dim=64 if fmt in ("bf16", "fp8") else 128)
    base.update(kw)
    return kvgen.make_inputs(kvgen.spec("c1", **base))


def _vs_brute(inp, tol=1e-12):
    o = oracle.decode_attention(*oracle_args(inp))
    b = brute_as_array(brute_decode_attention(*oracle_args(inp)))
    assert np.isfinite(o).all()
    err = np.abs(o - b).max()
    assert err <= tol, err
    return o


# --------------------------------------------------------------------------------------------
# oracle vs brute force
# --------------------------------------------------------------------------------------------
def test_brute_c1_tiny_config():
    """The tiny config itself: 1 seq, 4:1 GQA, D=64, L=300, scale 1/8, 19 pages of 64."""
    inp = kvgen.make_inputs(kvgen.SPECS["c1"])
    assert inp.block_table.shape == (1, 19) and inp.num_pool_blocks == 64
    assert len(set(inp.block_table[0].tolist())) == 19
    _vs_brute(inp)


@pytest.mark.parametrize("fmt", kvgen.FORMATS)
@pytest.mark.parametrize("L", [1, 2, 15, 16, 17])
def test_brute_formats_lengths(fmt, L):
    _vs_brute(_tiny(fmt, context=L, num_q_heads=2))


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_brute_multi_head_window_cap(fmt):
    """Several KV heads (GQA mapping), ragged lengths, windows on some sequences, softcap."""
    inp = _tiny(fmt, num_seqs=3, num_q_heads=6, num_kv_heads=2, context=None, ctx_range=(1, 60),
                window=9, window_frac=0.67, softcap=3.0, softmax_scale=0.5)
    assert (inp.window > 0).sum() == 2
    _vs_brute(inp)


def test_brute_large_logits_cap_order():
    """Large logits (scale x8) with cap 5: the cap must act on the scaled logit."""
    inp = _tiny("bf16", context=40, softmax_scale=1.0, softcap=5.0)
    _vs_brute(inp)


@pytest.mark.parametrize("fmt", ["turbo4", "turbo3", "turbo8"])
def test_brute_turbo_window(fmt):
    inp = _tiny(fmt, num_seqs=2, context=None, ctx_range=(5, 24), window=7, window_frac=0.5,
                num_q_heads=2)
    _vs_brute(inp)


def test_zero_length_rows_are_zero():
    inp = kvgen.make_inputs(kvgen.spec("c1", num_seqs=3), lengths=[0, 5, 0])
    o = oracle.decode_attention(*oracle_args(inp))
    assert (o[0] == 0).all() and (o[2] == 0).all() and np.isfinite(o[1]).all()


# --------------------------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_orthogonal_exact(n):
    h = oracle.sylvester_hadamard(n)
    assert (h @ h.T == n * np.eye(n, dtype=np.int64)).all()
    assert (h == h.T).all()
    ij = np.arange(n)
    parity = np.array([[bin(i & j).count("1") % 2 for j in ij] for i in ij])
    assert (h == np.where(parity, -1, 1)).all()


def test_unrotate_inverts_rotation(rng):
    d = 128
    s = np.where(rng.integers(0, 2, d) == 1, 1.0, -1.0)
    x = rng.standard_normal((5, d))
    h = oracle.sylvester_hadamard(d)
    x_rot = ((x * s) @ h.T) / math.sqrt(d)
    assert np.abs(oracle.unrotate(x_rot, s) - x).max() < 1e-13
    assert np.abs(np.linalg.norm(x_rot, axis=1) - np.linalg.norm(x, axis=1)).max() < 1e-12


def test_e4m3fn_specials():
    cases = json.load(open(os.path.join(GOLDEN, "e4m3fn_specials.json")))["values"]
    for c in cases:
        v = oracle.e4m3fn_value(c["code"])
        if c["value"] == "nan":
            assert math.isnan(v)
        else:
            assert v == c["value"] and math.copysign(1, v) == math.copysign(1, c["value"])


def test_e4m3fn_table_matches_torch():
    torch = pytest.importorskip("torch")
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = oracle.E4M3FN_TABLE
    assert (np.isnan(lib) == np.isnan(ours)).all()
    ok = ~np.isnan(ours)
    assert (lib[ok] == ours[ok]).all()
    assert np.isnan(ours).sum() == 2


def test_unpack_le_golden():
    for c in json.load(open(os.path.join(GOLDEN, "bitpack_le.json")))["cases"]:
        got = oracle.unpack_le(np.array(c["bytes"], dtype=np.uint8), c["bits"])
        assert got[: len(c["indices"])].tolist() == c["indices"]


def _count_bit_set(a, b, d):
    """#{j in [a, b): bit d of j is 1} -- closed form: each period of 2^(d+1) integers holds
    2^d with the bit set, and a partial period contributes max(0, rest - 2^d)."""
    def f(n):
        period = 1 << (d + 1)
        return (n // period) * (1 << d) + max(0, n % period - (1 << d))
    return f(b) - f(a)


@pytest.mark.parametrize("L,W", [(300, 0), (300, 37), (1000, 513), (77, 100), (16, 16), (17, 1)])
def test_position_coded_v_closed_form(L, W):
    """K = 0 gives uniform weights, and V[j][d] = bit d of j gives out[d] = count / span."""
    D = 64

    def kv(seq, n):
        j = np.arange(n)
        v = ((j[None, :, None] >> np.arange(D)[None, None, :]) & 1).astype(np.float32)
        return np.zeros((1, n, D), np.float32), v

    inp = kvgen.make_inputs(kvgen.spec("c1", pool_total=None), lengths=[L], windows=[W],
                            kv_override=kv)
    o = oracle.decode_attention(*oracle_args(inp))[0]
    lo = max(0, L - W) if W else 0
    want = np.array([_count_bit_set(lo, L, d) for d in range(D)]) / (L - lo)
    assert np.abs(o - want[None, :]).max() < 1e-15


# --------------------------------------------------------------------------------------------
# identities
# --------------------------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", kvgen.FORMATS)
def test_single_token_returns_v0(fmt):
    inp = _tiny(fmt, context=1)
    o = oracle.decode_attention(*oracle_args(inp))[0]
    v0 = oa.gather_kv(fmt, "v", inp.v_cache, inp.block_table[0], 0, 0, 1, inp.spec.head_dim,
                      scales=inp.scales, codebook=inp.codebook, sign=inp.sign)[0]
    assert (o == v0[None, :]).all()


def test_uniform_v_gives_constant():
    D = 64

    def kv(seq, n):
        r = np.random.default_rng(seq)
        return r.standard_normal((1, n, D)).astype(np.float32), np.full((1, n, D), 0.75, np.float32)

    inp = kvgen.make_inputs(kvgen.spec("c1"), kv_override=kv)
    o = oracle.decode_attention(*oracle_args(inp))
    assert np.abs(o - 0.75).max() <= 4e-16   # a few ulp of 0.75


def test_zero_k_gives_mean_of_v():
    D = 64
    inp = kvgen.make_inputs(kvgen.spec("c1"), windows=[100],
                            kv_override=lambda s, n: (np.zeros((1, n, D), np.float32),
                                                      np.random.default_rng(7).standard_normal((1, n, D)).astype(np.float32)))
    o = oracle.decode_attention(*oracle_args(inp))[0]
    v = oa.gather_kv("bf16", "v", inp.v_cache, inp.block_table[0], 0, 200, 300, D)
    assert np.abs(o - v.mean(axis=0)[None, :]).max() < 1e-14


@pytest.mark.parametrize("ps", [0, -1, 16, 128, 512])
def test_split_equals_unsplit(ps):
    inp = kvgen.make_inputs(kvgen.spec("c1", context=2100, head_dim=64, pool_total=None))
    full = oracle.decode_attention(*oracle_args(inp))[0]
    parts = oracle.partition_partials(*oracle_args(inp), ps, 0, 0)
    if ps == 0:
        assert [(a, b) for a, b, *_ in parts] == [(512 * i, min(2100, 512 * i + 512)) for i in range(5)]
    if ps == 128:
        assert len(parts) == math.ceil(2100 / 128)
    merged = oracle.lse_merge([p[2] for p in parts], [p[3] for p in parts], [p[4] for p in parts])
    assert np.abs(merged - full).max() < 1e-13


def test_partition_rule():
    p = oracle.partitions
    assert p(300, 0) == [(0, 300)]
    assert p(1023, 0) == [(0, 1023)]
    assert p(1024, 0) == [(0, 512), (512, 1024)]
    assert p(300, 0, 128) == [(0, 128), (128, 256), (256, 300)]
    assert p(5000, 4096) == [(904, 1024), (1024, 1536), (1536, 2048), (2048, 2560), (2560, 3072),
                             (3072, 3584), (3584, 4096), (4096, 4608), (4608, 5000)]
    assert p(5000, 1000) == [(4000, 5000)]
    assert p(0, 0) == []
    assert p(40000, 0, -1) == [(0, 40000)]


def test_softcap_infinite_equals_none():
    a = _tiny("bf16", context=50)
    o1 = oracle.decode_attention(*oracle_args(a))
    import dataclasses
    b = dataclasses.replace(a, softcap=np.float32(1e30))
    o2 = oracle.decode_attention(*oracle_args(b))
    assert np.abs(o1 - o2).max() < 1e-15


# --------------------------------------------------------------------------------------------
# planted mistakes: each must trip one of the pins above
# --------------------------------------------------------------------------------------------
def _brute_mismatch(inp):
    o = oracle.decode_attention(*oracle_args(inp))
    b = brute_as_array(brute_decode_attention(*oracle_args(inp)))
    return not (np.abs(o - b).max() <= 1e-12)


def test_planted_v_layout_transposed(monkeypatch):
    # reads V as row-major [16][D] instead of the transposed [D][16]
    monkeypatch.setattr(oa, "_page_elems_v", lambda fmt, c, d: c.view(np.uint16).reshape(16, d))
    assert _brute_mismatch(_tiny("bf16", context=40))


def test_planted_k_layout_rowmajor(monkeypatch):
    monkeypatch.setattr(oa, "_page_elems_k",
                        lambda fmt, c, d: c.view(np.uint16).reshape(16, d))
    assert _brute_mismatch(_tiny("bf16", context=40))


def test_planted_missing_sign(monkeypatch):
    orig = oa.unrotate
    monkeypatch.setattr(oa, "unrotate", lambda x, s: orig(x, np.ones_like(s)))
    assert _brute_mismatch(_tiny("turbo4", context=9, num_q_heads=2))


def test_planted_turbo8_scale_of_wrong_head(monkeypatch):
    """Turbo8 with two KV heads: the K scale of head 0 used for both heads, or the inline V norms
    read one token off, is caught by the brute force."""
    inp = _tiny("turbo8", num_seqs=2, num_q_heads=4, num_kv_heads=2, context=None,
                ctx_range=(3, 30))
    good = oa.fp8_scale
    monkeypatch.setattr(oa, "fp8_scale", lambda f, sc, w, hk, hkv: good(f, sc, w, 0, hkv))
    assert _brute_mismatch(inp)
    monkeypatch.setattr(oa, "fp8_scale", good)
    norms = oa.token_norms
    monkeypatch.setattr(oa, "token_norms", lambda *a: np.roll(norms(*a), 1))
    assert _brute_mismatch(inp)


def test_planted_window_off_by_one(monkeypatch):
    monkeypatch.setattr(oa, "attended_range", lambda L, W: ((max(0, L - W + 1) if W > 0 else 0), L))
    D = 64

    def kv(seq, n):
        j = np.arange(n)
        return (np.zeros((1, n, D), np.float32),
                ((j[None, :, None] >> np.arange(D)[None, None, :]) & 1).astype(np.float32))

    inp = kvgen.make_inputs(kvgen.spec("c1"), windows=[37], kv_override=kv)
    o = oracle.decode_attention(*oracle_args(inp))[0]
    want = np.array([_count_bit_set(263, 300, d) for d in range(D)]) / 37
    assert np.abs(o - want[None, :]).max() > 1e-3


def test_planted_cap_before_scale(monkeypatch):
    def bad(q, k, scale, cap, bias=None):
        z = q @ k.T
        c = float(np.float32(cap))
        if c > 0:
            z = c * np.tanh(z / c)
        return float(np.float32(scale)) * z
    monkeypatch.setattr(oa, "logits", bad)
    assert _brute_mismatch(_tiny("bf16", context=40, softmax_scale=0.25, softcap=5.0))


def test_planted_alibi_before_cap_or_flipped(monkeypatch):
    """The ALiBi term added before the cap, or with the distance's sign flipped, is caught
    by the brute force."""
    inp = _tiny("bf16", num_q_heads=4, num_kv_heads=2, context=30, softcap=2.0)
    sl = _slopes(4)
    want = brute_as_array(brute_decode_attention(*oracle_args(inp), alibi=sl))
    good = oa.logits

    def before_cap(q, k, scale, cap, bias=None):
        return good(q, k, scale, 0.0, None) if bias is None else \
            float(np.float32(cap)) * np.tanh((good(q, k, scale, 0.0, None) + bias) / float(np.float32(cap)))
    monkeypatch.setattr(oa, "logits", before_cap)
    assert np.abs(oracle.decode_attention(*oracle_args(inp), alibi=sl) - want).max() > 1e-6
    monkeypatch.setattr(oa, "logits", good)
    monkeypatch.setattr(oa, "alibi_bias", lambda s, L, t0, t1: -good_bias(s, L, t0, t1))
    assert np.abs(oracle.decode_attention(*oracle_args(inp), alibi=sl) - want).max() > 1e-6


good_bias = oa.alibi_bias


def test_planted_gqa_mapping(monkeypatch):
    monkeypatch.setattr(oa, "_q_rows", bf16_rows_interleaved)
    inp = _tiny("bf16", num_q_heads=4, num_kv_heads=2, context=20)
    assert _brute_mismatch(inp)


def bf16_rows_interleaved(q, b, h0, g):
    """A wrong GQA mapping: query head h -> KV head h mod Hkv instead of h div g."""
    hkv = q.shape[1] // g
    hk = h0 // g
    rows = [hk + i * hkv for i in range(g)]
    return oracle.bf16_to_f64(np.asarray(q)[b, rows])


def test_planted_merge_without_l(monkeypatch):
    def bad(ms, ls, os_):
        ms = np.asarray(ms)
        w = np.exp(ms - ms.max(axis=0))
        return np.einsum("pg,pgd->gd", w, np.asarray(os_)) / w.sum(axis=0)[:, None]
    monkeypatch.setattr(oa, "lse_merge", bad)
    inp = kvgen.make_inputs(kvgen.spec("c1", context=2100, pool_total=None))
    full = oracle.decode_attention(*oracle_args(inp), chunk=1 << 20)[0]
    parts = oracle.partition_partials(*oracle_args(inp), 0, 0, 0)
    merged = oa.lse_merge([p[2] for p in parts], [p[3] for p in parts], [p[4] for p in parts])
    assert np.abs(merged - full).max() > 1e-6


def test_planted_fnuz_decode():
    """The gfx942 FNUZ reading of FP8 (bias 8) would disagree with torch's E4M3FN decode."""
    torch = pytest.importorskip("torch")
    fnuz = np.array([oracle.e4m3fn_value(c) / 2 for c in range(256)])
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ok = ~np.isnan(lib)
    assert (fnuz[ok] != lib[ok]).any()


# --------------------------------------------------------------------------------------------
# ALiBi (the "ALiBi slopes" feature of the attention.rs README)
# --------------------------------------------------------------------------------------------
def _slopes(h, base=8.0):
    """The usual geometric ALiBi slopes 2^(-base (i+1) / h), as fp32."""
    return (2.0 ** (-base * (np.arange(h) + 1) / h)).astype(np.float32)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "turbo4", "turbo8"])
def test_brute_alibi(fmt):
    inp = _tiny(fmt, num_seqs=2, num_q_heads=4, num_kv_heads=2, context=None, ctx_range=(3, 40),
                window=11, window_frac=0.5, softcap=2.0 if fmt == "bf16" else 0.0)
    sl = _slopes(4)
    o = oracle.decode_attention(*oracle_args(inp), alibi=sl)
    b = brute_as_array(brute_decode_attention(*oracle_args(inp), alibi=sl))
    assert np.abs(o - b).max() <= 1e-12


@pytest.mark.parametrize("L,W", [(300, 0), (300, 40), (17, 0)])
def test_alibi_closed_form(L, W):
    """K = 0: the logits are the ALiBi terms alone, slope * (j - (L - 1)); with V[j][d] = bit
    d of j the output is the exp-weighted share of keys with that bit set."""
    D = 64

    def kv(seq, n):
        j = np.arange(n)
        v = ((j[None, :, None] >> np.arange(D)[None, None, :]) & 1).astype(np.float32)
        return np.zeros((1, n, D), np.float32), v

    inp = kvgen.make_inputs(kvgen.spec("c1", pool_total=None), lengths=[L], windows=[W],
                            kv_override=kv)
    sl = _slopes(4, base=5.0)
    o = oracle.decode_attention(*oracle_args(inp), alibi=sl)[0]
    lo = max(0, L - W) if W else 0
    j = np.arange(lo, L)
    bits = (j[:, None] >> np.arange(D)[None, :]) & 1
    for h in range(4):
        w = np.exp(np.float64(sl[h]) * (j - (L - 1)))
        want = (w[:, None] * bits).sum(axis=0) / w.sum()
        assert np.abs(o[h] - want).max() < 1e-14, h
