"""Pins of the oracle's cache writer (oracle/encode.py), CPU only.

Each encoder is checked against something other than itself: torch's bfloat16 and
float8_e4m3fn casts, exhaustive enumeration of the E4M3FN codes and of the midpoints between
them, the Hadamard matrix identities H H = D I and norm preservation, brute-force nearest
level, the hand-worked little-endian packing fixture, the oracle's independent bit reader, and
the input generator's own (separately written) rotated-codebook encoder.
"""
import json
import math
import os

import numpy as np
import pytest

import kvgen
import oracle
import oracle.attention as oa
from oracle import encode as enc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- BF16 ----------------------------------------------------------------------------------
def test_bf16_matches_torch(rng):
    torch = pytest.importorskip("torch")
    x = np.concatenate([rng.standard_normal(50000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 50000),
                        np.array([0.0, -0.0, 1.0, 3.3895314e38, 1e-40, -1e-40, np.inf, -np.inf], np.float32)])
    x = x.astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (enc.bf16_encode(x) == lib).all()


def test_bf16_nan_is_canonical():
    assert enc.bf16_encode(np.array([np.nan, -np.nan], np.float32)).tolist() == [0x7FC0, 0x7FC0]


# ---- FP8 E4M3FN ----------------------------------------------------------------------------
def test_e4m3_every_finite_code_round_trips():
    for c in range(256):
        v = oracle.e4m3fn_value(c)
        if math.isnan(v):
            continue
        assert enc.e4m3fn_code(v) == c, hex(c)


def test_e4m3_midpoints_round_to_even():
    """Exactly halfway between two neighbouring positive codes -> the even code."""
    for c in range(0, 0x7E):
        lo, hi = oracle.e4m3fn_value(c), oracle.e4m3fn_value(c + 1)
        want = c if c % 2 == 0 else c + 1
        assert enc.e4m3fn_code((lo + hi) / 2) == want, hex(c)
        assert enc.e4m3fn_code(-(lo + hi) / 2) == 0x80 | want, hex(c)
        # just either side of the midpoint
        assert enc.e4m3fn_code(np.nextafter((lo + hi) / 2, 0.0)) == c
        assert enc.e4m3fn_code(np.nextafter((lo + hi) / 2, 1e9)) == c + 1


def test_e4m3_matches_torch(rng):
    torch = pytest.importorskip("torch")
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 60,
                        (rng.standard_normal(5000) * 1e-3).astype(np.float32)])
    x = x[np.abs(x) <= 448].astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (enc.fp8_encode(x, 1.0) == lib).all()


def test_e4m3_saturates_and_nan():
    codes = enc.fp8_encode(np.array([448.01, 470.0, 1e6, -1e6, np.inf, np.nan], np.float32), 1.0)
    assert codes.tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0x7F]


def test_e4m3_scale_is_one_fp32_division(rng):
    x = rng.standard_normal(3000).astype(np.float32) * 3
    s = np.float32(0.00731)
    assert (enc.fp8_encode(x, s) == enc.fp8_encode((x / s).astype(np.float32), 1.0)).all()


# ---- rotated codebook ------------------------------------------------------------------------
def test_hadamard_rows_is_the_sylvester_matrix(rng):
    x = rng.standard_normal((5, 128))
    h = oracle.sylvester_hadamard(128).astype(np.float64)
    assert np.allclose(enc.hadamard_rows(x), x @ h.T, rtol=0, atol=1e-12)
    # H H = D I, exactly for integer inputs
    xi = rng.integers(-1000, 1000, (3, 128)).astype(np.float64)
    assert np.array_equal(enc.hadamard_rows(enc.hadamard_rows(xi)), 128 * xi)


def test_pairwise_sum_tree_order():
    # 1e16 + 1 - 1e16 ... the tree order is visible: (a0+a1) + (a2+a3)
    v = np.array([1e16, 1.0, -1e16, 1.0])
    assert enc.pairwise_sum(v) == (1e16 + 1.0) + (-1e16 + 1.0)
    assert enc.pairwise_sum(np.arange(64.0)) == 64 * 63 / 2


def test_nearest_index_brute_force(rng):
    levels = kvgen.codebook(16, 128)
    u = np.concatenate([rng.standard_normal(5000) * 0.12,
                        (levels[1:].astype(np.float64) + levels[:-1].astype(np.float64)) / 2])
    got = enc.nearest_index(u, levels)
    lv = levels.astype(np.float64)
    for ui, gi in zip(u, got):
        dist = np.abs(ui - lv)
        best = np.flatnonzero(dist == dist.min())
        assert gi == best.min()      # nearest, ties to the lower level


@pytest.mark.parametrize("levels_n", [16, 8])
def test_turbo_encode_properties(levels_n, rng):
    d = 128
    x = rng.standard_normal((200, d)).astype(np.float32)
    sign = np.where(rng.integers(0, 2, d) == 1, 1.0, -1.0).astype(np.float32)
    levels = kvgen.codebook(levels_n, d)
    idx, norm = enc.turbo_encode(x, sign, levels)
    # norm is the fp32-rounded L2 norm of x (= of the rotated vector)
    assert np.allclose(norm, np.linalg.norm(x.astype(np.float64), axis=1), rtol=1e-7)
    # decoding (norm * level, un-rotated) is the Lloyd-Max approximation of x
    back = oracle.unrotate(norm[:, None].astype(np.float64) * levels.astype(np.float64)[idx], sign)
    rel = np.sum((back - x) ** 2, axis=1) / np.sum(x.astype(np.float64) ** 2, axis=1)
    # Lloyd-Max distortion for N(0,1): 0.00950 (16 levels), 0.03455 (8 levels)
    assert rel.mean() < (0.0125 if levels_n == 16 else 0.042)
    # every coordinate sits in the cell of its level
    r = enc.hadamard_rows(x.astype(np.float64) * sign) / math.sqrt(d) / norm[:, None]
    lv = levels.astype(np.float64)
    mids = np.concatenate([[-np.inf], (lv[1:] + lv[:-1]) / 2, [np.inf]])
    assert ((r > mids[idx]) & (r <= mids[idx + 1])).all()


def test_turbo_encode_zero_vector():
    levels = kvgen.codebook(16, 128)
    idx, norm = enc.turbo_encode(np.zeros((1, 128), np.float32), np.ones(128, np.float32), levels)
    assert norm[0] == 0 and (idx == 7).all()     # 0 is the midpoint of levels 7 and 8 -> 7


def test_turbo_encode_agrees_with_generator(rng):
    """kvgen's encoder is written separately (einsum norm, other transform code)."""
    d = 128
    x = rng.standard_normal((500, d)).astype(np.float32)
    sign = np.where(rng.integers(0, 2, d) == 1, 1.0, -1.0).astype(np.float32)
    for n in (16, 8):
        levels = kvgen.codebook(n, d)
        a, na = enc.turbo_encode(x, sign, levels)
        b, nb = kvgen.turbo_encode(x, sign, levels)
        assert np.array_equal(na, nb)
        assert np.array_equal(a, b.astype(np.int64))


# ---- packing and placement -----------------------------------------------------------------
def test_pack_le_golden():
    for case in json.load(open(os.path.join(GOLDEN, "bitpack_le.json")))["cases"]:
        assert enc.pack_le(np.array(case["indices"]), case["bits"]).tolist() == case["bytes"]


@pytest.mark.parametrize("bits", [3, 4])
def test_pack_le_inverts_the_reader(bits, rng):
    v = rng.integers(0, 1 << bits, (7, 32))
    assert np.array_equal(oracle.unpack_le(enc.pack_le(v, bits), bits), v)


@pytest.mark.parametrize("fmt", kvgen.FORMATS)
def test_append_then_gather(fmt, rng):
    """Tokens written by append_tokens read back (through the oracle's gather) as their
    encodings; the other tokens of the pages are unchanged."""
    s = kvgen.spec("c1", fmt=fmt, head_dim=128, num_q_heads=4, num_kv_heads=2, pool_total=None,
                   num_seqs=2)
    inp = kvgen.make_inputs(s, lengths=[40, 70])
    T = 20
    pos = np.array([5, 43])      # sequence 1 writes tokens 43..62, crossing a page boundary
    kn = rng.standard_normal((2, T, 2, 128)).astype(np.float32)
    vn = rng.standard_normal((2, T, 2, 128)).astype(np.float32)
    k2, v2, sc2 = enc.append_tokens(fmt, kn, vn, inp.block_table, pos, inp.k_cache, inp.v_cache,
                                    inp.scales, inp.codebook, inp.sign)
    for b in range(2):
        for hk in range(2):
            for which, new, cache, old in (("k", kn, k2, inp.k_cache), ("v", vn, v2, inp.v_cache)):
                got = oracle.gather_stored(fmt, which, cache, inp.block_table[b], hk, pos[b], pos[b] + T, 128)
                want, norm = enc.encode_tokens(fmt, which, new[b, :, hk], hk=hk, hkv=2,
                                               scales=inp.scales, codebook=inp.codebook,
                                               sign=inp.sign)
                assert np.array_equal(got, want)
                if norm is not None:    # fp32 norms after each chunk's indices
                    got_n = oa.token_norms(fmt, which, cache, inp.block_table[b], hk, pos[b],
                                           pos[b] + T, 128)
                    assert np.array_equal(got_n, norm)
                    before_n = oa.token_norms(fmt, which, old, inp.block_table[b], hk, 0, pos[b], 128)
                    after_n = oa.token_norms(fmt, which, cache, inp.block_table[b], hk, 0, pos[b], 128)
                    assert np.array_equal(before_n, after_n, equal_nan=True)
                before = oracle.gather_stored(fmt, which, old, inp.block_table[b], hk, 0, pos[b], 128)
                after = oracle.gather_stored(fmt, which, cache, inp.block_table[b], hk, 0, pos[b], 128)
                assert np.array_equal(before, after)
