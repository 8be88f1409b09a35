"""Pins of the seeded input generator (the cache writer side), CPU only.

Encoders are checked against library routines (torch's bfloat16 / float8_e4m3fn casts, scipy
quadrature of the normal density), packers against hand-worked bytes and the oracle's
independent bit reader.
"""
import json
import math
import os

import numpy as np
import pytest

import kvgen
import oracle
from conftest import oracle_args

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_rounding_matches_torch(rng):
    torch = pytest.importorskip("torch")
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 3.3895314e38, 1e-40, -1e-40], np.float32)]).astype(np.float32)
    ours = kvgen.bf16_bits(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == lib).all()


def test_e4m3fn_encode_matches_torch(rng):
    torch = pytest.importorskip("torch")
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 60,
                        (rng.standard_normal(20000) * 1e-3).astype(np.float32),
                        np.array([448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 0.0], np.float32)])
    x = x[np.abs(x) <= 448].astype(np.float32)
    ours = kvgen.e4m3fn_encode(x)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == lib).all()


def test_e4m3fn_encode_saturates():
    codes = kvgen.e4m3fn_encode(np.array([470.0, 1e6, -1e6, 448.01], np.float32))
    assert codes.tolist() == [0x7E, 0x7E, 0xFE, 0x7E]


@pytest.mark.parametrize("n,mse_max", [(8, 0.03455), (16, 0.009502)])
def test_lloyd_max_fixed_point(n, mse_max):
    """Each level is its cell's conditional mean and each boundary the midpoint of its levels
    (checked by numerical quadrature of the N(0,1) density); distortion as Max (1960)."""
    from scipy import integrate, stats
    c = np.array(kvgen.lloyd_max_normal(n))
    b = np.concatenate(([-np.inf], 0.5 * (c[1:] + c[:-1]), [np.inf]))
    for i in range(n):
        mass = integrate.quad(stats.norm.pdf, b[i], b[i + 1], epsabs=1e-15)[0]
        mean = integrate.quad(lambda x: x * stats.norm.pdf(x), b[i], b[i + 1], epsabs=1e-15)[0] / mass
        assert abs(mean - c[i]) < 1e-9
    mse = sum(integrate.quad(lambda x: (x - c[i]) ** 2 * stats.norm.pdf(x), b[i], b[i + 1],
                             epsabs=1e-14)[0] for i in range(n))
    assert mse < mse_max
    assert np.allclose(c, -c[::-1], atol=0)


def test_codebook_scaled_fp32():
    cb = kvgen.codebook(16, 128)
    assert cb.dtype == np.float32 and np.all(np.diff(cb) > 0)
    assert cb[-1] == np.float32(kvgen.lloyd_max_normal(16)[-1] / math.sqrt(128))


def test_nearest_level_ties_low():
    lv = np.array([-1.0, 0.0, 1.0], np.float32)
    assert kvgen.nearest_level(np.array([-0.5, 0.5, 0.49, 0.51, 9.0, -9.0]), lv).tolist() == [0, 1, 1, 2, 2, 0]


@pytest.mark.parametrize("bits", [4, 3])
def test_turbo_encode_roundtrip(bits, rng):
    """Decoding (oracle's dense Hadamard path) recovers x to the codebook's distortion."""
    d = 128
    x = rng.standard_normal((2000, d)).astype(np.float32)
    s = kvgen.sign_pattern(rng, d)
    cb = kvgen.codebook(1 << bits, d)
    idx, norm = kvgen.turbo_encode(x, s, cb)
    assert np.abs(norm - np.linalg.norm(x.astype(np.float64), axis=1).astype(np.float32)).max() == 0
    x_hat = oracle.unrotate(norm[:, None].astype(np.float64) * cb.astype(np.float64)[idx], s)
    rel = ((x_hat - x) ** 2).sum(1) / (x.astype(np.float64) ** 2).sum(1)
    mse = {4: 0.009501, 3: 0.034548}[bits]
    assert 0.8 * mse < rel.mean() < 1.25 * mse


def test_pack_golden():
    for c in json.load(open(os.path.join(GOLDEN, "bitpack_le.json")))["cases"]:
        idx = np.array(c["indices"], np.uint8)
        if c["bits"] == 4:
            got = kvgen._pack_nibbles(idx)
        else:
            idx = np.concatenate([idx, np.zeros(32 - len(idx), np.uint8)])
            got = kvgen._pack_3bit(idx)
        assert got[: len(c["bytes"])].tolist() == c["bytes"]


@pytest.mark.parametrize("bits", [4, 3])
def test_pack_unpack_random(bits, rng):
    idx = rng.integers(0, 1 << bits, size=(500, 32)).astype(np.uint8)
    packed = kvgen._pack_nibbles(idx) if bits == 4 else kvgen._pack_3bit(idx)
    assert packed.shape[-1] == 4 * bits
    assert (oracle.unpack_le(packed, bits) == idx).all()


def test_layout_sizes():
    # codebook chunks: the indices, then 16 fp32 per-token norms (64 bytes)
    for fmt, kb, vb in [("bf16", 4096, 4096), ("fp8", 2048, 2048), ("turbo4", 1088, 1088),
                        ("turbo3", 832, 1088), ("turbo8", 2048, 1088)]:
        assert kvgen.k_chunk_bytes(fmt, 128) == kb and kvgen.v_chunk_bytes(fmt, 128) == vb
        assert kb % 16 == 0 and vb % 16 == 0          # chunks stay 16-byte aligned
    # bytes per (token, KV head): 512 / 256 / 136 / 120 / 196 (Turbo8: 128 K + 64 V + 4 norm)
    assert [kvgen.kv_bytes_per_token_head(f, 128) for f in kvgen.FORMATS] == [512, 256, 136, 120, 196]


def test_config_shapes():
    inp = kvgen.make_inputs(kvgen.SPECS["c1"])
    assert inp.q.shape == (1, 4, 64) and inp.kv_bytes() == 76800
    s = kvgen.SPECS["c3"]
    r = kvgen.make_inputs(kvgen.spec("c3", num_seqs=64, num_kv_heads=1, num_q_heads=4, head_dim=16))
    assert (r.window == 4096).sum() == 32 and r.context_lens.min() >= 1 and r.context_lens.max() <= 32768
    assert s.softcap == 50.0


@pytest.mark.parametrize("fmt", ["turbo4", "turbo8"])
def test_relayout_same_logical_cache(fmt):
    inp = kvgen.make_inputs(kvgen.spec("c1", fmt=fmt, head_dim=128, context=100))
    other = kvgen.relayout(inp, 5)
    assert not (other.block_table == inp.block_table).all()
    a = oracle.decode_attention(*oracle_args(inp))
    b = oracle.decode_attention(*oracle_args(other))
    assert (a == b).all()


def test_turbo8_scales_layout():
    """Turbo8: K bytes and K scales exactly as the FP8 format writes them for the same draws,
    V chunks (indices and inline norms) exactly as Turbo4 writes them; scales = the K scales."""
    kw = dict(head_dim=128, num_seqs=2, num_q_heads=4, num_kv_heads=2, context=None,
              ctx_range=(3, 70))
    t8 = kvgen.make_inputs(kvgen.spec("c1", fmt="turbo8", **kw))
    f8 = kvgen.make_inputs(kvgen.spec("c1", fmt="fp8", **kw))
    t4 = kvgen.make_inputs(kvgen.spec("c1", fmt="turbo4", **kw))
    assert t8.scales.shape == (2,) and t4.scales is None
    assert np.array_equal(t8.k_cache, f8.k_cache) and np.array_equal(t8.scales, f8.scales[0])
    assert np.array_equal(t8.v_cache, t4.v_cache)
    assert np.array_equal(t8.codebook, t4.codebook[16:])


def test_inline_norms():
    """The 16 fp32 values after a codebook chunk's indices are its tokens' norms: NaN on spare
    pages and tail slots (poison), finite and positive on live tokens."""
    inp = kvgen.make_inputs(kvgen.spec("c1", fmt="turbo4", head_dim=128, context=40))
    nrm = inp.k_cache[:, :, 1024:].copy().view("<f4")           # [pool, Hkv, 16]
    used = inp.block_table[0, :3]
    assert np.isfinite(nrm[used[0]]).all() and (nrm[used[0]] > 0).all()
    assert np.isfinite(nrm[used[2], 0, :8]).all() and np.isnan(nrm[used[2], 0, 8:]).all()
    spare = [p for p in range(inp.num_pool_blocks) if p not in set(inp.block_table[0, :3].tolist())]
    assert np.isnan(nrm[spare]).all()


def test_poison_spare_and_tail():
    inp = kvgen.make_inputs(kvgen.SPECS["c1"])
    used = set(inp.block_table[0].tolist())
    spare = [p for p in range(64) if p not in used]
    assert (inp.k_cache.view(np.uint16)[spare] == 0x7FC0).all()
    last = inp.block_table[0, 18]          # tokens 288..299 live, slots 12..15 are tail
    v = inp.v_cache.view(np.uint16)[last, 0].reshape(64, 16)
    assert (v[:, 12:] == 0x7FC0).all() and not (v[:, :12] == 0x7FC0).any()
