"""GPU, bit-exact: the matrix-core operands the partition kernel itself forms from the cache.

kvd_dequant_operands runs the partition kernel's own load (lane map, 16-byte loads), FP8 decode
and codebook pair-table code (table fill and v_perm / bit-field addressing) on page pairs and
exports every lane's operand registers.  The expected words are built here from the oracle's
gather of the stored elements (its own layout reader and little-endian bit unpacking), the
E4M3FN closed form and the codebook levels, with the lane -> (token, element) placement the
header documents.  Any permutation of nibbles, 3-bit fields, lanes, slots or table entries in
the hot path changes some word.
"""
import numpy as np
import pytest

import kvgen
import oracle
from gpu_harness import GpuBatch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bf16_bits_of(values):
    """bf16 bit patterns of values that are exactly representable in bf16 (NaN -> 0x7FC0)."""
    f = np.asarray(values, dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint32)
    assert ((f.view(np.uint32) & 0xFFFF) == 0)[~np.isnan(f)].all()
    return np.where(np.isnan(f), np.uint32(0x7FC0), bits)


def _hilo_bits(levels):
    """fp16 (hi, lo) bit patterns of each level scaled by 2^-E (largest magnitude in [0.5, 1)):
    hi = fp16(c), lo = fp16(c - hi), both rounded to nearest even."""
    lv = np.asarray(levels, dtype=np.float32)
    _, e = np.frexp(np.abs(lv).max())
    c = (lv * np.float32(2.0 ** -int(e))).astype(np.float32)
    hi = c.astype(np.float16)
    lo = (c - hi.astype(np.float32)).astype(np.float16)
    return hi.view(np.uint16).astype(np.uint32), lo.view(np.uint16).astype(np.uint32)


def _f16_bits(levels):
    """fp16 bit patterns of each level scaled by 2^-E (largest magnitude in [0.5, 1)), rounded
    once to nearest even."""
    lv = np.asarray(levels, dtype=np.float32)
    _, e = np.frexp(np.abs(lv).max())
    return (lv * np.float32(2.0 ** -int(e))).astype(np.float16).view(np.uint16).astype(np.uint32)


def _split(idx8, hi, lo):
    """Words [h0|h1, h2|h3, h4|h5, h6|h7] then [l0|l1, ..., l6|l7] of eight indices (the K-table
    operands: hi parts, then lo parts)."""
    h = [hi[i] for i in idx8]
    l = [lo[i] for i in idx8]
    return np.array([h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16, h[6] | h[7] << 16,
                     l[0] | l[1] << 16, l[2] | l[3] << 16, l[4] | l[5] << 16, l[6] | l[7] << 16],
                    dtype=np.uint32)


def _pairs_of_bits(b8):
    return np.array([b8[0] | b8[1] << 16, b8[2] | b8[3] << 16, b8[4] | b8[5] << 16,
                     b8[6] | b8[7] << 16], dtype=np.uint32)


def expected_records(inp, b, hk, n_pairs):
    """uint32 [n_pairs][64][D + 16] the export must write, and a mask of words whose value is a
    NaN (compared as NaN-ness only)."""
    s, fmt, D = inp.spec, inp.spec.fmt, inp.spec.head_dim
    T = 32 * n_pairs
    ks = oracle.gather_stored(fmt, "k", inp.k_cache, inp.block_table[b], hk, 0, T, D)
    vs = oracle.gather_stored(fmt, "v", inp.v_cache, inp.block_table[b], hk, 0, T, D)
    kkind, vkind = oracle.attention.elem_kind(fmt, "k"), oracle.attention.elem_kind(fmt, "v")
    klev, vlev = (oracle.attention.codebooks(fmt, inp.codebook) if vkind == "cb" else (None, None))
    kh = kl = vh = None
    if kkind == "cb":
        kh, kl = _hilo_bits(klev)
    if vkind == "cb":
        vh = _f16_bits(vlev)
    e4m3_bf16 = _bf16_bits_of(oracle.E4M3FN_TABLE.astype(np.float32))
    kn = vn = None      # [pool][Hkv][16]: the norms after each chunk's indices
    if kkind == "cb":
        kn = oracle.attention.chunk_norms(fmt, "k", inp.k_cache, D)
    if vkind == "cb":
        vn = oracle.attention.chunk_norms(fmt, "v", inp.v_cache, D)
    W = D + 16
    out = np.zeros((n_pairs, 64, W), dtype=np.uint32)
    nan = np.zeros_like(out, dtype=bool)
    for k in range(n_pairs):
        for lane in range(64):
            n, j = lane % 16, lane // 16
            a_sel, a_pos = n // 8, 8 * ((n // 4) % 2) + n % 4
            v_sel, v_pos0 = j // 2, 8 * (j % 2)
            rec = out[k, lane]
            for s_ in range(D // 32):
                for tile, tok in enumerate(((2 * k + a_sel) * 16 + a_pos, (2 * k + a_sel) * 16 + a_pos + 4)):
                    w0 = 16 * s_ + 8 * tile
                    if kkind == "bf16":
                        d = 32 * s_ + 8 * j + np.arange(8)
                        rec[w0: w0 + 4] = _pairs_of_bits(ks[tok, d].astype(np.uint32))
                    elif kkind == "fp8":
                        d = 64 * (s_ // 2) + 16 * j + 8 * (s_ % 2) + np.arange(8)
                        codes = ks[tok, d]
                        rec[w0: w0 + 4] = _pairs_of_bits(e4m3_bf16[codes])
                        for e in range(8):
                            if np.isnan(oracle.E4M3FN_TABLE[codes[e]]):
                                nan[k, lane, w0 + e // 2] = True
                    else:
                        d = 32 * j + 8 * s_ + np.arange(8)
                        rec[w0: w0 + 8] = _split(ks[tok, d], kh, kl)
            toks = (2 * k + v_sel) * 16 + v_pos0 + np.arange(8)
            for t in range(D // 16):
                w0 = D // 2 + 8 * t
                d = 16 * t + n
                if vkind == "bf16":
                    rec[w0: w0 + 4] = _pairs_of_bits(vs[toks, d].astype(np.uint32))
                elif vkind == "fp8":
                    codes = vs[toks, d]
                    rec[w0: w0 + 4] = _pairs_of_bits(e4m3_bf16[codes])
                    for e in range(8):
                        if np.isnan(oracle.E4M3FN_TABLE[codes[e]]):
                            nan[k, lane, w0 + e // 2] = True
                else:
                    rec[w0: w0 + 4] = _pairs_of_bits(vh[vs[toks, d]])
            phys = np.asarray(inp.block_table[b])[toks // 16]
            for plane, off in ((kn, D), (vn, D + 8)):
                if plane is not None:
                    vals = plane[phys, hk, toks % 16].astype(np.float32)
                    rec[off: off + 8] = vals.view(np.uint32)
                    nan[k, lane, off: off + 8] = np.isnan(vals)
    return out, nan


@pytest.mark.parametrize("fmt,D", [("bf16", 128), ("bf16", 64), ("fp8", 128), ("fp8", 64),
                                   ("turbo4", 128), ("turbo3", 128), ("turbo8", 128)])
def test_partition_kernel_operands_bit_exact(fmt, D):
    import torch
    inp = kvgen.make_inputs(kvgen.spec("c1", fmt=fmt, head_dim=D, num_seqs=2, num_q_heads=8,
                                       num_kv_heads=2, context=None, ctx_range=(300, 700),
                                       pool_total=None))
    gb = GpuBatch(inp)
    s = inp.spec
    n_pairs = inp.max_blocks_per_seq // 2
    seen = set()
    for b in range(s.num_seqs):
        for hk in range(s.num_kv_heads):
            out = torch.zeros((n_pairs, 64, D + 16), dtype=torch.int32, device="cuda:0")
            gb.kvd.dequant_operands(gb.dims, fmt, gb.t["k_cache"], gb.t["v_cache"], gb.t["scales"],
                                    gb.t["codebook"], gb.t["block_table"], b, hk, 0, n_pairs, out)
            torch.cuda.synchronize()
            got = out.cpu().numpy().view(np.uint32)
            want, nan = expected_records(inp, b, hk, n_pairs)
            bad = (got != want) & ~nan
            assert not bad.any(), (b, hk, np.argwhere(bad)[:5])
            if fmt.startswith("turbo"):
                seen |= set(oracle.gather_stored(fmt, "v", inp.v_cache, inp.block_table[b], hk, 0,
                                                 32 * n_pairs, D).ravel().tolist())
    if fmt.startswith("turbo"):
        assert seen == set(range(16))   # every V level went through the table


def test_operands_reject_pairs_past_the_table():
    import torch
    inp = kvgen.make_inputs(kvgen.spec("c1", fmt="fp8", head_dim=128, context=100,
                                       pool_total=None))
    gb = GpuBatch(inp)
    out = torch.zeros((8, 64, 144), dtype=torch.int32, device="cuda:0")
    n_pairs = inp.max_blocks_per_seq // 2 + 1
    with pytest.raises(gb.kvd.KvdError):
        gb.kvd.dequant_operands(gb.dims, "fp8", gb.t["k_cache"], gb.t["v_cache"], gb.t["scales"],
                                None, gb.t["block_table"], 0, 0, 0, n_pairs, out)
