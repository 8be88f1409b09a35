"""Oracle: plain CPU definition of writing new tokens into the paged KV cache -- the cache
writer whose output the decode path reads.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with the GPU
library (nor with the input generator ``kvgen``): encoding, bit packing and page placement are
written out here on their own.

What it follows (page titles and sections of the source pages):
  * attention.rs README, "KV Cache Formats": BF16, FP8 (E4M3) and the Walsh-Hadamard formats
    Turbo8 (FP8 K + 4-bit V), Turbo4 (4-bit K + 4-bit V) and Turbo3 (3-bit K + 4-bit V) are
    cache storage formats.
  * turboquant-rs 0.4.1 src/cache/cuda/attention.rs: the compressed cache holds packed indices
    and per-token scales, read back with a sign pattern and a codebook.
  * The recipe the compressed-cache workload states: each K and V token vector is multiplied
    by a +-1 sign pattern, then by the orthonormal Walsh-Hadamard transform, normalised by its
    fp32 L2 norm (stored per token), and every coordinate is replaced by the index of the
    nearest Lloyd-Max level; indices are bit-packed little-endian into bytes.

Readings taken where the pages are silent (the library header states the same ones):
  * BF16: the fp32 value rounded to nearest, ties to even; NaN is stored as 0x7FC0.
  * FP8: q = fp32(x / scale) (one IEEE fp32 division), then rounded to nearest-even OCP
    E4M3FN, saturating to +-448; NaN is stored as 0x7F.
  * Rotated codebook, decided in fp64: r = H (s * x) / sqrt(D) (H the Sylvester-order
    Hadamard matrix, applied as the usual butterfly stages h = 1, 2, 4, ...; exact in fp64 for
    fp32 inputs), norm = fp32(sqrt(sum x_i^2)) with the sum taken as a pairwise tree over the
    index order (adjacent pairs first), u = r / norm, index = the number of level midpoints
    (c_k + c_{k+1}) / 2 strictly below u (a tie goes to the lower level).  A zero vector has
    norm 0 and every index is the level nearest 0.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import (BLOCK, _FMT_BITS, _page_elems_k, _page_elems_v, code_bytes, elem_kind,
                        fp8_scale)


# --------------------------------------------------------------------------------------------
# Element encoders
# --------------------------------------------------------------------------------------------
def bf16_encode(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bits, round to nearest, ties to even (done on the integer bit pattern:
    add half an ulp of the kept part plus the kept part's lowest bit, truncate)."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    out = ((bits + 0x7FFF + lsb) >> 16).astype(np.uint16)
    out[np.isnan(np.asarray(x, dtype=np.float32))] = 0x7FC0
    return out


def e4m3fn_code(v: float) -> int:
    """One finite or NaN fp32 value -> OCP E4M3FN code, round to nearest even, saturating.

    Normal codes: (-1)^s 2^(e-7) (1 + m/8) for e in 1..15 (e = 15 with m = 7 is NaN, so the
    largest finite value is 1.75 * 2^8 = 448); subnormals (-1)^s 2^-6 (m/8)."""
    if math.isnan(v):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0x00
    a = abs(v)
    if a >= 448.0:
        return sign | 0x7E
    if a < 2.0 ** -6:                        # subnormal step 2^-9; 8 * 2^-9 is 2^-6 (code 8)
        return sign | int(np.rint(a * 512.0))
    e = math.floor(math.log2(a))
    if 2.0 ** e > a:                         # guard log2 rounding
        e -= 1
    if 2.0 ** (e + 1) <= a:
        e += 1
    m = int(np.rint((a / 2.0 ** e - 1.0) * 8.0))   # exact in fp64: a has 24 bits
    if m == 8:
        e, m = e + 1, 0
    code = ((e + 7) << 3) | m
    return sign | min(code, 0x7E)


def fp8_encode(x: np.ndarray, scale) -> np.ndarray:
    """fp32 values and one fp32 scale -> E4M3FN codes of fp32(x / scale)."""
    q = np.asarray(x, dtype=np.float32) / np.float32(scale)       # IEEE fp32 division
    flat = q.reshape(-1)
    out = np.fromiter((e4m3fn_code(float(v)) for v in flat), dtype=np.uint8, count=flat.size)
    return out.reshape(q.shape)


def hadamard_rows(x: np.ndarray) -> np.ndarray:
    """H x along the last axis in fp64, as butterfly stages h = 1, 2, 4, ...: in each block
    of 2h elements, (a, b) -> (a + b, a - b) for a in the first half and b in the second."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        blocks = y.reshape(*y.shape[:-1], d // (2 * h), 2, h)
        a = blocks[..., 0, :].copy()
        b = blocks[..., 1, :].copy()
        blocks[..., 0, :] = a + b
        blocks[..., 1, :] = a - b
        h *= 2
    return y


def pairwise_sum(v: np.ndarray) -> np.ndarray:
    """Sum along the last axis (a power of two long) as a pairwise tree: adjacent pairs
    first, then adjacent pair sums, and so on (fp64)."""
    s = np.asarray(v, dtype=np.float64)
    while s.shape[-1] > 1:
        s = s[..., 0::2] + s[..., 1::2]
    return s[..., 0]


def nearest_index(u: np.ndarray, levels) -> np.ndarray:
    """Index of the nearest level (levels ascending fp32, compared in fp64); a value exactly
    halfway between two levels takes the lower one."""
    lv = np.asarray(levels, dtype=np.float32).astype(np.float64)
    mids = (lv[1:] + lv[:-1]) / 2.0
    return (np.asarray(u, dtype=np.float64)[..., None] > mids).sum(axis=-1).astype(np.int64)


def turbo_encode(x: np.ndarray, sign, levels):
    """Token vectors x [..., D] (fp32) -> (indices [..., D] int64, norms [...] fp32)."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    xd = x.astype(np.float64)
    r = hadamard_rows(xd * np.asarray(sign, dtype=np.float32).astype(np.float64)) / math.sqrt(d)
    norm = np.sqrt(pairwise_sum(xd * xd)).astype(np.float32)
    n64 = norm.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(n64 > 0, r / np.where(n64 > 0, n64, 1.0), 0.0)
    return nearest_index(u, levels), norm


# --------------------------------------------------------------------------------------------
# Packing (the inverse of the oracle's readers) and page placement
# --------------------------------------------------------------------------------------------
def pack_le(values: np.ndarray, bits: int) -> np.ndarray:
    """Little-endian bitstream pack along the last axis: element i occupies stream bits
    [bits*i, bits*i + bits), stream bit k being bit (k mod 8) of byte floor(k / 8)."""
    v = np.asarray(values, dtype=np.int64)
    n = v.shape[-1]
    stream = ((v[..., :, None] >> np.arange(bits)) & 1).astype(np.uint8)
    stream = stream.reshape(*v.shape[:-1], n * bits)
    return np.packbits(stream, axis=-1, bitorder="little")


def _pack_k_chunk(fmt: str, elems: np.ndarray, d: int) -> np.ndarray:
    """Stored K elements [16 tokens, D] -> one K chunk (bytes), the header's layout."""
    if fmt == "bf16":     # [D/8][16][8] bf16
        x = np.asarray(elems, dtype=np.uint16).reshape(BLOCK, d // 8, 8).transpose(1, 0, 2)
        return np.ascontiguousarray(x).view(np.uint8).reshape(-1)
    if elem_kind(fmt, "k") == "fp8":      # [D/16][16][16] bytes (FP8 and Turbo8)
        x = np.asarray(elems, dtype=np.uint8).reshape(BLOCK, d // 16, 16).transpose(1, 0, 2)
        return np.ascontiguousarray(x).reshape(-1)
    kbits = _FMT_BITS[fmt][0]
    groups = np.asarray(elems).reshape(BLOCK, d // 32, 32).transpose(1, 0, 2)   # [D/32][16][32]
    return np.ascontiguousarray(pack_le(groups, kbits)).reshape(-1)


def _pack_v_chunk(fmt: str, elems: np.ndarray, d: int) -> np.ndarray:
    """Stored V elements [16 tokens, D] -> one V chunk, transposed [D][16]."""
    t = np.ascontiguousarray(np.asarray(elems).T)                 # [D][16]
    if fmt == "bf16":
        return t.astype(np.uint16).view(np.uint8).reshape(-1)
    if fmt == "fp8":
        return t.astype(np.uint8).reshape(-1)
    return np.ascontiguousarray(pack_le(t, 4)).reshape(-1)


def encode_tokens(fmt: str, which: str, x: np.ndarray, *, hk=None, hkv=None, scales=None,
                  codebook=None, sign=None):
    """Token vectors x [n, D] of one KV head hk (of hkv) -> (stored elements [n, D], norms [n]
    or None)."""
    kind = elem_kind(fmt, which)
    if kind == "bf16":
        return bf16_encode(x).astype(np.int64), None
    if kind == "fp8":
        sc = np.float32(fp8_scale(fmt, np.asarray(scales, dtype=np.float32), which, hk, hkv))
        return fp8_encode(x, sc).astype(np.int64), None
    cb = np.asarray(codebook, dtype=np.float32)
    if fmt == "turbo8":                   # the codebook is the 16 V levels
        return turbo_encode(x, sign, cb[:16])
    wi = 0 if which == "k" else 1
    bits = _FMT_BITS[fmt][wi]
    kl = 1 << _FMT_BITS[fmt][0]
    levels = cb[:kl] if which == "k" else cb[kl: kl + (1 << bits)]
    return turbo_encode(x, sign, levels)


def append_tokens(fmt: str, k_new, v_new, block_table, positions, k_cache, v_cache, scales,
                  codebook=None, sign=None):
    """Write new tokens into copies of the paged caches.

    k_new, v_new: fp32 [B][T][Hkv][D]; new token i of sequence b is token positions[b] + i,
    stored in page block_table[b][(positions[b] + i) // 16], slot (positions[b] + i) % 16.
    Tokens whose page index lies past the block table row, or whose page id lies outside the
    pool, are skipped.  Returns (k_cache, v_cache, scales); for the rotated formats each
    per-token norm goes to its slot of the 16 fp32 values after the chunk's indices (scales,
    read for FP8 and Turbo8 K, is returned unchanged)."""
    k_cache = np.array(k_cache, copy=True)
    v_cache = np.array(v_cache, copy=True)
    scales = None if scales is None else np.array(scales, copy=True)
    k_new = np.asarray(k_new, dtype=np.float32)
    v_new = np.asarray(v_new, dtype=np.float32)
    B, T, Hkv, d = k_new.shape
    pool = k_cache.shape[0]
    for b in range(B):
        for i in range(T):
            tok = int(positions[b]) + i
            if tok < 0 or tok // BLOCK >= len(block_table[b]):
                continue
            phys = int(block_table[b][tok // BLOCK])
            slot = tok % BLOCK
            if phys < 0 or phys >= pool:
                continue
            for hk in range(Hkv):
                for which, src, cache in (("k", k_new, k_cache), ("v", v_new, v_cache)):
                    el, norm = encode_tokens(fmt, which, src[b, i, hk][None, :], hk=hk,
                                             hkv=Hkv, scales=scales, codebook=codebook,
                                             sign=sign)
                    chunk = np.ascontiguousarray(cache[phys, hk])
                    read = _page_elems_k if which == "k" else _page_elems_v
                    pack = _pack_k_chunk if which == "k" else _pack_v_chunk
                    elems = np.array(read(fmt, chunk, d), dtype=np.int64)
                    elems[slot] = el[0]
                    c = code_bytes(fmt, which, d)
                    cache[phys, hk, :c] = pack(fmt, elems, d)
                    if norm is not None:    # fp32 little-endian, after the indices
                        off = c + 4 * slot
                        cache[phys, hk, off: off + 4] = np.array([norm[0]], "<f4").view(np.uint8)
    return k_cache, v_cache, scales
