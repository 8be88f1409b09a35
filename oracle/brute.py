"""Brute-force decode attention in pure-Python ``decimal`` arithmetic (40 digits), for tiny inputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/attention.py``).  It pins the fp64 oracle: every cache
element is located by its byte offset, written out from the layout the header documents
(no reshapes), decoded by scalar bit arithmetic, rotated back with Hadamard entries
H[i][j] = (-1)^popcount(i & j) (not the Sylvester recursion the oracle uses), and the softmax
is taken with ``Decimal.exp``.  Scalar loops only: token -> page -> slot -> element.
"""
from __future__ import annotations

import struct
from decimal import Decimal, getcontext

getcontext().prec = 40
BLOCK = 16


def _bf16(b0: int, b1: int) -> Decimal:
    bits = (b1 << 8) | b0                       # little-endian 16-bit word
    return Decimal(struct.unpack("<f", struct.pack("<I", bits << 16))[0])


def _e4m3(code: int) -> Decimal:
    sign = -1 if code >> 7 else 1
    exp = (code >> 3) & 15
    man = code & 7
    if exp == 15 and man == 7:
        return Decimal("NaN")
    if exp == 0:
        return sign * Decimal(man) / 8 * Decimal(2) ** -6
    return sign * (1 + Decimal(man) / 8) * Decimal(2) ** (exp - 7)


def _f32(x) -> Decimal:
    return Decimal(float(x))


def _bits_le(chunk_bytes, bit0: int, nbits: int) -> int:
    v = 0
    for i in range(nbits):
        k = bit0 + i
        v |= ((int(chunk_bytes[k // 8]) >> (k % 8)) & 1) << i
    return v


def _k_elem(fmt, kc, phys, hk, nkv, slot, d, D):
    if fmt == "bf16":
        base = (phys * nkv + hk) * 32 * D
        off = base + (((d // 8) * BLOCK + slot) * 8 + d % 8) * 2
        return ("v", _bf16(int(kc[off]), int(kc[off + 1])))
    if fmt in ("fp8", "turbo8"):               # Turbo8 K is stored exactly as FP8 K
        base = (phys * nkv + hk) * 16 * D
        return ("v", _e4m3(int(kc[base + ((d // 16) * BLOCK + slot) * 16 + d % 16])))
    bits = 4 if fmt == "turbo4" else 3
    gbytes = 4 * bits                           # 32 indices per group
    base = (phys * nkv + hk) * ((D // 32) * BLOCK * gbytes + 4 * BLOCK)   # + 16 fp32 norms
    grp = base + ((d // 32) * BLOCK + slot) * gbytes
    return ("i", _bits_le(kc[grp: grp + gbytes], (d % 32) * bits, bits))


def _v_elem(fmt, vc, phys, hk, nkv, slot, d, D):
    if fmt == "bf16":
        off = (phys * nkv + hk) * 32 * D + (d * BLOCK + slot) * 2
        return ("v", _bf16(int(vc[off]), int(vc[off + 1])))
    if fmt == "fp8":
        return ("v", _e4m3(int(vc[(phys * nkv + hk) * 16 * D + d * BLOCK + slot])))
    row = (phys * nkv + hk) * (8 * D + 4 * BLOCK) + d * 8     # chunk: 8 D index bytes, 16 norms
    return ("i", _bits_le(vc[row: row + 8], slot * 4, 4))


def _norm(fmt, which, cache_flat, phys, hk, nkv, slot, D):
    """The fp32 norm of token `slot`, stored after the index bytes of its (page, KV head) chunk
    (little-endian)."""
    codes = (D * 4 if fmt == "turbo4" else D * 3) * 2 if which == "k" else 8 * D
    off = (phys * nkv + hk) * (codes + 4 * BLOCK) + codes + 4 * slot
    return Decimal(struct.unpack("<f", bytes(int(cache_flat[off + i]) for i in range(4)))[0])


def _hadamard_entry(i: int, j: int) -> int:
    return -1 if bin(i & j).count("1") % 2 else 1


def _token_vector(fmt, which, cache_flat, phys, hk, nkv, slot, D, scales, codebook, sign):
    get = _k_elem if which == "k" else _v_elem
    wi = 0 if which == "k" else 1
    raw = [get(fmt, cache_flat, phys, hk, nkv, slot, d, D) for d in range(D)]
    if fmt == "bf16":
        return [x for _, x in raw]
    if fmt == "fp8":
        s = _f32(scales[wi][hk])
        return [x * s for _, x in raw]
    if fmt == "turbo8" and which == "k":       # K scale of head hk: scales = [Hkv]
        s = _f32(scales.reshape(-1)[hk])
        return [x * s for _, x in raw]
    levels = [_f32(c) for c in codebook]
    if fmt == "turbo8":                        # the 16 V levels
        table = levels[:16]
    else:
        kbits = 4 if fmt == "turbo4" else 3
        table = levels[: 1 << kbits] if which == "k" else levels[1 << kbits: (1 << kbits) + 16]
    norm = _norm(fmt, which, cache_flat, phys, hk, nkv, slot, D)
    rot = [norm * table[i] for _, i in raw]
    root = Decimal(D).sqrt()
    return [_f32(sign[d]) * sum(_hadamard_entry(d, e) * rot[e] for e in range(D)) / root
            for d in range(D)]


def _tanh(x: Decimal) -> Decimal:
    e = (2 * x).exp()
    return (e - 1) / (e + 1)


def brute_decode_attention(q_bits, k_cache, v_cache, block_table, context_lens, fmt, scales,
                           codebook, sign, softmax_scale, window, softcap, num_kv_heads,
                           head_dim, alibi=None):
    """Nested lists out[b][h][d] of Decimal.  ``alibi``: per-query-head slopes or None."""
    B, Hq, D = len(q_bits), len(q_bits[0]), head_dim
    g = Hq // num_kv_heads
    kc = k_cache.reshape(-1)
    vc = v_cache.reshape(-1)
    scale = _f32(softmax_scale)
    cap = _f32(softcap)
    out = []
    for b in range(B):
        L = int(context_lens[b])
        W = 0 if window is None else int(window[b])
        start = max(0, L - W) if W > 0 else 0
        keys, vals = {}, {}
        for j in range(start, L):
            phys = int(block_table[b][j // BLOCK])
            slot = j % BLOCK
            for hk in range(num_kv_heads):
                keys[hk, j] = _token_vector(fmt, "k", kc, phys, hk, num_kv_heads, slot, D,
                                            scales, codebook, sign)
                vals[hk, j] = _token_vector(fmt, "v", vc, phys, hk, num_kv_heads, slot, D,
                                            scales, codebook, sign)
        rows = []
        for h in range(Hq):
            hk = h // g
            if L == 0:
                rows.append([Decimal(0)] * D)
                continue
            qv = [_bf16(int(q_bits[b][h][d]) & 0xFF, int(q_bits[b][h][d]) >> 8) for d in range(D)]
            z = {}
            for j in range(start, L):
                x = scale * sum(qv[d] * keys[hk, j][d] for d in range(D))
                if cap > 0:
                    x = cap * _tanh(x / cap)
                if alibi is not None:
                    x += _f32(alibi[h]) * (j - (L - 1))
                z[j] = x
            m = max(z.values())
            p = {j: (z[j] - m).exp() for j in z}
            den = sum(p.values())
            rows.append([sum(p[j] * vals[hk, j][d] for j in z) / den for d in range(D)])
        out.append(rows)
    return out


def brute_multi_query(q_bits, k_cache, v_cache, block_table, context_lens, fmt, scales, codebook,
                      sign, softmax_scale, window, softcap, num_kv_heads, head_dim, alibi=None):
    """Chunk of n_q queries per sequence (q_bits nested [B][n_q][Hq][D]): query i at position
    p = L - n_q + i takes the keys j with lo <= j <= p, lo = p + 1 - W under a window W (else 0),
    and adds alibi[h] * (j - p) after the cap.  Nested lists out[b][i][h][d] of Decimal."""
    B, n_q, Hq, D = len(q_bits), len(q_bits[0]), len(q_bits[0][0]), head_dim
    g = Hq // num_kv_heads
    kc = k_cache.reshape(-1)
    vc = v_cache.reshape(-1)
    scale = _f32(softmax_scale)
    cap = _f32(softcap)
    out = []
    for b in range(B):
        L = int(context_lens[b])
        W = 0 if window is None else int(window[b])
        cache_k, cache_v = {}, {}

        def key(hk, j):
            if (hk, j) not in cache_k:
                phys = int(block_table[b][j // BLOCK])
                cache_k[hk, j] = _token_vector(fmt, "k", kc, phys, hk, num_kv_heads, j % BLOCK, D,
                                               scales, codebook, sign)
                cache_v[hk, j] = _token_vector(fmt, "v", vc, phys, hk, num_kv_heads, j % BLOCK, D,
                                               scales, codebook, sign)
            return cache_k[hk, j], cache_v[hk, j]

        seq = []
        for i in range(n_q):
            rows = []
            for h in range(Hq):
                if L == 0:
                    rows.append([Decimal(0)] * D)
                    continue
                hk = h // g
                pos = L - n_q + i
                lo = max(0, pos + 1 - W) if W > 0 else 0
                qv = [_bf16(int(q_bits[b][i][h][d]) & 0xFF, int(q_bits[b][i][h][d]) >> 8)
                      for d in range(D)]
                z = {}
                for j in range(lo, pos + 1):
                    kj = key(hk, j)[0]
                    x = scale * sum(qv[d] * kj[d] for d in range(D))
                    if cap > 0:
                        x = cap * _tanh(x / cap)
                    if alibi is not None:
                        x += _f32(alibi[h]) * (j - pos)
                    z[j] = x
                m = max(z.values())
                p = {j: (z[j] - m).exp() for j in z}
                den = sum(p.values())
                rows.append([sum(p[j] * key(hk, j)[1][d] for j in z) / den for d in range(D)])
            seq.append(rows)
        out.append(seq)
    return out
