"""Oracle: plain, slow fp64 CPU definition of single-query decode attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check in ``__graft_entry__`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with the GPU
library: it reads the paged layout, decodes FP8 and the rotated codebook format, rotates back
and computes softmax(q K^T * scale) V on its own, in float64.

What it follows (page titles and sections of the source pages):
  * attention.rs README, "KV Cache Formats": the formats BF16, FP8 (E4M3), Turbo8 (FP8 K +
    4-bit V, Walsh-Hadamard), Turbo4 (4-bit K + 4-bit V, Walsh-Hadamard) and Turbo3 (3-bit K +
    4-bit V); the Split-K paragraph below that
    table: long contexts are split (from 1024 tokens on) and the pieces are merged by a float
    reduce; "Features": softcapping, sliding window, GQA/MQA, paged block tables, causal mask.
  * turboquant-rs 0.4.1 src/cache/cuda/attention.rs: ``PARTITION_SIZE = 512`` and
    ``num_partitions = ceil(kv_len / 512)``; per-partition max, sum and output buffers; the
    all-zero output when ``kv_len == 0``; the kernel reads the compressed cache with a sign
    pattern and a codebook.

Readings taken where the pages are silent (the header of the library states the same ones):
  * window W: the query sees keys j in [L - W, L) (the W most recent, itself included);
  * softcap c > 0: logit x = scale * q.k is replaced by c * tanh(x / c) before the softmax;
  * GQA: query head h reads KV head floor(h / (Hq / Hkv));
  * ALiBi (the "ALiBi slopes" feature of the attention.rs README): query head h at position
    L - 1 adds slope_h * (j - (L - 1)) to its logit for key j, after the softcap;
  * rotated codebook: stored vector = norm * codebook[idx] in the rotated domain; the original
    vector is diag(s) H (that) / sqrt(D), H the Sylvester-order Hadamard matrix; the 16 fp32
    per-token norms of a page follow its index bytes inside the (page, KV head) chunk;
  * FP8 is OCP E4M3FN (bias 7, max 448, S.1111.111 = NaN) times one fp32 scale per KV head;
  * Turbo8 = K exactly as the FP8 format stores it (one scale per KV head, not rotated) and V
    exactly as Turbo4 stores it (rotated 4-bit codebook with per-token norms).  Its scale array
    is the [Hkv] K scales; its codebook is the 16 V levels.

Everything here is fp64; bf16 / fp8 / codebook values are widened exactly.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 16
_FMT_BITS = {"turbo4": (4, 4), "turbo3": (3, 4)}   # codebook K and V bits


def elem_kind(fmt: str, which: str) -> str:
    """How K or V of a format is stored: 'bf16', 'fp8' (E4M3FN code, per-head scale) or 'cb'
    (rotated-codebook index, per-token norm)."""
    if fmt == "bf16":
        return "bf16"
    if fmt == "fp8" or (fmt == "turbo8" and which == "k"):
        return "fp8"
    return "cb"


def fp8_scale(fmt: str, scales, which: str, hk: int, hkv: int):
    """The fp32 dequantisation scale of an FP8-stored K or V of KV head hk (of hkv)."""
    sc = np.asarray(scales)
    if fmt == "turbo8":                      # [Hkv]: the K scales
        return sc.reshape(-1)[hk]
    return sc[0 if which == "k" else 1, hk]


def code_bytes(fmt: str, which: str, d: int) -> int:
    """Bytes of stored elements at the start of one (page, KV head) chunk: 16 tokens x D
    elements of 16 (bf16), 8 (fp8) or 4 / 3 (codebook index) bits."""
    kind = elem_kind(fmt, which)
    if kind == "bf16":
        return 32 * d
    if kind == "fp8":
        return 16 * d
    bits = _FMT_BITS[fmt][0] if which == "k" and fmt in _FMT_BITS else 4
    return 2 * bits * d


def chunk_norms(fmt: str, which: str, cache: np.ndarray, d: int) -> np.ndarray:
    """The per-token norms [pool][Hkv][16] of a codebook-stored K or V: 16 little-endian fp32
    values right after each chunk's index bytes."""
    c = code_bytes(fmt, which, d)
    raw = np.ascontiguousarray(np.asarray(cache)[:, :, c: c + 4 * BLOCK])
    return raw.view("<f4").reshape(cache.shape[0], cache.shape[1], BLOCK)


# --------------------------------------------------------------------------------------------
# Scalar decoders
# --------------------------------------------------------------------------------------------
def e4m3fn_value(code: int) -> float:
    """OCP E4M3FN code -> value: (-1)^s 2^(e-7) (1 + m/8) for e > 0, (-1)^s 2^-6 (m/8) for
    e = 0; e = 15 and m = 7 is NaN (there is no infinity)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact)."""
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def sylvester_hadamard(n: int) -> np.ndarray:
    """Sylvester-order Hadamard matrix: H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    assert h.shape[0] == n, "n must be a power of two"
    return h


def unpack_le(buf: np.ndarray, bits: int) -> np.ndarray:
    """Little-endian bitstream unpack: element i of ``buf[..., nbytes]`` is bits
    [bits*i, bits*i + bits) where stream bit k is bit (k mod 8) of byte floor(k / 8)."""
    stream = np.unpackbits(np.asarray(buf, dtype=np.uint8), axis=-1, bitorder="little")
    n = stream.shape[-1] // bits
    groups = stream[..., : n * bits].reshape(*stream.shape[:-1], n, bits).astype(np.int64)
    return (groups << np.arange(bits, dtype=np.int64)).sum(axis=-1)


# --------------------------------------------------------------------------------------------
# Gather: logical token vectors of one (sequence, KV head) out of the paged cache
# --------------------------------------------------------------------------------------------
def _page_elems_k(fmt: str, chunk: np.ndarray, d: int) -> np.ndarray:
    """One K chunk (uint8 bytes) -> stored elements [16 tokens, D] (bf16 bits / fp8 codes /
    codebook indices), reading the layout the header documents."""
    chunk = chunk[: code_bytes(fmt, "k", d)]
    if fmt == "bf16":     # [D/8][16 tokens][8] bf16
        x = chunk.view(np.uint16).reshape(d // 8, BLOCK, 8)
        return x.transpose(1, 0, 2).reshape(BLOCK, d)
    if elem_kind(fmt, "k") == "fp8":   # [D/16][16 tokens][16] bytes
        x = chunk.reshape(d // 16, BLOCK, 16)
        return x.transpose(1, 0, 2).reshape(BLOCK, d)
    kbits = _FMT_BITS[fmt][0]
    xb = 32 * kbits // 8  # bytes per 32-index group
    x = chunk.reshape(d // 32, BLOCK, xb)             # [D/32][16 tokens][xb]
    idx = unpack_le(x, kbits)                         # [D/32][16][32]
    return idx.transpose(1, 0, 2).reshape(BLOCK, d)


def _page_elems_v(fmt: str, chunk: np.ndarray, d: int) -> np.ndarray:
    """One V chunk -> stored elements [16 tokens, D]; V is stored transposed, [D][16]."""
    chunk = chunk[: code_bytes(fmt, "v", d)]
    if fmt == "bf16":
        return chunk.view(np.uint16).reshape(d, BLOCK).T
    if fmt == "fp8":
        return chunk.reshape(d, BLOCK).T
    return unpack_le(chunk.reshape(d, BLOCK // 2), 4).T   # 16 nibbles per row


def gather_stored(fmt: str, which: str, cache: np.ndarray, block_table_row: np.ndarray,
                  hk: int, t0: int, t1: int, d: int) -> np.ndarray:
    """Stored elements of tokens [t0, t1) of one sequence's KV head: [n, D] (int64)."""
    out = np.empty((t1 - t0, d), dtype=np.int64)
    take = _page_elems_k if which == "k" else _page_elems_v
    for pg in range(t0 // BLOCK, (t1 - 1) // BLOCK + 1 if t1 > t0 else t0 // BLOCK):
        phys = int(block_table_row[pg])
        elems = take(fmt, np.ascontiguousarray(cache[phys, hk]), d)
        lo, hi = max(t0, pg * BLOCK), min(t1, (pg + 1) * BLOCK)
        out[lo - t0: hi - t0] = elems[lo - pg * BLOCK: hi - pg * BLOCK]
    return out


def token_norms(fmt: str, which: str, cache: np.ndarray, block_table_row: np.ndarray, hk: int,
                t0: int, t1: int, d: int) -> np.ndarray:
    """Per-token fp32 norms of tokens [t0, t1) of a codebook-stored K or V (the 16 fp32 values
    after each chunk's index bytes), as float32."""
    j = np.arange(t0, t1)
    phys = np.asarray(block_table_row)[j // BLOCK]
    c = code_bytes(fmt, which, d)
    raw = np.ascontiguousarray(np.asarray(cache)[phys, hk, c: c + 4 * BLOCK])
    return raw.view("<f4").reshape(len(j), BLOCK)[np.arange(len(j)), j % BLOCK]


def unrotate(x_rot: np.ndarray, sign: np.ndarray) -> np.ndarray:
    """x = diag(s) H x_rot / sqrt(D): the inverse of x_rot = H diag(s) x / sqrt(D)."""
    d = x_rot.shape[-1]
    h = sylvester_hadamard(d).astype(np.float64)
    return (x_rot @ h.T) * np.asarray(sign, dtype=np.float64) / math.sqrt(d)


def codebooks(fmt: str, codebook: np.ndarray):
    """(K levels or None, V levels) of a codebook format, fp32."""
    cb = np.asarray(codebook, dtype=np.float32)
    if fmt == "turbo8":
        return None, cb[:16]
    kbits, _ = _FMT_BITS[fmt]
    return cb[: 1 << kbits], cb[1 << kbits: (1 << kbits) + 16]


def gather_kv(fmt: str, which: str, cache, block_table_row, hk, t0, t1, d, *, scales=None,
              codebook=None, sign=None) -> np.ndarray:
    """Logical (original-domain) K or V vectors of tokens [t0, t1): fp64 [n, D]."""
    stored = gather_stored(fmt, which, cache, block_table_row, hk, t0, t1, d)
    kind = elem_kind(fmt, which)
    pool, hkv = cache.shape[0], cache.shape[1]
    if kind == "bf16":
        return bf16_to_f64(stored)
    if kind == "fp8":
        return E4M3FN_TABLE[stored] * np.float64(np.float32(fp8_scale(fmt, scales, which, hk, hkv)))
    norms = token_norms(fmt, which, cache, block_table_row, hk, t0, t1, d).astype(np.float64)
    cb = codebooks(fmt, codebook)[0 if which == "k" else 1]
    return unrotate(norms[:, None] * cb.astype(np.float64)[stored], sign)


# --------------------------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------------------------
def attended_range(L: int, W: int) -> tuple[int, int]:
    """Keys a decode query at position L-1 sees: [L - W, L) with a window, else [0, L)."""
    return (max(0, L - W) if W > 0 else 0), L


def logits(q: np.ndarray, k: np.ndarray, softmax_scale, softcap, bias=None) -> np.ndarray:
    """z = scale * q K^T, then cap * tanh(z / cap) when cap > 0, then + bias [g, n] (the
    ALiBi term) when given (fp64; scale is the fp32 value the caller passes, widened)."""
    z = float(np.float32(softmax_scale)) * (q @ k.T)
    cap = float(np.float32(softcap))
    if cap > 0:
        z = cap * np.tanh(z / cap)
    if bias is not None:
        z = z + bias
    return z


def alibi_bias(slopes, L: int, t0: int, t1: int) -> np.ndarray:
    """slope_h * (j - (L - 1)) for keys j in [t0, t1): [g, n] fp64 (slopes fp32, widened)."""
    s = np.asarray(slopes, dtype=np.float32).astype(np.float64)
    return s[:, None] * (np.arange(t0, t1, dtype=np.float64) - (L - 1))[None, :]


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, softmax_scale, softcap, bias=None):
    """Exact softmax attention of query rows q [g, D] over keys k and values v [n, D].

    Returns (m, l, o): the max logit m [g], the sum l = sum_j exp(z_j - m) [g] and the
    normalised output o = sum_j exp(z_j - m) v_j / l [g, D].
    """
    z = logits(q, k, softmax_scale, softcap, bias)
    m = z.max(axis=1)
    p = np.exp(z - m[:, None])
    l = p.sum(axis=1)
    return m, l, (p @ v) / l[:, None]


def partitions(L: int, W: int, partition_size: int = 0) -> list[tuple[int, int]]:
    """Token ranges the split decode uses for one sequence.

    partition_size 0 (auto): 512-token partitions when the attended span is >= 1024, else one
    range; > 0: always partitions of that size; -1: never split.  Partition boundaries sit at
    absolute multiples of the size, intersected with the attended range; empty ones dropped.
    """
    lo, hi = attended_range(L, W)
    if hi <= lo:
        return []
    if partition_size == -1 or (partition_size == 0 and hi - lo < 1024):
        return [(lo, hi)]
    ps = 512 if partition_size == 0 else partition_size
    return [(max(lo, p * ps), min(hi, (p + 1) * ps)) for p in range(lo // ps, (hi - 1) // ps + 1)]


def lse_merge(ms, ls, os_):
    """Merge per-partition (m_p, l_p, o_p) triples: w_p = l_p exp(m_p - M), o = sum w_p o_p / sum w_p."""
    ms = np.asarray(ms, dtype=np.float64)
    M = ms.max(axis=0)
    w = np.asarray(ls, dtype=np.float64) * np.exp(ms - M)
    return np.einsum("pg,pgd->gd", w, np.asarray(os_, dtype=np.float64)) / w.sum(axis=0)[:, None]


def _q_rows(q_bits, b, h0, g):
    return bf16_to_f64(np.asarray(q_bits)[b, h0: h0 + g])


# Memory bound of the oracle: the keys of one (sequence, KV head) are gathered at most this many
# at a time.  One block's K and V in fp64 take 2 * 65536 * D * 8 bytes (128 MiB at D = 128), so
# every context up to 64K keys is computed in one piece, as the plain definition reads; only
# longer ones are cut into blocks, whose (max, sum, output) triples the LSE rule merges -- the
# same sum in another order, which the split decode itself relies on (turboquant-rs fused
# attention: per-partition max / sum / output, then the reduce).
KEY_BLOCK = 1 << 16


def key_blocks(lo: int, hi: int, block: int) -> list[tuple[int, int]]:
    """Consecutive ranges [t0, t1) of at most ``block`` keys that tile [lo, hi) exactly."""
    return [(t0, min(hi, t0 + block)) for t0 in range(lo, hi, block)]


def decode_attention(q, k_cache, v_cache, block_table, context_lens, fmt, scales, codebook,
                     sign, softmax_scale, window, softcap, num_kv_heads, head_dim,
                     seqs=None, kv_heads=None, chunk=KEY_BLOCK, alibi=None):
    """out[b, h] = softmax(scale * q_h K^T) V over the attended keys of sequence b, fp64.

    q: bf16 bits [B, Hq, D]; caches in the paged layout; context_lens / window int [B]
    (window None -> no window); alibi: per-query-head slopes [Hq] or None.  Rows of sequences
    with context length 0 are zero.
    ``seqs`` / ``kv_heads`` restrict the work to a sample (other rows are left NaN).
    Keys are gathered ``chunk`` at a time (``key_blocks``); a range of at most ``chunk`` keys is
    one block and needs no merge, longer ranges are merged with the LSE rule.
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    g = Hq // num_kv_heads
    out = np.full((B, Hq, D), np.nan)
    win = np.zeros(B, dtype=np.int64) if window is None else np.asarray(window)
    for b in (range(B) if seqs is None else seqs):
        L = int(context_lens[b])
        lo, hi = attended_range(L, int(win[b]))
        for hk in (range(num_kv_heads) if kv_heads is None else kv_heads):
            rows = slice(hk * g, hk * g + g)
            if hi <= lo:
                out[b, rows] = 0.0
                continue
            qr = _q_rows(q, b, hk * g, g)
            parts = []
            for t0, t1 in key_blocks(lo, hi, chunk):
                kk = gather_kv(fmt, "k", k_cache, block_table[b], hk, t0, t1, D, scales=scales,
                               codebook=codebook, sign=sign)
                vv = gather_kv(fmt, "v", v_cache, block_table[b], hk, t0, t1, D, scales=scales,
                               codebook=codebook, sign=sign)
                bias = None if alibi is None else alibi_bias(np.asarray(alibi)[rows], L, t0, t1)
                parts.append(attend(qr, kk, vv, softmax_scale, softcap, bias))
            if len(parts) == 1:
                out[b, rows] = parts[0][2]
            else:
                ms, ls, os_ = zip(*parts)
                out[b, rows] = lse_merge(ms, ls, os_)
    return out


def partition_partials(q, k_cache, v_cache, block_table, context_lens, fmt, scales, codebook,
                       sign, softmax_scale, window, softcap, num_kv_heads, head_dim,
                       partition_size, b, hk, rotated=False, alibi=None):
    """Per-partition triples for one (sequence, KV head): list of (lo, hi, m [g], l [g], o [g, D]).

    rotated=True returns o in the storage (rotated) domain for the codebook formats, which is
    what the GPU's partial buffers hold.
    """
    q = np.asarray(q)
    g = q.shape[1] // num_kv_heads
    win = 0 if window is None else int(window[b])
    qr = _q_rows(q, b, hk * g, g)
    res = []
    for lo, hi in partitions(int(context_lens[b]), win, partition_size):
        kk = gather_kv(fmt, "k", k_cache, block_table[b], hk, lo, hi, head_dim, scales=scales,
                       codebook=codebook, sign=sign)
        vv = gather_kv(fmt, "v", v_cache, block_table[b], hk, lo, hi, head_dim, scales=scales,
                       codebook=codebook, sign=sign)
        bias = None
        if alibi is not None:
            bias = alibi_bias(np.asarray(alibi)[hk * g: hk * g + g], int(context_lens[b]), lo, hi)
        m, l, o = attend(qr, kk, vv, softmax_scale, softcap, bias)
        if rotated and fmt.startswith("turbo"):
            d = head_dim
            h = sylvester_hadamard(d).astype(np.float64)
            o = ((o * np.asarray(sign, np.float64)) @ h.T) / math.sqrt(d)
        res.append((lo, hi, m, l, o))
    return res


def dequant_gather(fmt, which, cache, scales, codebook, block_table_row, hk, t0, n, d):
    """Storage-domain dequantised values of tokens [t0, t0+n), as the library's float32 gather
    export defines them: bf16 widened; fp8 value * scale rounded to fp32; codebook formats
    norm * level rounded to fp32 (still rotated)."""
    stored = gather_stored(fmt, which, cache, block_table_row, hk, t0, t0 + n, d)
    kind = elem_kind(fmt, which)
    pool, hkv = cache.shape[0], cache.shape[1]
    if kind == "bf16":
        return bf16_to_f64(stored).astype(np.float32)
    if kind == "fp8":
        sc = np.float32(fp8_scale(fmt, scales, which, hk, hkv))
        return E4M3FN_TABLE[stored].astype(np.float32) * sc
    nrm = token_norms(fmt, which, cache, block_table_row, hk, t0, t0 + n, d)
    cb = codebooks(fmt, codebook)[0 if which == "k" else 1].astype(np.float32)
    return nrm[:, None] * cb[stored]
