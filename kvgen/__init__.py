"""Seeded synthetic inputs for single-query (decode) attention over a paged KV cache.

This module draws random numbers and lays them out in the cache format that the library's
header documents: Gaussian q/K/V rounded to bf16, the FP8-E4M3FN and rotated-codebook
*encoders* (the cache writer that runs before the decode path), the page-pool permutation,
block tables, context lengths and window choices.

It holds none of the decode arithmetic -- no gather through block tables, no dequantisation,
no rotation of the query, no softmax.  The oracle (``oracle/``) and the GPU library each
implement those on their own; this is the only module both sides share.

Workload shapes follow the attention.rs README (page "guoqingbao/attention.rs", section
"KV Cache Formats": BF16, FP8 E4M3, Turbo8 = FP8 K + 4-bit V, Turbo4 = 4-bit K + 4-bit V,
Turbo3 = 3-bit K + 4-bit V)
and the turboquant-rs fused attention wrapper (page "turboquant-rs 0.4.1
src/cache/cuda/attention.rs": 512-token partitions, sign pattern, codebook, per-token scales).
"""
from __future__ import annotations

import dataclasses
import functools
import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16          # tokens per page
FORMATS = ("bf16", "fp8", "turbo4", "turbo3", "turbo8")
FORMAT_CODE = {"bf16": 0, "fp8": 1, "turbo4": 2, "turbo3": 3, "turbo8": 4}
KV_BITS = {"turbo4": (4, 4), "turbo3": (3, 4)}   # (K bits, V bits) of the all-codebook formats


def k_is_fp8(fmt: str) -> bool:
    """K stored as E4M3FN codes with one fp32 scale per KV head (FP8 and Turbo8)."""
    return fmt in ("fp8", "turbo8")


def v_is_codebook(fmt: str) -> bool:
    """V stored as 4-bit rotated-codebook indices with per-token norms (the Turbo formats)."""
    return fmt in ("turbo4", "turbo3", "turbo8")

BF16_POISON = np.uint16(0x7FC0)   # quiet NaN
FP8_POISON = np.uint8(0x7F)       # E4M3FN NaN (S.1111.111)


# --------------------------------------------------------------------------------------------
# Workload specifications
# --------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Spec:
    """Shape and recipe of one synthetic decode-attention batch."""
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    fmt: str
    context: int | None = None            # every sequence has this length ...
    ctx_range: tuple[int, int] | None = None   # ... or lengths ~ U{lo..hi} from the seed
    window: int = 0                       # sliding-window width (0 = none)
    window_frac: float = 0.0              # fraction of sequences that get the window
    softcap: float = 0.0                  # tanh logit cap (0 = off)
    softmax_scale: float | None = None    # default 1/sqrt(head_dim)
    pool_spare: int = 1024                # spare (poisoned) pages beyond what the batch needs
    pool_total: int | None = None         # explicit pool size (overrides pool_spare)
    partition_size: int = 0               # 0 = auto (512, split at >= 1024 tokens)
    seed: int = 0
    queries_per_seq: int = 1              # > 1: a chunk of queries at the last positions

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> np.float32:
        s = self.softmax_scale if self.softmax_scale is not None else 1.0 / math.sqrt(self.head_dim)
        return np.float32(s)

    @property
    def max_context(self) -> int:
        return self.context if self.context is not None else self.ctx_range[1]


SPECS: dict[str, Spec] = {
    # Tiny parity case: GQA 4:1, D=64, L=300, 19 pages placed by a permutation of a 64-page pool.
    "c1": Spec("tiny-bf16-L300", 1, 4, 1, 64, "bf16", context=300, softmax_scale=1.0 / 8,
               pool_total=64),
    # Llama-3-8B-shaped decode at 4K context.
    "c2": Spec("llama3-8b-bf16-L4096", 32, 32, 8, 128, "bf16", context=4096),
    # Ragged long-context batch with sliding window on half the sequences and tanh softcap.
    "c3": Spec("ragged-bf16-L1..32768-win4096-cap50", 64, 32, 8, 128, "bf16",
               ctx_range=(1, 32768), window=4096, window_frac=0.5, softcap=50.0),
    # FP8 E4M3 cache at 32K, GQA 8:1.
    "c4": Spec("fp8-e4m3-L32768-gqa8", 16, 64, 8, 128, "fp8", context=32768),
    # Rotated-codebook caches at 64K.
    "c5-t4": Spec("turbo4-L65536", 8, 32, 8, 128, "turbo4", context=65536),
    "c5-t3": Spec("turbo3-L65536", 8, 32, 8, 128, "turbo3", context=65536),
    # 32K-context shapes for the other formats (the headline metric is stated at 32K).
    "m-bf16": Spec("bf16-L32768-gqa8", 16, 64, 8, 128, "bf16", context=32768),
    "m-t4": Spec("turbo4-L32768", 8, 32, 8, 128, "turbo4", context=32768),
    "m-t3": Spec("turbo3-L32768", 8, 32, 8, 128, "turbo3", context=32768),
    "m-t8": Spec("turbo8-L32768", 8, 32, 8, 128, "turbo8", context=32768),
    "c5-t8": Spec("turbo8-L65536", 8, 32, 8, 128, "turbo8", context=65536),
    # Short rotated-codebook contexts in a large batch: each sequence is one workgroup's walk,
    # so a decode call is one partition launch with no reduce.
    "s-t4": Spec("turbo4-L4096", 64, 32, 8, 128, "turbo4", context=4096),
    "s-t3": Spec("turbo3-L4096", 64, 32, 8, 128, "turbo3", context=4096),
    # Batches of 6 sequences at 32K (48 work units, which do not divide the device's workgroup
    # slots): the run choice fills one round of workgroups with whole run blocks.
    "b6-fp8": Spec("fp8-e4m3-L32768-b6", 6, 64, 8, 128, "fp8", context=32768),
    "b6-bf16": Spec("bf16-L32768-b6", 6, 64, 8, 128, "bf16", context=32768),
    "b6-t4": Spec("turbo4-L32768-b6", 6, 32, 8, 128, "turbo4", context=32768),
    # One sequence at 32K (8 work units): runs shorter than a partition fill the device.
    "b1-fp8": Spec("fp8-e4m3-L32768-b1", 1, 64, 8, 128, "fp8", context=32768),
    "b1-t4": Spec("turbo4-L32768-b1", 1, 32, 8, 128, "turbo4", context=32768),
    # A large batch (64 sequences at 32K, 512 units): runs capped at 8 partitions.
    "b64-fp8": Spec("fp8-e4m3-L32768-b64", 64, 64, 8, 128, "fp8", context=32768),
    # Chunks of queries (chunked prefill / multi-token decode) at 32K: n_q * group = 16 rows
    # per KV head fill one MFMA tile, so the cache is read once for all of them.
    "mq-fp8": Spec("fp8-e4m3-L32768-gqa8-q2", 16, 64, 8, 128, "fp8", context=32768,
                   queries_per_seq=2),
    # a longer chunk: 8 queries x 8 heads = 64 rows, four 16-row tiles per KV head
    "mq8-fp8": Spec("fp8-e4m3-L32768-gqa8-q8", 16, 64, 8, 128, "fp8", context=32768,
                    queries_per_seq=8),
    "mq-t4": Spec("turbo4-L32768-q4", 8, 32, 8, 128, "turbo4", context=32768, queries_per_seq=4),
    "mq-t3": Spec("turbo3-L32768-q4", 8, 32, 8, 128, "turbo3", context=32768, queries_per_seq=4),
    # Multi-query attention (one KV head for all 64 query heads) at 32K: four 16-row query
    # tiles read each KV head's pages.
    "mqa-fp8": Spec("fp8-e4m3-L32768-mqa64", 16, 64, 1, 128, "fp8", context=32768),
    "mqa-bf16": Spec("bf16-L32768-mqa64", 16, 64, 1, 128, "bf16", context=32768),
    "mqa-t4": Spec("turbo4-L32768-mqa64", 8, 64, 1, 128, "turbo4", context=32768),
    "mqa-t8": Spec("turbo8-L32768-mqa64", 8, 64, 1, 128, "turbo8", context=32768),
}


def spec(name: str, **overrides) -> Spec:
    """A named workload, optionally with fields replaced (smaller batch, other format, ...)."""
    return dataclasses.replace(SPECS[name], **overrides)


# --------------------------------------------------------------------------------------------
# Byte sizes of the paged layout (documented in include/kvdecode.h)
# --------------------------------------------------------------------------------------------
NORM_BYTES = 4 * BLOCK_SIZE   # the 16 fp32 per-token norms after a codebook chunk's indices


def k_code_bytes(fmt: str, d: int) -> int:
    """Bytes of stored K elements at the start of one (page, KV head) chunk."""
    return {"bf16": 32 * d, "fp8": 16 * d, "turbo4": 8 * d, "turbo3": 6 * d, "turbo8": 16 * d}[fmt]


def v_code_bytes(fmt: str, d: int) -> int:
    """Bytes of stored V elements at the start of one chunk (Turbo V is always 4-bit)."""
    return {"bf16": 32 * d, "fp8": 16 * d, "turbo4": 8 * d, "turbo3": 8 * d, "turbo8": 8 * d}[fmt]


def k_chunk_bytes(fmt: str, d: int) -> int:
    """Bytes of one (page, KV head) chunk of the K cache (codebook K: indices, then norms)."""
    return k_code_bytes(fmt, d) + (NORM_BYTES if fmt in KV_BITS else 0)


def v_chunk_bytes(fmt: str, d: int) -> int:
    """Bytes of one (page, KV head) chunk of the V cache (codebook V: indices, then norms)."""
    return v_code_bytes(fmt, d) + (NORM_BYTES if v_is_codebook(fmt) else 0)


def kv_bytes_per_token_head(fmt: str, d: int) -> int:
    """Algorithmic cache bytes the method must read per (token, KV head), K + V (norms
    included)."""
    return (k_chunk_bytes(fmt, d) + v_chunk_bytes(fmt, d)) // BLOCK_SIZE


# --------------------------------------------------------------------------------------------
# Scalar encoders (cache writer side)
# --------------------------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_POISON
    return out


def e4m3fn_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP FP8 E4M3FN codes: round to nearest even, saturate to +-448.

    E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; S.1111.111 is NaN, there is no
    infinity, the largest finite value is 1.75 * 2^8 = 448 and the smallest subnormal 2^-9.
    """
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    sign = ((bits >> np.uint32(24)) & np.uint32(0x80)).astype(np.uint8)
    # |x| clamped to 448 (0x43E00000); for non-negative floats bit order is value order
    a = np.minimum(bits & np.uint32(0x7FFFFFFF), np.uint32(0x43E00000))
    # normal range: round the 23-bit mantissa to 3 bits (ties to even); a carry bumps the
    # exponent; then rebias 127 -> 7
    r = a >> np.uint32(20)
    r &= np.uint32(1)
    r += a
    r += np.uint32(0x7FFFF)
    r >>= np.uint32(20)
    r -= np.uint32((127 - 7) << 3)
    # subnormal range (|x| < 2^-6): multiples of 2^-9; 8 * 2^-9 is the smallest normal, 0x08
    small = a < np.uint32(0x3C800000)
    if small.any():
        r[small] = np.rint(a[small].view(np.float32) * np.float32(512.0)).astype(np.uint32)
    code = r.astype(np.uint8)
    code |= sign
    return code


def sign_pattern(rng: np.random.Generator, d: int) -> np.ndarray:
    """A seeded +-1 vector (float32)."""
    return np.where(rng.integers(0, 2, size=d) == 1, 1.0, -1.0).astype(np.float32)


def _wht_rows(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform (Sylvester order) along the last axis, in place."""
    d = x.shape[-1]
    h = 1
    lead = x.shape[:-1]
    while h < d:
        y = x.reshape(*lead, d // (2 * h), 2, h)
        a = y[..., 0, :].copy()
        b = y[..., 1, :]
        y[..., 0, :] += b
        y[..., 1, :] = a - b
        h *= 2
    return x


@functools.lru_cache(maxsize=None)
def lloyd_max_normal(levels: int) -> tuple[float, ...]:
    """Lloyd-Max levels (ascending, fp64) minimising MSE for a standard normal source.

    Fixed point of: boundaries are midpoints of neighbouring levels; each level is the
    conditional mean of N(0,1) on its cell, E[X | a<X<b] = (phi(a)-phi(b)) / (Phi(b)-Phi(a)).
    """
    from scipy.special import ndtr

    def phi(t):
        return np.exp(-0.5 * t * t) / math.sqrt(2.0 * math.pi)

    c = np.linspace(-2.5, 2.5, levels)
    for _ in range(100000):
        b = np.concatenate(([-np.inf], 0.5 * (c[1:] + c[:-1]), [np.inf]))
        lo, hi = b[:-1], b[1:]
        new = (phi(lo) - phi(hi)) / (ndtr(hi) - ndtr(lo))
        new = 0.5 * (new - new[::-1])          # the source is symmetric; keep the levels so
        done = np.max(np.abs(new - c)) < 4e-15
        c = new
        if done:
            break
    return tuple(float(v) for v in c)


def codebook(levels: int, d: int) -> np.ndarray:
    """Lloyd-Max codebook for a coordinate of a random unit vector in R^d, i.e. N(0, 1/d),
    rounded to float32, ascending."""
    return (np.asarray(lloyd_max_normal(levels)) / math.sqrt(d)).astype(np.float32)


def nearest_level(u: np.ndarray, levels_f32: np.ndarray) -> np.ndarray:
    """Index of the nearest codebook level (ties to the lower index), decided in fp64."""
    lv = levels_f32.astype(np.float64)
    mids = 0.5 * (lv[1:] + lv[:-1])
    return np.searchsorted(mids, u, side="left").astype(np.uint8)


def turbo_encode(x: np.ndarray, sign: np.ndarray, levels_f32: np.ndarray):
    """Rotated-codebook encoder for token vectors x [..., d] (float32).

    y = H_d (s * x) / sqrt(d) (orthonormal Walsh-Hadamard after a +-1 sign flip);
    norm = ||x||_2 (fp64, rounded to fp32); u = y / norm; idx = nearest level of u.
    Returns (idx uint8 [..., d], norm float32 [...]).
    """
    d = x.shape[-1]
    xd = x.astype(np.float64)
    y = _wht_rows(xd * sign.astype(np.float64)) / math.sqrt(d)
    norm = np.sqrt(np.einsum("...i,...i->...", xd, xd)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        u = y / norm.astype(np.float64)[..., None]
    u = np.nan_to_num(u, nan=0.0)
    return nearest_level(u, levels_f32), norm


# --------------------------------------------------------------------------------------------
# Page packing (layout of one (page, KV head) chunk; see include/kvdecode.h)
# --------------------------------------------------------------------------------------------
def _pack_nibbles(idx: np.ndarray) -> np.ndarray:
    """[..., 2n] 4-bit values -> [..., n] bytes, element 2i in the low nibble of byte i."""
    idx = idx.astype(np.uint8)
    return (idx[..., 0::2] & 0xF) | ((idx[..., 1::2] & 0xF) << 4)


def _pack_3bit(idx: np.ndarray) -> np.ndarray:
    """[..., 32] 3-bit values -> [..., 12] bytes; value e occupies bits [3e, 3e+3) of the
    little-endian 96-bit word formed by the 12 bytes."""
    v = idx.astype(np.uint64) & np.uint64(7)
    lo = np.zeros(v.shape[:-1], dtype=np.uint64)      # bits 0..63
    hi = np.zeros(v.shape[:-1], dtype=np.uint64)      # bits 64..95
    for e in range(32):
        bit = 3 * e
        ve = v[..., e]
        if bit + 3 <= 64:
            lo |= ve << np.uint64(bit)
        elif bit >= 64:
            hi |= ve << np.uint64(bit - 64)
        else:   # straddles bit 64
            lo |= (ve << np.uint64(bit)) & np.uint64(0xFFFFFFFFFFFFFFFF)
            hi |= ve >> np.uint64(64 - bit)
    out = np.empty(v.shape[:-1] + (12,), dtype=np.uint8)
    for i in range(8):
        out[..., i] = ((lo >> np.uint64(8 * i)) & np.uint64(0xFF)).astype(np.uint8)
    for i in range(4):
        out[..., 8 + i] = ((hi >> np.uint64(8 * i)) & np.uint64(0xFF)).astype(np.uint8)
    return out


def pack_k_pages(fmt: str, elems: np.ndarray) -> np.ndarray:
    """K elements [n_pages, Hkv, 16, D] (bf16 bits / fp8 codes / codebook indices) ->
    page chunks [n_pages, Hkv, k_chunk_bytes] (uint8)."""
    n, h, t, d = elems.shape
    if fmt == "bf16":      # [D/8][16][8] bf16
        c = elems.astype(np.uint16).reshape(n, h, t, d // 8, 8).transpose(0, 1, 3, 2, 4)
        return np.ascontiguousarray(c).view(np.uint8).reshape(n, h, -1)
    if k_is_fp8(fmt):      # [D/16][16][16] bytes
        c = elems.astype(np.uint8).reshape(n, h, t, d // 16, 16).transpose(0, 1, 3, 2, 4)
        return np.ascontiguousarray(c).reshape(n, h, -1)
    groups = elems.reshape(n, h, t, d // 32, 32).transpose(0, 1, 3, 2, 4)   # [D/32][16][32]
    packed = _pack_nibbles(groups) if fmt == "turbo4" else _pack_3bit(groups)
    return np.ascontiguousarray(packed).reshape(n, h, -1)


def pack_v_pages(fmt: str, elems: np.ndarray) -> np.ndarray:
    """V elements [n_pages, Hkv, 16, D] -> page chunks [n_pages, Hkv, v_chunk_bytes] (uint8);
    V is stored transposed, [D][16] per chunk (4-bit for both Turbo formats)."""
    n, h, t, d = elems.shape
    c = np.ascontiguousarray(elems.transpose(0, 1, 3, 2))          # [n, h, D, 16]
    if fmt == "bf16":
        return c.astype(np.uint16).view(np.uint8).reshape(n, h, -1)
    if fmt == "fp8":
        return c.astype(np.uint8).reshape(n, h, -1)
    return np.ascontiguousarray(_pack_nibbles(c)).reshape(n, h, -1)


# --------------------------------------------------------------------------------------------
# Batch generation
# --------------------------------------------------------------------------------------------
@dataclass
class Inputs:
    """One synthetic batch, host-side, exactly as the C ABI consumes it."""
    spec: Spec
    q: np.ndarray                 # uint16 [B, Hq, D] bf16 bits ([B, n_q, Hq, D] for n_q > 1)
    k_cache: np.ndarray           # uint8 [pool, Hkv, k_chunk_bytes]
    v_cache: np.ndarray           # uint8 [pool, Hkv, v_chunk_bytes]
    scales: np.ndarray | None     # fp8: f32 [2, Hkv]; turbo8: f32 [Hkv] K scales; else None
                                  # (codebook norms live inside the cache chunks);
                                  # bf16: None
    codebook: np.ndarray | None   # turbo4/3: f32 [2^kbits + 16] (K levels then V levels);
                                  # turbo8: f32 [16] (V levels)
    sign: np.ndarray | None       # turbo: f32 [D] of +-1
    block_table: np.ndarray       # int32 [B, max_blocks_per_seq]
    context_lens: np.ndarray      # int32 [B]
    window: np.ndarray            # int32 [B]; 0 = no window
    softmax_scale: np.float32
    softcap: np.float32
    max_context_len: int
    extra: dict = field(default_factory=dict)

    @property
    def num_pool_blocks(self) -> int:
        return self.k_cache.shape[0]

    @property
    def max_blocks_per_seq(self) -> int:
        return self.block_table.shape[1]

    def spans(self) -> np.ndarray:
        """Keys any query of a sequence attends to: min(L, W + n_q - 1) if windowed, else L
        (n_q = 1 for decode)."""
        L = self.context_lens.astype(np.int64)
        W = self.window.astype(np.int64)
        return np.where(W > 0, np.minimum(L, W + self.spec.queries_per_seq - 1), L)

    def kv_bytes(self) -> int:
        """Algorithmic cache bytes one call must read."""
        s = self.spec
        return int(self.spans().sum()) * s.num_kv_heads * kv_bytes_per_token_head(s.fmt, s.head_dim)


# Named child streams of one SeedSequence, in a fixed order.
_STREAMS = ("q", "k", "v", "pool", "lengths", "window", "sign")


def _rngs(seed: int) -> dict:
    """Generators of the named streams, plus the K / V SeedSequences ('k_seq', 'v_seq') whose
    per-sequence children draw the cache contents."""
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    out = {name: np.random.default_rng(k) for name, k in zip(_STREAMS, kids)}
    out["k_seq"], out["v_seq"] = kids[1], kids[2]
    return out


def make_inputs(s: Spec, *, poison: bool = True, poison_before_window: bool = False,
                unused_fill: str = "spare", kv_override=None,
                fp8_scale: np.ndarray | None = None, lengths: np.ndarray | None = None,
                windows: np.ndarray | None = None) -> Inputs:
    """Build one batch.

    poison: spare pages and tail slots past each context length hold NaN (bf16 0x7FC0,
        fp8 0x7F, codebook norm NaN), so any read that reaches the arithmetic shows up.
    poison_before_window: also poison pages that lie wholly before the first key any query of
        the sequence attends (L - W, or L - n_q + 1 - W for a chunk of n_q queries).
    unused_fill: block-table entries past a sequence's last page -> 'spare' (a poisoned spare
        page) or -1.
    kv_override: callable(seq, L) -> (K [Hkv, L, D], V [Hkv, L, D]) float32 logical values,
        replacing the Gaussian draws (identity tests).
    fp8_scale: optional f32 [2, Hkv] replacing amax/448 (Turbo8 uses the K row).
    lengths / windows: optional explicit context lengths / window widths per sequence.
    """
    assert s.fmt in FORMATS and s.num_q_heads % s.num_kv_heads == 0
    B, Hkv, D, fmt = s.num_seqs, s.num_kv_heads, s.head_dim, s.fmt
    r = _rngs(s.seed)

    # lengths and windows
    if lengths is not None:
        L = np.asarray(lengths, dtype=np.int32)
    elif s.context is not None:
        L = np.full(B, s.context, dtype=np.int32)
    else:
        L = r["lengths"].integers(s.ctx_range[0], s.ctx_range[1] + 1, size=B).astype(np.int32)
    if windows is not None:
        W = np.asarray(windows, dtype=np.int32)
    else:
        W = np.zeros(B, dtype=np.int32)
        if s.window > 0 and s.window_frac > 0:
            n_win = int(round(B * s.window_frac))
            W[r["window"].permutation(B)[:n_win]] = s.window
    max_ctx = max(int(L.max(initial=0)), 1) if lengths is not None else s.max_context
    max_blocks = -(-max_ctx // BLOCK_SIZE)

    # pool and block tables
    n_pages = (-(-L.astype(np.int64) // BLOCK_SIZE))
    need = int(n_pages.sum())
    pool = s.pool_total if s.pool_total is not None else need + s.pool_spare
    assert pool >= need
    perm = r["pool"].permutation(pool).astype(np.int32)
    spare = perm[need:]
    bt = np.empty((B, max_blocks), dtype=np.int32)
    cur = 0
    for b in range(B):
        bt[b, : n_pages[b]] = perm[cur: cur + n_pages[b]]
        cur += n_pages[b]
        if unused_fill == "spare" and len(spare):
            bt[b, n_pages[b]:] = spare[b % len(spare)]
        else:
            bt[b, n_pages[b]:] = -1

    # query: [B, Hq, D], or [B, n_q, Hq, D] for a chunk of n_q queries per sequence
    qshape = (B, s.num_q_heads, D) if s.queries_per_seq == 1 else (B, s.queries_per_seq, s.num_q_heads, D)
    q = bf16_bits(r["q"].standard_normal(qshape, dtype=np.float32))

    kb, vb = k_chunk_bytes(fmt, D), v_chunk_bytes(fmt, D)
    k_cache = np.empty((pool, Hkv, kb), dtype=np.uint8)
    v_cache = np.empty((pool, Hkv, vb), dtype=np.uint8)
    scales = codebook_arr = sgn = None
    k_fp8, v_cb, k_cb = k_is_fp8(fmt), v_is_codebook(fmt), fmt in KV_BITS
    knorm = vnorm = kscale = None
    nan_or_0 = np.float32(np.nan if poison else 0.0)
    if v_cb:
        cb_v = codebook(16, D)
        sgn = sign_pattern(r["sign"], D)
        vnorm = np.full((pool, Hkv, BLOCK_SIZE), nan_or_0, dtype=np.float32)
        if k_cb:
            cb_k = codebook(1 << KV_BITS[fmt][0], D)
            codebook_arr = np.concatenate([cb_k, cb_v]).astype(np.float32)
            knorm = np.full((pool, Hkv, BLOCK_SIZE), nan_or_0, dtype=np.float32)
        else:
            codebook_arr = cb_v.copy()

    # poison everything first; real pages are overwritten below
    k_poison = BF16_POISON if fmt == "bf16" else (FP8_POISON if k_fp8 else np.uint8(0x5A))
    v_poison = BF16_POISON if fmt == "bf16" else (FP8_POISON if fmt == "fp8" else np.uint8(0xA5))
    kview = k_cache.view(np.uint16) if fmt == "bf16" else k_cache
    vview = v_cache.view(np.uint16) if fmt == "bf16" else v_cache
    kview[...] = k_poison if poison else 0
    vview[...] = v_poison if poison else 0

    # K and V of sequence b come from child b of the K / V stream, so sequences can be drawn and
    # encoded in parallel threads with a result that does not depend on the thread count.
    k_kids, v_kids = r["k_seq"].spawn(B), r["v_seq"].spawn(B)

    def draw(seq):
        if kv_override is not None:
            kk, vv = kv_override(seq, int(L[seq]))
            return np.asarray(kk, np.float32), np.asarray(vv, np.float32)
        shape = (Hkv, int(L[seq]), D)
        return (np.random.default_rng(k_kids[seq]).standard_normal(shape, dtype=np.float32),
                np.random.default_rng(v_kids[seq]).standard_normal(shape, dtype=np.float32))

    starts = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int64)
    workers = max(1, min(16, os.cpu_count() or 1, B))
    drawn = {}
    fp8_scales = None
    if k_fp8:
        # one fp32 scale per (K|V, KV head) = amax / 448 over the whole batch: draw first
        def first(b):
            kk, vv = draw(b)
            drawn[b] = (kk, vv)
            if not kk.size:
                return np.zeros((2, Hkv), np.float32)
            return np.stack([np.abs(kk).max(axis=(1, 2)), np.abs(vv).max(axis=(1, 2))])
        with ThreadPoolExecutor(workers) as ex:
            amaxes = list(ex.map(first, range(B)))
        if fp8_scale is None:
            amax = np.max(np.stack(amaxes), axis=0).astype(np.float32)
            fp8_scales = (amax / np.float32(448.0)).astype(np.float32)
            fp8_scales[fp8_scales == 0] = np.float32(1.0)
        else:
            fp8_scales = np.asarray(fp8_scale, dtype=np.float32).reshape(2, Hkv)
        kscale = fp8_scales[0]
        if fmt == "fp8":
            scales = fp8_scales

    def fill_seq(b):
        Lb, npg = int(L[b]), int(n_pages[b])
        phys = perm[starts[b]: starts[b] + npg]
        kk, vv = drawn.pop(b) if b in drawn else draw(b)
        if npg == 0:
            return
        pad = npg * BLOCK_SIZE - Lb

        def put_norms(plane, nrm):
            nrm = np.concatenate([nrm, np.full((Hkv, pad), nan_or_0, np.float32)], axis=1)
            plane[phys] = nrm.reshape(Hkv, npg, BLOCK_SIZE).transpose(1, 0, 2)

        if fmt == "bf16":
            ke, ve = bf16_bits(kk), bf16_bits(vv)
        elif k_fp8:
            ke = e4m3fn_encode(kk / kscale[:, None, None])
        else:
            ke, kn = turbo_encode(kk, sgn, cb_k)
            put_norms(knorm, kn)
        if fmt == "fp8":
            ve = e4m3fn_encode(vv / fp8_scales[1][:, None, None])
        elif v_cb:
            ve, vn = turbo_encode(vv, sgn, cb_v)
            put_norms(vnorm, vn)
        kfill = k_poison if (poison and (fmt == "bf16" or k_fp8)) else np.zeros((), ke.dtype)
        vfill = v_poison if (poison and not v_cb) else np.zeros((), ve.dtype)
        del kk, vv
        ke = np.concatenate([ke, np.full((Hkv, pad, D), kfill, ke.dtype)], axis=1)
        ve = np.concatenate([ve, np.full((Hkv, pad, D), vfill, ve.dtype)], axis=1)
        ke = ke.reshape(Hkv, npg, BLOCK_SIZE, D).transpose(1, 0, 2, 3)
        ve = ve.reshape(Hkv, npg, BLOCK_SIZE, D).transpose(1, 0, 2, 3)
        k_cache[phys, :, : k_code_bytes(fmt, D)] = pack_k_pages(fmt, ke)
        v_cache[phys, :, : v_code_bytes(fmt, D)] = pack_v_pages(fmt, ve)
        first_key = Lb - s.queries_per_seq + 1 - int(W[b])   # of the chunk's first query
        if poison_before_window and W[b] > 0 and first_key > 0:
            first_live = first_key // BLOCK_SIZE
            dead = phys[:first_live]
            if fmt == "bf16" or k_fp8:
                kview[dead] = k_poison
            else:
                knorm[dead] = np.nan
            if v_cb:
                vnorm[dead] = np.nan
            else:
                vview[dead] = v_poison

    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill_seq, range(B)))

    # per-token norms: 16 little-endian fp32 after the indices of each (page, KV head) chunk
    if knorm is not None:
        k_cache[:, :, k_code_bytes(fmt, D):] = knorm.astype("<f4").view(np.uint8).reshape(pool, Hkv, -1)
    if vnorm is not None:
        v_cache[:, :, v_code_bytes(fmt, D):] = vnorm.astype("<f4").view(np.uint8).reshape(pool, Hkv, -1)
    if fmt == "turbo8":
        scales = np.asarray(kscale, dtype=np.float32).copy()
    return Inputs(spec=s, q=q, k_cache=k_cache, v_cache=v_cache, scales=scales,
                  codebook=codebook_arr, sign=sgn, block_table=bt, context_lens=L, window=W,
                  softmax_scale=s.scale, softcap=np.float32(s.softcap), max_context_len=max_ctx)


def relayout(inp: Inputs, seed: int) -> Inputs:
    """The same logical cache placed in a different random set of physical pages."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xB10C]))
    pool = inp.num_pool_blocks
    new_of_old = rng.permutation(pool).astype(np.int32)
    k = np.empty_like(inp.k_cache)
    v = np.empty_like(inp.v_cache)
    k[new_of_old] = inp.k_cache
    v[new_of_old] = inp.v_cache
    bt = inp.block_table.copy()
    ok = bt >= 0
    bt[ok] = new_of_old[bt[ok]]
    return dataclasses.replace(inp, k_cache=k, v_cache=v, block_table=bt)
