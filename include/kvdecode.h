/*
 * kvdecode.h -- C ABI of a gfx950 (AMD Instinct MI355X) library for single-query (decode-phase)
 * attention over a paged KV cache.
 *
 * What it computes.  For each sequence b and query head h, with L = context_lens[b] and the
 * attended key range [lo, L) (lo = max(0, L - window[b]) when window[b] > 0, else 0):
 *
 *     z_j   = softmax_scale * <q[b,h], k_j>            j in [lo, L)
 *     z_j   = softcap * tanh(z_j / softcap)             only when softcap > 0
 *     z_j  += alibi_slopes[h] * (j - (L - 1))           only when alibi_slopes != NULL
 *     out[b,h] = sum_j exp(z_j - max z) v_j / sum_j exp(z_j - max z)
 *
 * with k_j, v_j the dequantised key/value vectors of KV head floor(h / (Hq / Hkv)) (GQA/MQA).
 * Sources: attention.rs README ("KV Cache Formats": BF16, FP8 E4M3, Turbo8, Turbo4 and Turbo3
 * caches,
 * each with decode and Split-K decode kernels sharing one float reduce, Split-K from 1024
 * tokens; "Features": softcapping, sliding window, GQA/MQA, paged block tables, causal mask;
 * the paged-attention bullet list adds "ALiBi slopes")
 * and turboquant-rs 0.4.1 src/cache/cuda/attention.rs (two phases, partitioned attention then
 * a reduce; 512-token partitions, ceil(kv_len / 512) of them; fp32 per-partition max, sum and
 * output; the compressed cache is read directly with a sign pattern and a codebook; an empty
 * context yields an all-zero fp32 output).
 *
 * Readings where those pages are silent: the window holds the W most recent keys including
 * the query's own position; the cap acts on the scaled logit before the max; the ALiBi term
 * (per query head, the query at position L - 1) is added after the cap; an empty context
 * gives zero rows; partitions sit at absolute multiples of the partition size.
 *
 * A chunk of queries per sequence (kvd_dims.queries_per_seq = n_q > 1; the README's "Chunked
 * Prefill" and "causal masking" over the same paged, possibly compressed cache): the n_q
 * queries occupy the last n_q positions of the context (their K and V are already in the
 * cache).  Query i sits at position p = L - n_q + i and attends causally exactly like the
 * decode query of the context prefix that ends there: keys [lo_i, p] with lo_i = max(0, p + 1 -
 * window[b]) under a window, else 0; the ALiBi term is alibi_slopes[h] * (j - p).  A sequence
 * with 0 < L < n_q gets NaN rows (its query positions would be negative).  The queries of a
 * chunk share the value operand of one matrix product, so a non-finite value stored in a key
 * that one query attends reaches the rows of the others that do not (weight 0 times NaN);
 * keys outside every query's range are never multiplied.
 *
 * Conventions for every entry point.
 *   - All array pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates, frees or synchronises; it keeps no state between calls.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null stream).
 *     Buffers must stay alive until that work has finished.
 *   - Errors are returned as an int status (kvd_status), never printed.  Arguments are checked
 *     on the host before anything is launched, so a call that returns an error has launched
 *     nothing.  After launching, a pending HIP launch error maps to KVD_ERR_HIP.
 *   - Data-dependent faults the host cannot see are caught on the device, never by reading
 *     out of bounds: a sequence whose context length is negative or above max_context_len, or
 *     any of whose block-table entries in the attended range lies outside [0, num_pool_blocks),
 *     gets NaN in all of its output rows.
 *
 * PAGED LAYOUT (block_size is 16 tokens; "chunk" = the bytes of one (page, KV head)).
 * The K cache is an array [num_pool_blocks][num_kv_heads][k_chunk] of bytes, the V cache
 * [num_pool_blocks][num_kv_heads][v_chunk]; chunk (p, h) starts at byte (p * Hkv + h) * chunk.
 * Inside one chunk, with D = head_dim, t the token slot 0..15 and d the element index:
 *
 *   BF16  (KVD_BF16)      K: [D/8][16][8] bf16   -- element (t, d) at ((d/8)*16 + t)*8 + d%8
 *                         V: [D][16]      bf16   -- element (t, d) at d*16 + t (transposed)
 *                         k_chunk = v_chunk = 32*D bytes
 *   FP8   (KVD_FP8_E4M3)  K: [D/16][16][16] u8   -- element (t, d) at ((d/16)*16 + t)*16 + d%16
 *                         V: [D][16] u8          -- element (t, d) at d*16 + t
 *                         codes are OCP E4M3FN (bias 7, max 448, S.1111.111 = NaN);
 *                         value = E4M3FN(code) * scale, one fp32 scale per (K|V, KV head).
 *                         k_chunk = v_chunk = 16*D bytes
 *   TURBO4 (KVD_TURBO4)   K: [D/32][16][16 B]    -- 32 4-bit indices per 16-byte group
 *   TURBO3 (KVD_TURBO3)   K: [D/32][16][12 B]    -- 32 3-bit indices per 12-byte group
 *                         index of (t, d) sits in group ((d/32)*16 + t) at position e = d%32:
 *                         bits [b*e, b*e + b) of the group's little-endian bitstream (stream
 *                         bit k = bit k%8 of byte k/8; 4-bit: even e in the low nibble).
 *                         V (both Turbo formats, 4-bit): [D][16 nibbles = 8 B] -- index of
 *                         (t, d) is nibble t of row d (even t in the low nibble).
 *                         After the indices of every K and V chunk: norm[16], the fp32
 *                         (little-endian) per-token norms of the page's 16 slots, so one page
 *                         of one head is one contiguous record.
 *                         k_chunk = 8*D + 64 (TURBO4) or 6*D + 64 (TURBO3), v_chunk = 8*D + 64.
 *                         Stored value in the rotated domain: norm[t] * codebook[index];
 *                         the original vector is  x = diag(s) H x_rot / sqrt(D), H the
 *                         Sylvester-order D x D Hadamard matrix, s = sign_pattern.
 *   TURBO8 (KVD_TURBO8)   FP8 K + 4-bit V ("FP8 K + 4-bit V (Walsh-Hadamard)" in the formats
 *                         table; reading: K exactly as the FP8 format stores it -- not
 *                         rotated, one fp32 scale per KV head -- and V exactly as the Turbo
 *                         formats store it, norms included).  k_chunk = 16*D,
 *                         v_chunk = 8*D + 64 bytes.
 *
 * Query q: bf16 [num_seqs][n_q][num_q_heads][D] (n_q = 1: [num_seqs][num_q_heads][D]).
 * Output out: fp32 with the same shape, in the original (un-rotated) domain for every format.
 */
#ifndef KVDECODE_H
#define KVDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvd_format {
    KVD_BF16 = 0,       /* unquantised bfloat16 K and V */
    KVD_FP8_E4M3 = 1,   /* OCP E4M3FN codes, fp32 scale per KV head */
    KVD_TURBO4 = 2,     /* rotated codebook: 4-bit K, 4-bit V, fp32 per-token norms */
    KVD_TURBO3 = 3,     /* rotated codebook: 3-bit K, 4-bit V, fp32 per-token norms */
    KVD_TURBO8 = 4      /* FP8 K (fp32 scale per KV head) + rotated 4-bit V (per-token norms) */
} kvd_format;

typedef enum kvd_status {
    KVD_OK = 0,
    KVD_ERR_NULL = -1,       /* a required pointer is NULL */
    KVD_ERR_SHAPE = -2,      /* unsupported or inconsistent dimensions */
    KVD_ERR_FORMAT = -3,     /* unknown kv format */
    KVD_ERR_ALIGN = -4,      /* a pointer is not 16-byte aligned */
    KVD_ERR_WORKSPACE = -5,  /* workspace missing or smaller than kvd_workspace_bytes() */
    KVD_ERR_HIP = -6         /* the HIP runtime reported an error while launching */
} kvd_status;

/* Shapes.  Supported: block_size == 16; head_dim 64 or 128 for BF16/FP8, 128 for the Turbo
 * formats; num_q_heads a multiple of num_kv_heads.  A query group larger than 16 (MQA-like
 * shapes) is processed in tiles of 16 query heads; single-query BF16 / FP8 compute two tiles
 * per wavefront, which share its page loads, and other cases read a KV head's pages once per
 * tile.  Size limits (KVD_ERR_SHAPE beyond them): num_seqs, num_kv_heads <= 65535;
 * num_seqs * n_q * num_q_heads < 2^31 query rows; the workspace of a split (its m, l and
 * outputs for every row and partition) below 2^62 bytes. */
typedef struct kvd_dims {
    int32_t num_seqs;            /* B */
    int32_t num_q_heads;         /* Hq */
    int32_t num_kv_heads;        /* Hkv */
    int32_t head_dim;            /* D */
    int32_t block_size;          /* tokens per page; must be 16 */
    int32_t max_blocks_per_seq;  /* row length of block_table */
    int32_t num_pool_blocks;     /* pages in the K/V pools (device-side bounds check) */
    int32_t max_context_len;     /* upper bound on context_lens[], >= 1, <= 16 * max_blocks_per_seq */
    int32_t partition_size;      /* 0: auto -- 512-token partitions when a sequence attends to
                                    >= 1024 tokens, else a single partition;
                                    > 0: always split at that many tokens (a multiple of 16);
                                    -1: never split */
    int32_t partitions_per_wave; /* launch tuning: the run one wavefront walks through a split
                                    sequence; a workgroup's runs give one triple (results
                                    agree to rounding: the online softmax groups its sums by
                                    run and workgroup).
                                    0: auto -- for a batch of max_context_len sequences,
                                    each (sequence, KV head, unit) gets as many whole
                                    workgroups as one round of the device's resident
                                    wavefronts holds, its page pairs spread over their
                                    wavefronts (whole 32-token pairs, a workgroup's runs at
                                    least one partition, at most 4 partitions per run, one
                                    workgroup per CU where two would get runs under 16
                                    pairs; a wavefront computing two query
                                    tiles counts twice; with a mean_context_len hint, the
                                    batch's mean work over about 2.5 rounds; single-query BF16 at head_dim 128
                                    with at most 16 query heads per KV head uses a layout with
                                    one workgroup per CU and runs of up to 8 partitions when
                                    that covers the device in one round; BF16 / FP8 runs
                                    alternate slightly longer and shorter between workgroups
                                    that run on the faster and the slower XCDs, and with two
                                    workgroups per CU the half dispatched first gets slightly
                                    longer runs);
                                    > 0: runs of that many partitions.  Capped at the
                                    partitions of max_context_len; runs are one partition when
                                    the partition size is not a multiple of 32.  >= 0. */
    int32_t queries_per_seq;     /* n_q: queries per sequence, a chunk at the last n_q positions
                                    (above); 0 or 1: single-query decode.  The n_q * Hq / Hkv
                                    query rows of a KV head share one pass over its pages per
                                    16 rows (32 for BF16 / FP8).  Requires n_q <= max_context_len and
                                    num_seqs * n_q <= 65535. */
    int32_t mean_context_len;    /* launch hint, results do not depend on it: the batch's mean
                                    attended span in tokens (min(L, window + n_q - 1) for
                                    windowed sequences, else L), as the caller's host-side
                                    bookkeeping knows it; 0 = unknown, taken as
                                    max_context_len.  Below max_context_len (a ragged batch)
                                    the automatic run choice makes about 2.5 waves of work per
                                    resident wavefront slot instead of one, so runs of unequal
                                    sequences even out.  0 <= mean_context_len. */
} kvd_dims;

/* Bytes of device workspace kvd_decode_attn_paged needs: slots for per-partition fp32 triples
 * (the workgroups of a sequence write consecutive slots from its first partition's)
 * m [B][n_q][Hq][P], l [B][n_q][Hq][P] and o [B][n_q][Hq][P][D], P = ceil(max_context_len /
 * partition size), each array starting on a 256-byte boundary.  Returns 0 for invalid dims. */
size_t kvd_workspace_bytes(const kvd_dims* dims);

/* Decode attention, both phases (partition kernel, then the reduce kernel when any sequence
 * is split).  When every split sequence is one workgroup's walk (a single run block, below),
 * nothing is merged across workgroups: the partition kernel writes the final rows as for an
 * unsplit sequence and the reduce is not launched.
 *   q            bf16 [B][n_q][Hq][D]
 *   k_cache      K pool in `fmt`'s layout (above);  v_cache  V pool
 *   block_table  int32 [B][max_blocks_per_seq]; entries for the pages holding the attended
 *                range [lo, L) must be valid pool indices (others are never read)
 *   context_lens int32 [B]; 0 gives an all-zero output row
 *   fmt          a kvd_format
 *   scales       KVD_FP8_E4M3: fp32 [2][Hkv], K scales then V; KVD_TURBO8: fp32 [Hkv], the K
 *                scales; KVD_BF16 / KVD_TURBO4 / KVD_TURBO3: unused, may be NULL (the Turbo
 *                per-token norms live in the cache chunks)
 *   codebook     KVD_TURBO4/3: fp32 levels, 2^kbits for K then 16 for V (kbits 4 or 3);
 *                KVD_TURBO8: the 16 V levels; else unused
 *   sign_pattern Turbo: fp32 [D] of +1.0 / -1.0; else unused
 *   softmax_scale  logit scale (e.g. 1/sqrt(D))
 *   window       int32 [B] sliding-window widths (0 = none), or NULL for no window at all
 *   softcap      tanh cap on the scaled logits; 0 = off
 *   alibi_slopes fp32 [Hq] per-query-head ALiBi slopes, or NULL for none
 *   out          fp32 [B][n_q][Hq][D]; must not alias any input
 *   workspace    >= kvd_workspace_bytes(dims) bytes, 256-byte aligned; contents on entry do
 *                not matter; on return it holds the partials of split sequences (untouched
 *                when each sequence is a single run block)
 *   stream       hipStream_t
 * All pointers 16-byte aligned. */
int kvd_decode_attn_paged(const kvd_dims* dims, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* block_table,
                          const int32_t* context_lens, int fmt, const float* scales,
                          const float* codebook, const float* sign_pattern, float softmax_scale,
                          const int32_t* window, float softcap, const float* alibi_slopes,
                          float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Largest partition workspace (bytes) kvd_decode_attn_paged_noalloc can use. */
#define KVD_NOALLOC_WORKSPACE_BYTES ((size_t)128 << 20)

/* For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  kvd_decode_attn_paged without the workspace
 * arguments: the partition triples go to a device array inside the library,
 * KVD_NOALLOC_WORKSPACE_BYTES on each GPU the library runs on, held from the library's load
 * until the process ends.  The first call on a GPU looks up that GPU's copy of the array
 * (hipGetSymbolAddress, with the GPU current); no call allocates or frees memory.
 * Errors: as kvd_decode_attn_paged; KVD_ERR_WORKSPACE when kvd_workspace_bytes(dims) exceeds
 * KVD_NOALLOC_WORKSPACE_BYTES (each (query row, partition) triple takes (head_dim + 2) * 4
 * bytes: the array holds about 258,000 of them at head_dim 128, e.g. 16 sequences x 64 query
 * heads at 32K context use 65,536); KVD_ERR_HIP when the array's address cannot be obtained.
 * All calls on one GPU share its array, which keeps the last call's contents.  Nothing in it
 * needs to start at zero (each call writes every triple it reads back), but calls that overlap
 * in time on one GPU -- on different streams, or from host threads without ordering -- race on
 * it and give wrong results; calls enqueued on one stream are ordered and safe. */
int kvd_decode_attn_paged_noalloc(const kvd_dims* dims, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table,
                                  const int32_t* context_lens, int fmt, const float* scales,
                                  const float* codebook, const float* sign_pattern,
                                  float softmax_scale, const int32_t* window, float softcap,
                                  const float* alibi_slopes, float* out, void* stream);

/* Phase 1 alone (same arguments).  Wavefronts per (KV head, sequence) walk runs of T tokens
 * (partitions_per_wave > 0: T = that many partitions; 0: the automatic choice, a whole number
 * of 32-token page pairs of at least one partition), W = 4 wavefronts per workgroup (8 for
 * the Turbo formats).  For a split sequence with attended range [lo, L), let p0 be the first
 * partition the range touches (P tokens per partition); run k covers tokens
 * [p0*P + k*T, p0*P + (k+1)*T) intersected with [lo, L), and workgroup x walks runs
 * W*x .. W*x + W - 1.  (The automatic choice may instead alternate run lengths T + s in even
 * workgroups and T - s in odd ones, s a multiple of 32 and T - s at least a partition, so
 * workgroup x starts at p0*P + (x/2)*2*W*T + (x%2)*W*(T + s); BF16 / FP8, one query tile per
 * KV head, no ragged-length hint.  Where that grid is also exactly two workgroups per CU and
 * holds an even number Y of workgroup pairs (2y, 2y + 1) per sequence, both runs of the pairs
 * y >= Y/2, which go out first, are a tokens longer and those of pairs y < Y/2 a shorter, a a
 * multiple of 32 and T - s - a at least a partition: pair y starts at p0*P + 2*W*y*(T - a)
 * for y <= Y/2 and at p0*P + W*Y*(T - a) + 2*W*(y - Y/2)*(T + a) beyond, and its odd
 * workgroup starts W*(T + s + a) (y >= Y/2) or W*(T + s - a) tokens after its even one.)
 * Their keys j together give one triple at workspace slot (b, i, h, p0 + x):
 * m = max_j z_j * log2(e)  (base-2 units),  l = sum_j exp(z_j - max z),
 * o[d] = sum_j exp(z_j - max z) v_j[d] / l  -- with o in the rotated domain for the Turbo
 * formats; the keys j are those of the workgroup's runs that query i sees, and a query that
 * sees none of them gets m = -inf, l = 0, o = 0.  Other slots are not written.  Sequences that
 * are not split get their final output row written here. */
int kvd_decode_partitions(const kvd_dims* dims, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* block_table,
                          const int32_t* context_lens, int fmt, const float* scales,
                          const float* codebook, const float* sign_pattern, float softmax_scale,
                          const int32_t* window, float softcap, const float* alibi_slopes,
                          float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Phase 2 alone (same arguments, so the same run length R; reads the workspace phase 1
 * filled).  For each split (b, h), over its triples k: M = max_k m_k, w_k = l_k 2^(m_k - M),
 * out = sum_k w_k o_k / sum_k w_k, then (Turbo)
 * out <- diag(s) H out / sqrt(D).  Rows of sequences that are not split are left untouched. */
int kvd_reduce_partitions(const kvd_dims* dims, const void* q, const void* k_cache,
                          const void* v_cache, const int32_t* block_table,
                          const int32_t* context_lens, int fmt, const float* scales,
                          const float* codebook, const float* sign_pattern, float softmax_scale,
                          const int32_t* window, float softcap, const float* alibi_slopes,
                          float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Test export: dequantised cache values of tokens [token_begin, token_begin + n_tokens) of
 * sequence `seq`, KV head `kv_head`, gathered through the block table, written as fp32
 * [n_tokens][D] in the storage domain: BF16 widened; FP8 E4M3FN(code) * scale rounded to fp32;
 * Turbo norm * codebook[index] rounded to fp32 (still rotated).  is_v selects V (1) or K (0).
 * `scales`, `codebook` as for kvd_decode_attn_paged.  A separate gather kernel forms these
 * values (one thread per element, its own page addressing and index extraction; it shares the
 * FP8 -> bf16 decode and the 3-bit field selection with the attention kernel).  The attention
 * kernel never forms norm * codebook[index]: it factors the norm out and feeds the levels to
 * its matrix cores in fp16 (K levels as hi + lo pairs, V levels rounded once);
 * kvd_dequant_operands exports those operands.  Tokens
 * must lie in [0, 16 * max_blocks_per_seq). */
int kvd_dequant_gather(const kvd_dims* dims, int fmt, int is_v, const void* cache,
                       const float* scales, const float* codebook, const int32_t* block_table,
                       int32_t seq, int32_t kv_head, int32_t token_begin, int32_t n_tokens,
                       float* out, void* stream);

/* Test export: the matrix-core operands the partition kernel forms from the cache, produced by
 * the partition kernel's own load (lane map, 16-byte loads), FP8 decode and codebook pair-table
 * code, for page pairs pair_begin .. pair_begin + n_pairs - 1 of sequence `seq`, KV head
 * `kv_head` (pair k = the sequence's pages 2k and 2k + 1; requires
 * 2 * (pair_begin + n_pairs) <= max_blocks_per_seq).  Arguments as for kvd_decode_attn_paged.
 * out: uint32 [n_pairs][64][head_dim + 16], one record per lane l of a 64-lane wavefront, with
 * n = l % 16, j = l / 16.  The lane's tokens (page 0/1 of the pair, slot):
 *   QK tile X: (n / 8, 8 ((n / 4) % 2) + n % 4); tile Y: four slots later;
 *   softmax / PV: (j / 2, 8 (j % 2) + e), e = 0..7.
 * Words [16 s, 16 s + 16), s = 0 .. D/32 - 1: QK step s operands x0, x1 (tile X), y0, y1 (Y), 4
 *   words each, covering head elements
 *     BF16: d = 32 s + 8 j + e;  FP8 / Turbo8 K: d = 64 (s / 2) + 16 j + 8 (s % 2) + e;
 *     Turbo4/3 K: d = 32 j + 8 s + e   (e = 0..7).
 *   BF16 / FP8 / Turbo8 K: x0 = the eight values as bf16 (FP8 exact: E4M3FN(code), unscaled),
 *   x1 = 0.  Turbo4/3 K: x0 = fp16 [h0 .. h7], x1 = fp16 [l0 .. l7] of the eight elements,
 *   with (h, l) = (fp16(c), fp16(c - h)) of c = codebook level * 2^-E, 2^-E the power of two
 *   that puts the largest K level magnitude in [0.5, 1).
 * Words [D/2 + 8 t, D/2 + 8 t + 8), t = 0 .. D/16 - 1: PV tile t operand v (4 words), then 4
 *   zero words, for head element d = 16 t + n and the lane's eight softmax tokens e: BF16 /
 *   FP8 v = bf16 values; codebook V: v = fp16 [c0 .. c7], c = fp16(V level * 2^-E), 2^-E the
 *   power of two that puts the largest V level magnitude in [0.5, 1).
 * Words [D, D + 16): fp32 K norms of the eight softmax tokens (Turbo4/3; else 0), then their
 *   V norms (codebook V; else 0), as stored after the chunks' indices.
 * A pair with a block-table entry outside the pool gets all-ones records. */
int kvd_dequant_operands(const kvd_dims* dims, int fmt, const void* k_cache,
                         const void* v_cache, const float* scales, const float* codebook,
                         const int32_t* block_table, int32_t seq, int32_t kv_head,
                         int32_t pair_begin, int32_t n_pairs, uint32_t* out, void* stream);

/* KV append (quantize-on-write): stores n_new new tokens of every sequence in the paged cache,
 * in the layout above, so the decode entry points read them back.  Sources: the attention.rs
 * README "KV Cache Formats" table (the storage formats) and the compressed-cache recipe
 * (each token vector is flipped by the +-1 sign pattern, transformed by the orthonormal
 * Walsh-Hadamard transform, normalised by its fp32 L2 norm, stored per token, and each
 * coordinate replaced by the index of the nearest codebook level, indices bit-packed
 * little-endian); turboquant-rs 0.4.1 src/cache/cuda/attention.rs reads those packed indices,
 * per-token scales, the sign pattern and the codebook.
 *   k_new, v_new  fp32 [B][n_new][Hkv][D], device; 8-byte aligned
 *   block_table   int32 [B][max_blocks_per_seq]; must already map the pages of the new tokens
 *   positions     int32 [B]: new token i of sequence b is token positions[b] + i (its page is
 *                 block_table[b][(positions[b] + i) / 16], slot (positions[b] + i) % 16)
 *   n_new         tokens per sequence in this call (>= 0; 0 does nothing)
 *   k_cache, v_cache  the pools, updated in place (other tokens' bytes are preserved)
 *   scales        KVD_FP8_E4M3: fp32 [2][Hkv] per-head scales; KVD_TURBO8: fp32 [Hkv] K scales;
 *                 else unused, may be NULL (read only: Turbo norms are written into the
 *                 chunks)
 *   codebook, sign_pattern  Turbo: as for kvd_decode_attn_paged; else unused
 * Codes, decided exactly (readings where the pages are silent):
 *   BF16  round to nearest even; NaN stored as 0x7FC0.
 *   FP8   E4M3FN(fp32(x / scale)), round to nearest even, saturating to +-448; NaN as 0x7F.
 *   Turbo r = H (s * x) / sqrt(D) in fp64; norm = fp32(sqrt(sum x_i^2)), the fp64 sum taken as
 *         a pairwise tree over adjacent elements; u = r / norm in fp64; index = the number of
 *         level midpoints (c_k + c_{k+1}) / 2 below u (a tie takes the lower level); a zero
 *         vector stores norm 0 and the level nearest 0.
 * Tokens whose page index is out of range or whose page id lies outside [0, num_pool_blocks)
 * are skipped (nothing written).  Different tokens of one call may share pages; calls that
 * overlap in time on different streams must not write the same page. */
int kvd_append_kv(const kvd_dims* dims, int fmt, const float* k_new, const float* v_new,
                  const int32_t* block_table, const int32_t* positions, int32_t n_new,
                  void* k_cache, void* v_cache, const float* scales, const float* codebook,
                  const float* sign_pattern, void* stream);

/* Measurement export: an HBM read probe giving the decode kernels' practical ceiling.
 * Reads n_chunks chunks of chunk_bytes (a power of two, >= 1024) from buf, chunk chunk_ids[c] (at
 * byte chunk_ids[c] * chunk_bytes; ids outside the buffer read chunk 0) in list order, with
 * device_CUs * waves_per_cu / 4 workgroups of four wavefronts (waves_per_cu a multiple of 4,
 * 4..32).  Each wavefront takes loads_in_flight (1, 2, 4, 8 or 16) consecutive 1 KB pieces of
 * the list per turn -- all issued before any is used -- then the pieces nwaves * loads_in_flight
 * further on.  Consecutive ids make a plain read stream; a random permutation reads chunks at
 * random places like a paged cache.  The data is folded into sink (uint32, at least
 * device_CUs * waves_per_cu * 64 words, write-only) so nothing is skipped.  Asynchronous on
 * stream; time it with events. */
int kvd_read_probe(const void* buf, size_t buf_bytes, const int32_t* chunk_ids, int64_t n_chunks,
                   int32_t chunk_bytes, int32_t waves_per_cu, int32_t loads_in_flight,
                   uint32_t* sink, size_t sink_bytes, void* stream);

/* A static, human-readable name for a status code. */
const char* kvd_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVDECODE_H */
