// HIP kernels for decode attention over a paged KV cache on gfx950 (MI355X): one query per
// sequence, or a chunk of queries at a sequence's last positions (multi-token decode / chunked
// prefill over the same cache).
//
// Two phases, as in turboquant-rs 0.4.1 src/cache/cuda/attention.rs ("partitioned attention +
// reduce"; 512-token partitions; fp32 per-partition max, sum and output) and the attention.rs
// README (Split-K decode for every cache format from 1024 tokens on, one shared float reduce):
//
//   partition_kernel<FMT, D, CAP, PF, MQ, WIDE, NT>  a 1-D grid of workgroups (4 waves for
//       BF16 / FP8, two per CU, or one per CU in the WIDE layout of single-query BF16; 8 for
//       the codebook formats) over (run block, sequence, KV head x unit of NT query tiles).
//       For a split sequence each wave walks a run of consecutive page pairs of one (sequence,
//       KV head, unit), and the workgroup merges its waves' runs into one (m, l, o) triple;
//       an unsplit sequence's pages are shared by the workgroup's waves, which merge through
//       LDS into the final rows.  A wave
//       walks pairs of 16-token pages, software-pipelined: PF pairs' loads are in flight while
//       it computes, and the block-table entries ahead of them come in with scalar loads.  Per
//       pair it
//         - loads K and V of both pages straight into MFMA operand registers (16-byte loads
//           for K; V rows are 32/16/8 bytes per 16-token row depending on the format);
//         - computes S^T = K Q^T for 32 tokens x 16 query rows (the GQA group -- or, with a
//           chunk of queries, (query, head) pairs -- zero padded) with
//           v_mfma_f32_16x16x32_{bf16,f16}, dequantising in registers on the way: FP8 -> bf16
//           is exact; codebook levels come from conflict-free pair tables in LDS;
//         - runs an fp32 online softmax in the base-2 domain (the per-row max crosses the four
//           16-lane groups with two permlane swaps; the reference max moves lazily);
//         - accumulates O^T += V^T P^T with the same MFMA shape.
//       Operand precision: BF16 and FP8 K/V (and Turbo8 K) use exact bf16 operands and feed P
//       as a bf16 hi + lo pair (2^-16 relative).  Codebook K levels and the rotated query are
//       fp16 hi + lo pairs (about 2^-20 relative; plain fp16 levels or query would add a
//       logit error that large logits turn into a visible output error).  Codebook V levels
//       and P are each rounded once to fp16 (2^-12 relative; the output error they add is
//       relative to the row and independent of the logits' size).  Power-of-two scalings
//       keep every fp16 value in range.
//       The MFMA output layout of S^T (lane = query row, 4 lane groups x 4 rows = 16 tokens) is
//       exactly the B-operand layout of P^T for the PV product once the pair's two pages are
//       interleaved as below, so no data moves between the two products.
//   reduce_kernel<FMT, D>    one wave per (query head, sequence x query of the chunk): LSE
//       merge of the run blocks' triples, then (codebook V) the inverse rotation
//       diag(s) H / sqrt(D).
//   gather_kernel            test export: dequantised values through the block table, one
//       thread per element with its own page addressing and index unpacking (the FP8 decode
//       and the 3-bit field extraction are the attention kernel's).
//   operand_kernel           test export: the attention kernel's own page loads, lane map,
//       FP8 decode and pair-table reads, writing every lane's MFMA operands and norms.
//
// MFMA 16x16x32 operand layout used throughout (lane = 0..63, n = lane % 16, j = lane / 16):
//   A operand: row n, 8 consecutive k-slots of group j;  B operand: column n, same k-slots;
//   C/D: column n, rows 4j..4j+3.
// Token placement for one page pair (pages A, B): QK tile X row m holds token
//   (page m/8, slot 8*((m/4)%2) + m%4), tile Y the slot 4 higher; after the QK product lane
//   (n, j) then holds query n's logits for tokens (page j/2, slots 8*(j%2) + e), e = 0..7,
//   which is also the k-slot order of group j in the PV product.
#include <float.h>
#include <math.h>

#include <atomic>
#include <type_traits>

#include "kvd_internal.h"
#include "kvdecode.h"

namespace kvd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

constexpr int kLutCopies = 32;   // copies of each codebook pair table (one per LDS bank pair)
// K pair table (codebook K): hi dwords of entry e at e * 256 + [0, 128), lo dwords 4 entries
// further on, at (e + 4) * 256 + [128, 256): the two reads of one entry are kKLoOffset bytes
// apart, more than a two-address LDS read can span, so each lands in its own register.
constexpr int kKLoOffset = 4 * 256 + 128;
constexpr int kKTableBytes = (256 + 4) * 256;
constexpr int kVTableBytes = 256 * 256;

constexpr float kLog2e = 1.4426950408889634f;

// How K and V of each format are stored:
//   K codebook (Turbo4, Turbo3): rotated-codebook indices with per-token norms;
//   K FP8 (FP8, Turbo8): E4M3FN codes with one scale per KV head, not rotated;
//   V codebook (Turbo4, Turbo3, Turbo8): rotated 4-bit codebook indices with per-token norms.
template <int FMT>
constexpr bool k_codebook() { return FMT == KVD_TURBO4 || FMT == KVD_TURBO3; }
template <int FMT>
constexpr bool k_fp8() { return FMT == KVD_FP8_E4M3 || FMT == KVD_TURBO8; }
template <int FMT>
constexpr bool v_codebook() { return k_codebook<FMT>() || FMT == KVD_TURBO8; }
// LDS byte of the V pair table: after the K table (codebook K), else 0.  The lane's V address
// comes from one v_perm with byte 2 = 1 (64 KB) plus this constant's remaining 1024 bytes.
template <int FMT>
constexpr int v_table_base() { return k_codebook<FMT>() ? kKTableBytes : 0; }
template <int FMT, int D>
constexpr int k_code() { return FMT == KVD_BF16 ? 32 * D : k_fp8<FMT>() ? 16 * D : FMT == KVD_TURBO4 ? 8 * D : 6 * D; }
template <int FMT, int D>
constexpr int v_code() { return FMT == KVD_BF16 ? 32 * D : FMT == KVD_FP8_E4M3 ? 16 * D : 8 * D; }
// Bytes of one (page, KV head) chunk: the stored elements, then (codebook-stored K or V) the 16
// fp32 per-token norms of the page.
template <int FMT, int D>
constexpr int k_chunk() { return k_code<FMT, D>() + (k_codebook<FMT>() ? 64 : 0); }
template <int FMT, int D>
constexpr int v_chunk() { return v_code<FMT, D>() + (v_codebook<FMT>() ? 64 : 0); }

// ------------------------------------------------------------------------------------------
// small helpers
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Max over the four 16-lane groups (rows) of a wave, returned in every lane.  gfx950's
// permlane swaps exchange rows 1<->0, 3<->2 (16) and rows 2,3<->0,1 (32) in registers, without
// LDS traffic.
// The max is v_max_f32 written out: the swap results arrive as integers, and fmaxf on them
// would first quiet possible signalling NaNs (an extra v_max per operand); nothing here
// produces one.
__device__ __forceinline__ float max_over_groups(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    uint32_t w, r;
    asm("v_max_f32 %0, %1, %2" : "=v"(w) : "v"(a[0]), "v"(a[1]));
    const auto c = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(c[0]), "v"(c[1]));
    return __uint_as_float(r);
}

// 4 E4M3FN codes (little-endian bytes of w) -> 4 bf16 in two packed pairs.  Exact: every
// E4M3FN value is a bf16 value.  gfx950 decodes OCP E4M3FN natively.
__device__ __forceinline__ u32x2 fp8x4_to_bf16(uint32_t w) {
    bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Codebook pair tables.  Entry (i0 + n * i1), n = 16 (4-bit) or 8 (3-bit), holds packed fp16
// dwords of the two levels (c[i0], c[i1]).  Entries are 256 bytes apart, and each table is
// stored kLutCopies = 32 times so that lane l reads copy l % 32: the lanes of one LDS pass then
// hit different banks whatever the indices (a single shared table costs about 3.3x more LDS
// cycles for random indices).  The address of entry b (a byte of the index word w) is
// lanebase.byte0 | b << 8 | lanebase.byte2 << 16, one v_perm_b32.
//
// V table (after the K table, else at LDS byte 0): copy c of entry e is the dword
// fp16(c[i0]) | fp16(c[i1]) << 16 at e * 256 + c * 4 (lanebase = (l % 32) * 4 plus the table's
// offset; the upper half of each 256-byte row is unused).  Four reads give eight indices as one
// MFMA operand, fp16 k-slots [c0 .. c7], against P' in the same slots.
//
// K table (codebook K, LDS byte 0): levels as hi + lo fp16 pairs, hi = hi(c[i0]) | hi(c[i1]) << 16
// and lo = lo(c[i0]) | lo(c[i1]) << 16 with c ~= hi + lo, the two halves stored separately:
// copy c of entry e's hi dword at
// e * 256 + c * 4 and of its lo dword kKLoOffset bytes further on (lanebase = (l % 32) * 4).
// Eight reads give eight indices as two plain operands, k-slots [h0 .. h7] and [l0 .. l7], so
// the query operand needs no repeated slots: hi * q_hi + lo * q_hi + hi * q_lo takes three MFMAs
// per eight elements and 8 VGPRs of query per 32 elements.
// V table: 8 4-bit indices (index e at bits 4e of w) -> one operand.
__device__ __forceinline__ u32x4 vlut_nib8(const char* lds, uint32_t lanebase, uint32_t w) {
    u32x4 a;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t addr = __builtin_amdgcn_perm(w, lanebase, (12u << 24) | (2u << 16) | ((4u + k) << 8));
        a[k] = *reinterpret_cast<const uint32_t*>(lds + addr);
    }
    return a;
}
// K table: 8 4-bit indices (index e at bits 4e of w) -> hi and lo operands.
__device__ __forceinline__ void klut_nib8(const char* lds, uint32_t lanebase, uint32_t w,
                                          u32x4& ahi, u32x4& alo) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t addr = __builtin_amdgcn_perm(w, lanebase, (12u << 24) | (2u << 16) | ((4u + k) << 8));
        ahi[k] = *reinterpret_cast<const uint32_t*>(lds + addr);
        alo[k] = *reinterpret_cast<const uint32_t*>(lds + addr + kKLoOffset);
    }
}
// K table: 8 3-bit indices (index e at bits 3e of the low 24 bits of f), as 6-bit pair indices.
__device__ __forceinline__ void klut_tri8(const char* lds, uint32_t lanebase, uint32_t f,
                                          u32x4& ahi, u32x4& alo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t addr = (__builtin_amdgcn_ubfe(f, 6 * i, 6) << 8) | lanebase;
        ahi[i] = *reinterpret_cast<const uint32_t*>(lds + addr);
        alo[i] = *reinterpret_cast<const uint32_t*>(lds + addr + kKLoOffset);
    }
}
// The 24-bit field holding indices 8h..8h+7 of a 32-index, 3-bit group (w0..w2 = its 12 bytes).
__device__ __forceinline__ uint32_t tri_field(uint32_t w0, uint32_t w1, uint32_t w2, int h) {
    switch (h) {
        case 0: return w0;
        case 1: return (w0 >> 24) | (w1 << 8);
        case 2: return (w1 >> 16) | (w2 << 16);
        default: return w2 >> 8;
    }
}

// fp32 pair -> (hi, lo) fp16 pairs with x ~= hi + lo.
__device__ __forceinline__ void f16_hilo(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    const f16x2 h = {(_Float16)x0, (_Float16)x1};
    const f16x2 l = {(_Float16)(x0 - (float)h[0]), (_Float16)(x1 - (float)h[1])};
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
}

// Power of two 2^-e with max_abs * 2^-e in [0.5, 1) (1 when max_abs is 0 or not finite).
__device__ __forceinline__ float pow2_normaliser(float max_abs) {
    if (!(max_abs > 0.0f) || !isfinite(max_abs)) return 1.0f;
    int e;
    frexpf(max_abs, &e);
    return ldexpf(1.0f, -e);
}

// In-place unnormalised Walsh-Hadamard transform (Sylvester order) of `rows` rows of length D
// in LDS.  Every thread of the block must call it.
template <int D>
__device__ void fwht_rows(float* buf, int rows, int tid, int nthreads) {
#pragma unroll 1
    for (int h = 1; h < D; h <<= 1) {
        for (int i = tid; i < rows * (D / 2); i += nthreads) {
            const int r = i / (D / 2), k = i % (D / 2);
            const int i0 = r * D + (k / h) * 2 * h + (k % h), i1 = i0 + h;
            const float a = buf[i0], c = buf[i1];
            buf[i0] = a + c;
            buf[i1] = a - c;
        }
        __syncthreads();
    }
}

struct SeqInfo {
    int L, lo, W;
    bool bad, split;
};

// Range [lo, L) of the keys any query of sequence b attends to and whether it is split into
// partitions.  With a chunk of nq queries (the last nq positions), query i at position
// L - nq + i sees [max(0, L - nq + i + 1 - W), L - nq + i] under a window W, so the sequence's
// range starts at query 0's window.  MQ = false: one query per sequence (nq = 1).
template <bool MQ>
__device__ __forceinline__ SeqInfo seq_info(const LaunchParams& p, int b) {
    SeqInfo s;
    const int nq = MQ ? p.nq : 1;
    // one value per workgroup: keep it in scalar registers so loops over it stay uniform
    int L = __builtin_amdgcn_readfirstlane(p.ctx[b]);
    const int W = p.win ? __builtin_amdgcn_readfirstlane(p.win[b]) : 0;
    s.bad = (L < 0) || (L > p.max_ctx) || (W < 0) || (MQ && L > 0 && L < nq);
    if (s.bad) L = 0;
    s.L = L;
    s.W = W;
    s.lo = W > 0 ? max(0, L - nq + 1 - W) : 0;
    const int span = L - s.lo;
    s.split = p.part_mode == kPartFixed ? true
            : (p.part_mode == kPartNever ? false : span >= kAutoSplitMin);
    return s;
}

// Runs of a split sequence.  A run is p.run_tokens consecutive tokens (a whole number of
// partitions, or of page pairs covering at least one partition) counted from the first token
// of the first partition the attended range touches (base = plo * part_size); a workgroup of
// kw waves walks a block of kw consecutive runs, one per wave, and its merged triple goes to
// workspace slot plo + (block index).  With p.run_skew = s > 0 the runs of even blocks are
// T + s tokens long and those of odd blocks T - s (T = p.run_tokens): block x starts at
// base + (x / 2) * 2 kw T + (x % 2) * kw (T + s).  Even blocks run on the even XCDs (see the
// grid order), which read the random pages of a BF16 / FP8 cache faster.  With also
// p.early_skew = e > 0 (the grid holds exactly two workgroups per CU and an even number
// 2H = p.run_pairs of block pairs) both runs of pairs H .. 2H - 1, which the grid dispatches
// first, are e tokens longer, and those of pairs 0 .. H - 1 e tokens shorter: the pairs are
// 2 kw (T + e) and 2 kw (T - e) tokens long.
struct RunBlocks {
    int plo, base, n;   // first partition, its first token, blocks of the sequence
};
// Length of the runs of the even block of pair q, and the pair's first token past base.
__device__ __forceinline__ int even_run(const LaunchParams& p, int q) {
    const int e = q >= (p.run_pairs >> 1) ? p.early_skew : -p.early_skew;
    return p.run_tokens + p.run_skew + e;
}
__device__ __forceinline__ int64_t pair_start(const LaunchParams& p, int kw, int q) {
    const int64_t H = p.run_pairs >> 1;
    const int64_t late = 2LL * kw * (p.run_tokens - p.early_skew);
    const int64_t early = 2LL * kw * (p.run_tokens + p.early_skew);
    return q <= H ? q * late : H * late + (q - H) * early;
}
__device__ __forceinline__ RunBlocks run_blocks(const LaunchParams& p, const SeqInfo& si, int kw) {
    RunBlocks r;
    r.plo = si.lo / p.part_size;
    r.base = r.plo * p.part_size;
    const int span = si.L - r.base;
    if (p.run_skew == 0) {
        const int runs = (span + p.run_tokens - 1) / p.run_tokens;
        r.n = (runs + kw - 1) / kw;
    } else if (p.early_skew == 0) {
        const int64_t two = 2LL * kw * p.run_tokens;   // tokens of an even and an odd block
        const int64_t q = span / two, rem = span - q * two;
        r.n = (int)(2 * q) + (rem == 0 ? 0 : rem <= (int64_t)kw * (p.run_tokens + p.run_skew) ? 1 : 2);
    } else if (span <= 0) {
        r.n = 0;
    } else {
        // the pair holding the range's last token, then whether its odd block is reached
        const int64_t H = p.run_pairs >> 1;
        const int64_t late = 2LL * kw * (p.run_tokens - p.early_skew);
        const int64_t early = 2LL * kw * (p.run_tokens + p.early_skew);
        const int q = (int)(span <= H * late ? (span + late - 1) / late - 1
                                             : H + (span - H * late + early - 1) / early - 1);
        r.n = 2 * q + (span - pair_start(p, kw, q) <= (int64_t)kw * even_run(p, q) ? 1 : 2);
    }
    return r;
}
// First token and run length of block x.
__device__ __forceinline__ void block_runs(const LaunchParams& p, int base, int x, int kw,
                                           int64_t& start, int& len) {
    if (p.run_skew == 0) {
        start = base + (int64_t)x * kw * p.run_tokens;
        len = p.run_tokens;
        return;
    }
    if (p.early_skew == 0) {
        const int tf = p.run_tokens + p.run_skew;
        start = base + (int64_t)(x >> 1) * 2 * kw * p.run_tokens + (int64_t)(x & 1) * kw * tf;
        len = (x & 1) ? p.run_tokens - p.run_skew : tf;
        return;
    }
    const int q = x >> 1, ev = even_run(p, q);
    start = base + pair_start(p, kw, q) + (int64_t)(x & 1) * kw * ev;
    len = (x & 1) ? ev - 2 * p.run_skew : ev;
}

// ------------------------------------------------------------------------------------------
// per-format raw registers of one page pair, as loaded from HBM
// ------------------------------------------------------------------------------------------
template <int FMT, int D> struct PairRaw;
template <int D> struct PairRaw<KVD_BF16, D> {      // K [D/8][16][8], V [D][16] bf16
    u32x4 kx[D / 32], ky[D / 32];
    u32x4 v[D / 16];
};
template <int D> struct PairRaw<KVD_FP8_E4M3, D> {  // K [D/16][16][16], V [D][16] bytes
    u32x4 kx[D / 64], ky[D / 64];
    u32x2 v[D / 16];
};
template <> struct PairRaw<KVD_TURBO4, 128> {       // K [4][16][16 B], V [128][8 B], norms
    u32x4 kx, ky;
    uint32_t v[8];
    f32x4 kn0, kn1, vn0, vn1;
};
template <> struct PairRaw<KVD_TURBO3, 128> {       // K [4][16][12 B], V [128][8 B], norms
    uint32_t kx[3], ky[3];
    uint32_t v[8];
    f32x4 kn0, kn1, vn0, vn1;
};
template <> struct PairRaw<KVD_TURBO8, 128> {       // K [8][16][16] bytes, V [128][8 B], V norms
    u32x4 kx[2], ky[2];
    uint32_t v[8];
    f32x4 vn0, vn1;
};

// Per-lane placement of the pair's tokens (see the header comment).
struct LaneMap {
    int n, j;
    int a_sel, a_pos;    // QK A row n: page (0 = A, 1 = B) and slot of its tile-X token
    int v_sel, v_pos0;   // softmax / PV group j: page and first of its eight slots
};

template <int FMT, int D>
__device__ __forceinline__ void load_pair(PairRaw<FMT, D>& r, const LaunchParams& p,
                                          const LaneMap& ln, size_t headA, size_t headB) {
    const uint8_t* kch = p.k + (ln.a_sel ? headB : headA) * (size_t)k_chunk<FMT, D>();
    const uint8_t* vch = p.v + (ln.v_sel ? headB : headA) * (size_t)v_chunk<FMT, D>();
    if constexpr (FMT == KVD_BF16) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {   // x-vector 4s + j of the lane's tokens
            const uint8_t* base = kch + 1024 * s + 256 * ln.j + 16 * ln.a_pos;
            r.kx[s] = *reinterpret_cast<const u32x4*>(base);
            r.ky[s] = *reinterpret_cast<const u32x4*>(base + 64);
        }
#pragma unroll
        for (int i = 0; i < D / 16; ++i)
            r.v[i] = *reinterpret_cast<const u32x4*>(vch + (16 * i + ln.n) * 32 + 2 * ln.v_pos0);
    } else if constexpr (FMT == KVD_FP8_E4M3) {
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {   // x-vector 4i + j (16 codes)
            const uint8_t* base = kch + 1024 * i + 256 * ln.j + 16 * ln.a_pos;
            r.kx[i] = *reinterpret_cast<const u32x4*>(base);
            r.ky[i] = *reinterpret_cast<const u32x4*>(base + 64);
        }
#pragma unroll
        for (int i = 0; i < D / 16; ++i)
            r.v[i] = *reinterpret_cast<const u32x2*>(vch + (16 * i + ln.n) * 16 + ln.v_pos0);
    } else if constexpr (FMT == KVD_TURBO8) {   // K as FP8, V and its norms as Turbo4
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const uint8_t* base = kch + 1024 * i + 256 * ln.j + 16 * ln.a_pos;
            r.kx[i] = *reinterpret_cast<const u32x4*>(base);
            r.ky[i] = *reinterpret_cast<const u32x4*>(base + 64);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            r.v[i] = *reinterpret_cast<const uint32_t*>(vch + (16 * i + ln.n) * 8 + ln.v_pos0 / 2);
        // the V norms of the lane's eight softmax tokens, after the V chunk's indices
        const float* vn = reinterpret_cast<const float*>(vch + v_code<FMT, D>()) + ln.v_pos0;
        r.vn0 = *reinterpret_cast<const f32x4*>(vn);
        r.vn1 = *reinterpret_cast<const f32x4*>(vn + 4);
    } else {
        if constexpr (FMT == KVD_TURBO4) {   // 32-index group j of the lane's tokens
            const uint8_t* base = kch + 256 * ln.j + 16 * ln.a_pos;
            r.kx = *reinterpret_cast<const u32x4*>(base);
            r.ky = *reinterpret_cast<const u32x4*>(base + 64);
        } else {
            const uint32_t* bx = reinterpret_cast<const uint32_t*>(kch + 192 * ln.j + 12 * ln.a_pos);
            const uint32_t* by = reinterpret_cast<const uint32_t*>(kch + 192 * ln.j + 12 * (ln.a_pos + 4));
#pragma unroll
            for (int w = 0; w < 3; ++w) { r.kx[w] = bx[w]; r.ky[w] = by[w]; }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            r.v[i] = *reinterpret_cast<const uint32_t*>(vch + (16 * i + ln.n) * 8 + ln.v_pos0 / 2);
        // the K and V norms of the lane's eight softmax tokens (page v_sel), after the indices
        // of that page's K and V chunks
        const float* kn = reinterpret_cast<const float*>(
            p.k + (ln.v_sel ? headB : headA) * (size_t)k_chunk<FMT, D>() + k_code<FMT, D>()) + ln.v_pos0;
        const float* vn = reinterpret_cast<const float*>(vch + v_code<FMT, D>()) + ln.v_pos0;
        r.kn0 = *reinterpret_cast<const f32x4*>(kn);
        r.kn1 = *reinterpret_cast<const f32x4*>(kn + 4);
        r.vn0 = *reinterpret_cast<const f32x4*>(vn);
        r.vn1 = *reinterpret_cast<const f32x4*>(vn + 4);
    }
}

// ------------------------------------------------------------------------------------------
// in-register dequantisation: MFMA operands of one page pair
// ------------------------------------------------------------------------------------------
// The A operands of QK step s (head elements 32s .. 32s + 31 in the order of the query operand)
// for the pair's two 16-token tiles X and Y.  BF16 / FP8 K (also Turbo8 K): one bf16x8 operand
// per tile in x0 / y0 (FP8 -> bf16 is exact); x1 / y1 are zero.  Codebook K: the fp16 hi parts
// of the lane's eight elements in x0 (y0) and their lo parts in x1 (y1), from the K table.
template <int FMT, int D>
__device__ __forceinline__ void k_operands(const PairRaw<FMT, D>& r, int s, const char* lds,
                                           uint32_t kbase, u32x4& x0, u32x4& x1, u32x4& y0,
                                           u32x4& y1) {
    x1 = y1 = u32x4{0u, 0u, 0u, 0u};
    if constexpr (FMT == KVD_BF16) {
        x0 = r.kx[s];
        y0 = r.ky[s];
    } else if constexpr (k_fp8<FMT>()) {
        const int i = s / 2, h = s % 2;   // codes 8h .. 8h + 7 of x-vector 4i + j
        const u32x2 ax0 = fp8x4_to_bf16(r.kx[i][2 * h]), ax1 = fp8x4_to_bf16(r.kx[i][2 * h + 1]);
        const u32x2 ay0 = fp8x4_to_bf16(r.ky[i][2 * h]), ay1 = fp8x4_to_bf16(r.ky[i][2 * h + 1]);
        x0 = u32x4{ax0[0], ax0[1], ax1[0], ax1[1]};
        y0 = u32x4{ay0[0], ay0[1], ay1[0], ay1[1]};
    } else if constexpr (FMT == KVD_TURBO4) {
        klut_nib8(lds, kbase, r.kx[s], x0, x1);
        klut_nib8(lds, kbase, r.ky[s], y0, y1);
    } else {
        klut_tri8(lds, kbase, tri_field(r.kx[0], r.kx[1], r.kx[2], s), x0, x1);
        klut_tri8(lds, kbase, tri_field(r.ky[0], r.ky[1], r.ky[2], s), y0, y1);
    }
}

// The A operand of PV tile t (head elements 16t + n, the lane's eight tokens as k-slots):
// bf16x8 for BF16 / FP8 V, fp16x8 from the V pair table for codebook V.
template <int FMT, int D>
__device__ __forceinline__ u32x4 v_operand(const PairRaw<FMT, D>& r, int t, const char* lds,
                                           uint32_t vbase) {
    if constexpr (FMT == KVD_BF16) {
        return r.v[t];
    } else if constexpr (FMT == KVD_FP8_E4M3) {
        const u32x2 a0 = fp8x4_to_bf16(r.v[t][0]), a1 = fp8x4_to_bf16(r.v[t][1]);
        return u32x4{a0[0], a0[1], a1[0], a1[1]};
    } else {
        return vlut_nib8(lds + (v_table_base<FMT>() & 0xFFFF), vbase, r.v[t]);
    }
}

// Codebook levels a workgroup's tables are built from: the two levels of this thread's table
// entry e = tid % 256 (entry i0 + n i1 holds levels i0 and i1; n = 2^kbits for K, 16 for V; the
// entry fill_tables gives the thread) and the largest level magnitudes.  The array holds 2^kbits K levels then 16 V levels
// (Turbo8: the 16 V levels).
struct Levels {
    float k0, k1, v0, v1, kmax, vmax;
};
template <int FMT>
__device__ __forceinline__ Levels load_levels(const float* codebook, int kbits, int tid) {
    constexpr bool kKcb = k_codebook<FMT>();
    Levels lv{0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int kl = kKcb ? 1 << kbits : 0;
    if constexpr (kKcb) {
        // a fixed trip count (one scalar load); the array holds kl + 16 >= 24 floats
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float c = fabsf(codebook[i]);
            lv.kmax = i < kl ? fmaxf(lv.kmax, c) : lv.kmax;
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) lv.vmax = fmaxf(lv.vmax, fabsf(codebook[kl + i]));
    const int e = tid & 255;
    if constexpr (kKcb) {
        lv.k0 = codebook[e % kl];
        lv.k1 = codebook[(e / kl) % kl];
    }
    lv.v0 = codebook[kl + (e & 15)];
    lv.v1 = codebook[kl + (e >> 4)];
    return lv;
}

// Fills the conflict-free pair tables (K table at LDS byte 0 for codebook K, then the V table)
// with the levels scaled by the power-of-two normalisers ksc / vsc.  NT threads (a multiple of
// 256): thread t takes entry t % 256 and every (NT / 256)-th of its sixteen 16-byte slots
// (K: slots 0..7 hold four hi copies each, 8..15 four lo copies, kKLoOffset - 128 bytes
// further on; V: slots 0..7 hold four copies each, 8..15 are unused).
// The slot order is staggered by entry, so the 16 lanes of a store pass write 16 different
// 16-byte bank groups (entries are 256 bytes apart: the same slot of every entry would sit in
// the same banks).
template <int FMT, int NT>
__device__ __forceinline__ void fill_tables(char* lds, int tid, const Levels& lv, float ksc,
                                            float vsc) {
    static_assert(NT % 256 == 0, "whole entries per thread group");
    constexpr bool kKcb = k_codebook<FMT>();
    constexpr int kParts = NT / 256;
    const int e = tid & 255, part = tid >> 8;
    uint32_t kh = 0u, kl = 0u;
    if constexpr (kKcb) f16_hilo(lv.k0 * ksc, lv.k1 * ksc, kh, kl);
    const f16x2 vp = {(_Float16)(lv.v0 * vsc), (_Float16)(lv.v1 * vsc)};
    const uint32_t vh = __builtin_bit_cast(uint32_t, vp);
    const u32x4 khi = {kh, kh, kh, kh}, klo = {kl, kl, kl, kl}, vv = {vh, vh, vh, vh};
    char* const vt = lds + v_table_base<FMT>();
#pragma unroll
    for (int i = 0; i < (16 + kParts - 1) / kParts; ++i) {
        const int v = part + i * kParts;
        if (kParts * i + kParts <= 16 || v < 16) {
            const int slot = (v + e) & 15;
            if constexpr (kKcb)
                *reinterpret_cast<u32x4*>(lds + e * 256 + slot * 16 + (slot < 8 ? 0 : kKLoOffset - 128)) =
                slot < 8 ? khi : klo;
            if (slot < 8) *reinterpret_cast<u32x4*>(vt + e * 256 + slot * 16) = vv;
        }
    }
}

__device__ __forceinline__ LaneMap lane_map(int lane) {
    LaneMap ln;
    ln.n = lane & 15;
    ln.j = lane >> 4;
    ln.a_sel = ln.n >> 3;
    ln.a_pos = 8 * ((ln.n >> 2) & 1) + (ln.n & 3);
    ln.v_sel = ln.j >> 1;
    ln.v_pos0 = 8 * (ln.j & 1);
    return ln;
}

// ------------------------------------------------------------------------------------------
// phase 1: partitioned attention
// ------------------------------------------------------------------------------------------
// Grid (run blocks) * Hkv * units * B (1-D), W waves per workgroup.  For a split sequence
// wave w of the workgroup of run block x owns the block's run w (run_blocks / block_runs:
// whole page pairs from the first attended partition's start, at least one partition) and
// streams through it without draining its load pipeline (the online softmax merges as it
// goes); the workgroup merges its W runs' triples through LDS into one, at slot plo + x, and
// the reduce merges the blocks'.  For an unsplit sequence (block 0 only) the waves share the
// attended range (consecutive parts of its page pairs) and merge through LDS into the final
// rows.  Page pairs start at even page indices, so when the partition size is a multiple of
// 32 tokens (required for runs of more than one partition) no pair straddles two
// partitions.
template <int FMT, int D, bool CAP, int PF, bool MQ, bool WIDE, int NT>
__global__ __launch_bounds__(64 * waves_per_group(FMT), waves_per_simd(WIDE)) void partition_kernel(const LaunchParams p) {
    constexpr bool kKcb = k_codebook<FMT>();   // rotated query, K table, K norms
    constexpr bool kVcb = v_codebook<FMT>();   // V table, V norms, output in the rotated domain
    static_assert(NT == 1 || tile_pairs_built(FMT, MQ, WIDE), "query tiles per wave");
    constexpr int kRows = NT * kMaxGroup;      // query rows of one work unit
    constexpr int kW = waves_per_group(FMT);   // waves per workgroup
    constexpr int kThr = 64 * kW;
    constexpr int KS = D / 32;   // QK MFMA steps (k = 32 head elements each)
    constexpr int VT = D / 16;   // PV MFMA tiles (16 head elements each)
    static_assert(!kVcb || D == 128, "codebook formats are built for head_dim 128");
    using Raw = PairRaw<FMT, D>;

    // LDS.  BF16 / FP8 (4 waves): per-wave rows of the unsplit merge (rows 0..g-1), D + 4
    // floats apart so the 16 query rows a ds_write_b128 touches start in different banks.  The
    // area is sized (stage_rows) so that two workgroups fit per CU, or one in the WIDE layout:
    // it sets the occupancy.  Codebook-V formats (8 waves): the conflict-free pair tables at LDS
    // address 0 (K and V, 128 KB, one workgroup per CU for Turbo4 / Turbo3; V only, 64 KB, two
    // per CU for Turbo8), reused for the unsplit merge once every wave has finished its walk.
    constexpr int SR = kVcb ? kMaxGroup : stage_rows(D, WIDE);
    static_assert(SR >= kRows, "merge rows of a unit");
    constexpr int SD = D + 4;
    struct Merge {
        float m[kW][SR];
        float l[kW][SR];
        f32x4 o[kW][SR * SD / 4];
    };
    struct LdsStage {
        Merge st;
    };
    struct LdsTurbo {
        union {
            u32x4 lut[(v_table_base<FMT>() + kVTableBytes) / 16];   // [K table,] V table
            Merge st;
        } u;
        float row[kMaxGroup * D];                 // query rotation / output rotation
        float rowscale[kMaxGroup];
    };
    using Lds = typename std::conditional<kVcb, LdsTurbo, LdsStage>::type;
    __shared__ Lds lds;
    Merge& stg = [&]() -> Merge& { if constexpr (kVcb) return lds.u.st; else return lds.st; }();
    auto& sm_m = stg.m;
    auto& sm_l = stg.l;
    float (&sm_o)[kW][SR * SD] = *reinterpret_cast<float (*)[kW][SR * SD]>(&stg.o);
    const char* const lds_bytes = reinterpret_cast<const char*>(&lds);

    // 1-D grid, KV head fastest, then sequence, then the partition slot x.  Workgroups are
    // handed to the eight XCDs round-robin by linear id, so this order spreads every
    // sequence's work over the XCDs (with 8 KV heads each XCD gets one head of every
    // sequence); x fastest would pile the short sequences' work onto the XCDs of small x.
    // The query rows of one KV head are (query i of the chunk, head of the group), i-major:
    // p.nq * p.g rows (p.g for single-query decode).  More rows than kMaxGroup are split into
    // p.qt MFMA tiles of up to kMaxGroup rows; a work unit ("virtual head") takes NT of them,
    // so a KV head has p.qg = ceil(p.qt / NT) units, each processed like a KV head of its own
    // (its pages are read once per unit; NT tiles share each load and dequantisation).
    // Units that read the same lines run on one XCD at the same time, so its L2 fetches each
    // line once for all of them: the p.qg units of a KV head read the same pages.  With
    // m such consecutive units, within every full block of 8m workgroups, unit m * x + j goes
    // to linear id 8 * j + x (XCD x, dispatched in consecutive rounds).  A bijection on full
    // blocks, the identity on the tail.
    int wg = blockIdx.x;
    if (const int m = p.qg; m > 1) {
        const int blk = 8 * m;
        if (wg < (int)gridDim.x / blk * blk) {
            const int r = wg % blk;
            wg += (r & 7) * m + (r >> 3) - r;
        }
    }
    const int nvh = p.Hkv * p.qg;
    // Run blocks are dispatched last block first: only long sequences have work in the high
    // blocks, so in a ragged batch their runs start at once and the short sequences' runs (and
    // the empty high blocks of short sequences, which exit at once) fill in behind them, as a
    // longest-first schedule would; in a uniform batch the order changes nothing.
    const int nxb = (int)gridDim.x / (nvh * p.B);
    int vh, b, xb;
    if (p.run_skew == 0) {
        vh = wg % nvh;
        b = (wg / nvh) % p.B;
        xb = nxb - 1 - wg / (nvh * p.B);
    } else {
        // skewed runs (p.qg == 1, nxb even): the block index's parity is the workgroup id's,
        // so the even blocks, with the longer runs, land on the even XCDs (workgroups reach
        // the XCDs round-robin by id); blocks go out in pairs, last pair first
        const int rest = wg >> 1;
        vh = rest % nvh;
        b = (rest / nvh) % p.B;
        xb = 2 * (nxb / 2 - 1 - rest / (nvh * p.B)) + (wg & 1);
    }
    const int hk = vh / p.qg, unit = vh - hk * p.qg;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rbase = unit * kRows;                           // first row of the unit
    const int g = min(kRows, (MQ ? p.nq : 1) * p.g - rbase);  // rows in the unit
    const SeqInfo si = seq_info<MQ>(p, b);
    // q / out / workspace row (b, i, h) of tile row t (q and out are [B][nq][Hq][D]): row
    // rbase + t of the KV head is query i = (rbase + t) / g, head hk * g + (rbase + t) - i * g,
    // i.e. row0 + t + i * (Hq - g).  MQ = false: one query per sequence (p.nq == 1, i = 0).
    const size_t row0 = (size_t)b * (MQ ? p.nq : 1) * p.Hq + (size_t)hk * p.g + rbase;
    auto row_index = [&](int t) -> size_t {
        if constexpr (!MQ) return row0 + t;
        const int i = (rbase + t) / p.g;
        return row0 + t + (size_t)i * (p.Hq - p.g);
    };

    // Start-up loads of the codebook formats: the levels for the tables and (codebook K) the
    // query rows to rotate depend only on the launch and on this workgroup's head and
    // sequence.  They go out together here, ahead of the first wait on the sequence's length,
    // so the round trips overlap (issued one after another they took ~5 of the ~8 us
    // start-up).
    [[maybe_unused]] Levels lv{0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // codebook K: wave w rotates query rows w, w + kW, ... (lane l holds elements 2l, 2l + 1)
    constexpr int kQRows = kKcb ? (kMaxGroup + kW - 1) / kW : 1;
    [[maybe_unused]] uint32_t q_raw[kQRows];
    [[maybe_unused]] float q_s0 = 0.0f, q_s1 = 0.0f;
    if constexpr (kVcb) lv = load_levels<FMT>(p.codebook, p.kbits, tid);
    if constexpr (kKcb) {
        static_assert(D == 128, "two query elements per lane");
        q_s0 = p.sign[2 * lane];
        q_s1 = p.sign[2 * lane + 1];
#pragma unroll
        for (int u = 0; u < kQRows; ++u) {   // rows past g are clamped (loaded, never used)
            const int r = min(wave + kW * u, g - 1);
            q_raw[u] = *reinterpret_cast<const uint32_t*>(p.q + row_index(r) * D + 2 * lane);
        }
    }

    if (si.bad || si.L == 0) {
        if (xb == 0) {
            const float v = si.bad ? __builtin_nanf("") : 0.0f;
            for (int i = tid; i < g * D; i += kThr) p.out[row_index(i / D) * D + i % D] = v;
        }
        return;
    }
    // token range [lo, hi) of this wave (uniform per workgroup: whether any wave has work);
    // split waves also track their workspace slot and the next partition boundary
    int lo, hi, part_end = 0, run_slot = 0;
    if (si.split) {
        const RunBlocks rb = run_blocks(p, si, kW);
        if (xb >= rb.n) return;
        int64_t start;
        int len;
        block_runs(p, rb.base, xb, kW, start, len);
        run_slot = rb.plo + xb;
        lo = (int)max((int64_t)si.lo, start + (int64_t)wave * len);
        hi = (int)min((int64_t)si.L, start + (int64_t)(wave + 1) * len);
        part_end = min(hi, (lo / p.part_size + 1) * p.part_size);
    } else {
        if (xb != 0) return;
        const int pg0 = (si.lo / kPageTokens) & ~1, pg1 = (si.L - 1) / kPageTokens + 1;
        const int np = (pg1 - pg0 + 1) >> 1;
        const int per = (np + kW - 1) / kW;
        lo = max(si.lo, (pg0 + 2 * per * wave) * kPageTokens);
        hi = min(si.L, (pg0 + 2 * per * (wave + 1)) * kPageTokens);
    }
    const bool live = lo < hi;

    const LaneMap ln = lane_map(lane);
    const int n = ln.n, j = ln.j;
    // table copy of this lane: 4-byte K halves at byte 0, 8-byte V pairs after the K table
    const uint32_t kbase = (uint32_t)(lane & (kLutCopies - 1)) * 4u;
    const uint32_t vbase = (uint32_t)(lane & (kLutCopies - 1)) * 4u | (uint32_t)(v_table_base<FMT>() & 0x10000);

    // ---- query operand (B of the QK product): lane (n, j), step s -------------------------
    const int qn = min(n, g - 1);          // clamp the address; rows n >= g are zeroed
    const bool qlive = n < g;
    // tile u of the unit: rows 16u + n (NT > 1 only for BF16 / FP8)
    bool tlive[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) tlive[u] = kMaxGroup * u + n < g;
    // the lane's query in tile u: index in the chunk, position, and the keys
    // [row_lo, row_hi) it sees; the keys every row of the unit sees: [tile_lo, tile_hi) (the
    // unmasked fast path).  One query per sequence: every row sees the sequence's whole range.
    int q_i[NT], q_pos[NT], row_lo[NT], row_hi[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        q_i[u] = MQ ? (rbase + min(kMaxGroup * u + n, g - 1)) / p.g : 0;
        q_pos[u] = MQ ? si.L - p.nq + q_i[u] : si.L - 1;
        row_hi[u] = MQ ? q_pos[u] + 1 : si.L;
        row_lo[u] = MQ ? (si.W > 0 ? max(0, row_hi[u] - si.W) : 0) : si.lo;
    }
    const int tile_hi = MQ ? si.L - p.nq + rbase / p.g + 1 : si.L;
    const int tile_lo = MQ ? (si.W > 0 ? max(0, si.L - p.nq + (rbase + g - 1) / p.g + 1 - si.W) : 0)
                           : si.lo;
    u32x4 qop[NT][KS];                  // BF16 / FP8 K: q (bf16) of tile u for step s
    u32x4 qhi[kKcb ? KS : 1];           // codebook K: fp16 hi parts of q for step s
    u32x4 qlo[kKcb ? KS : 1];           // codebook K: fp16 lo parts
    float zscale;           // logit -> base-2 softmax argument (without per-token factors)
    float oscale = 1.0f;    // accumulator -> output units (FP8 V scale / codebook scales)
    float ksc = 1.0f;       // K table normaliser (codebook K)

    if constexpr (kVcb) {
        // codebook pair tables (levels scaled by a power of two so the largest magnitude is in
        // [0.5, 1)), from the levels loaded at the start
        ksc = pow2_normaliser(lv.kmax);
        const float vsc = pow2_normaliser(lv.vmax);
        fill_tables<FMT, kThr>(reinterpret_cast<char*>(&lds.u.lut[0]), tid, lv, ksc, vsc);
        oscale = 1.0f / vsc;
        // the tables are complete before any wave's walk reads them (codebook K: the query
        // rotation's barriers below do the same)
        if constexpr (!kKcb) __syncthreads();
    }
    if constexpr (kKcb) {
        // q_rot = H (s * q), one row per wave in registers: the butterfly stages of the
        // Sylvester-order transform in the usual order (element stride 1 inside the lane, then
        // strides 2 .. 64 across lanes 1 .. 32 apart), and the row's power-of-two normaliser;
        // rows and normalisers then go to LDS for every wave's operands (one barrier, which
        // also completes the tables)
        float* const sm_row = lds.row;
        auto& sm_rowscale = lds.rowscale;
#pragma unroll
        for (int u = 0; u < kQRows; ++u) {
            const int r = wave + kW * u;
            if (r < g) {
                const float a0 = bf16_bits_to_f32(q_raw[u] & 0xFFFFu) * q_s0;
                const float a1 = bf16_bits_to_f32(q_raw[u] >> 16) * q_s1;
                float b0 = a0 + a1, b1 = a0 - a1;
#pragma unroll
                for (int h = 1; h < 64; h <<= 1) {
                    const bool upper = (lane & h) != 0;
                    const float o0 = __shfl_xor(b0, h), o1 = __shfl_xor(b1, h);
                    b0 = upper ? o0 - b0 : b0 + o0;
                    b1 = upper ? o1 - b1 : b1 + o1;
                }
                float mx = fmaxf(fabsf(b0), fabsf(b1));
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
                sm_row[r * D + 2 * lane] = b0;
                sm_row[r * D + 2 * lane + 1] = b1;
                if (lane == 0) sm_rowscale[r] = pow2_normaliser(mx);
            }
        }
        __syncthreads();
        const float qs = sm_rowscale[qn];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int d0 = 32 * j + 8 * s;
            uint32_t h[4], l[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f16_hilo(sm_row[qn * D + d0 + 2 * i] * qs, sm_row[qn * D + d0 + 2 * i + 1] * qs,
                         h[i], l[i]);
                if (!qlive) h[i] = l[i] = 0u;
            }
            qhi[s] = u32x4{h[0], h[1], h[2], h[3]};
            qlo[s] = u32x4{l[0], l[1], l[2], l[3]};
        }
        zscale = p.softmax_scale * kLog2e / (qs * ksc * sqrtf((float)D));
    } else {
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            const uint16_t* qptr = p.q + row_index(min(kMaxGroup * u + n, g - 1)) * D;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int d0 = (FMT == KVD_BF16) ? 32 * s + 8 * j : 64 * (s / 2) + 16 * j + 8 * (s % 2);
                const u32x4 w = *reinterpret_cast<const u32x4*>(qptr + d0);
                qop[u][s] = tlive[u] ? w : u32x4{0u, 0u, 0u, 0u};
            }
        }
        zscale = p.softmax_scale * kLog2e;
        if constexpr (FMT == KVD_FP8_E4M3) {   // scales [2][Hkv]: K then V
            zscale *= p.scales[hk];
            oscale = p.scales[p.Hkv + hk];
        } else if constexpr (FMT == KVD_TURBO8) {   // scales: the [Hkv] K scales
            zscale *= p.scales[hk];
        }
    }
    const float cap_l2 = CAP ? p.softcap * kLog2e : 0.0f;      // cap in base-2 units
    const float inv_cap_l2 = CAP ? 1.0f / cap_l2 : 0.0f;
    // ALiBi slope of the lane's query head in each tile, in base-2 units (0 without ALiBi)
    const bool alibi = p.alibi != nullptr;
    float slope_l2[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u)
        slope_l2[u] = alibi ? p.alibi[hk * p.g + (rbase + min(kMaxGroup * u + n, g - 1) - q_i[u] * p.g)] * kLog2e
                            : 0.0f;

    // ---- state -------------------------------------------------------------------------
    f32x4 oacc[NT][VT];
    float m_run[NT], l_run[NT];   // per tile: softmax reference max (base 2) and sum
    float m_true[NT];             // per tile: the exact running max of the lane's logits
#pragma unroll
    for (int u = 0; u < NT; ++u) {
#pragma unroll
        for (int i = 0; i < VT; ++i) oacc[u][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        m_run[u] = -INFINITY;
        l_run[u] = 0.0f;
        m_true[u] = -INFINITY;
    }
    constexpr float kSigInit = 1.17549435e-38f;
    constexpr float kLazyLog2 = 8.0f, kLazySig = 16.0f;
    float sig_run = kSigInit;   // reference V norm (codebook formats), 1 / sig_run
    float inv_sig = 1.0f / kSigInit;
    bool bad_ids = false;

    // pair k covers pages pg0 + 2k and pg0 + 2k + 1 (pg0 even)
    const int pgLo = live ? lo / kPageTokens : 0;
    const int pg0 = pgLo & ~1, pg1 = live ? (hi - 1) / kPageTokens + 1 : 1;
    const int npairs = live ? (pg1 - pg0 + 1) >> 1 : 0;
    const_i32_ptr btrow = (const_i32_ptr)(p.bt + (size_t)b * p.max_blocks);

    // physical pages of pair k (scalar loads).  Only entries of pages inside [pgLo, pg1) are
    // read: a first page below the range or a missing second page reads the row of the
    // range's page next to it, whose tokens the mask then hides.  Ids outside the pool are
    // clamped and flagged.
    auto fetch_ids = [&](int k, int& pa, int& pb) {
        const int pgA = pg0 + 2 * k;
        pa = btrow[max(pgA, pgLo)];
        pb = btrow[min(pgA + 1, pg1 - 1)];
    };
    auto heads = [&](int pa, int pb, size_t& ha, size_t& hb) {
        if (pa < 0 || pa >= p.pool) { bad_ids = true; pa = 0; }
        if (pb < 0 || pb >= p.pool) { bad_ids = true; pb = 0; }
        ha = (size_t)pa * p.Hkv + hk;
        hb = (size_t)pb * p.Hkv + hk;
    };

    // ---- one pair's logits: S^T = K Q^T for its two 16-token tiles ------------------------
    // (one set of K operands per step serves all NT query tiles)
    auto qk = [&](Raw& r, f32x4 (&sx)[NT], f32x4 (&sy)[NT]) {
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            sx[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            sy[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if constexpr (!kKcb) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                u32x4 x0, x1, y0, y1;
                k_operands<FMT, D>(r, s, lds_bytes, kbase, x0, x1, y0, y1);
#pragma unroll
                for (int u = 0; u < NT; ++u) {
                    sx[u] = mfma_bf16(x0, qop[u][s], sx[u]);
                    sy[u] = mfma_bf16(y0, qop[u][s], sy[u]);
                }
            }
        } else {
            f32x4 sx2 = {0.f, 0.f, 0.f, 0.f}, sy2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                u32x4 x0, x1, y0, y1;
                k_operands<FMT, D>(r, s, lds_bytes, kbase, x0, x1, y0, y1);
                // k hi * q hi + k lo * q hi + k hi * q lo, two accumulator chains per tile
                sx[0] = mfma_f16(x0, qhi[s], sx[0]);
                sx2 = mfma_f16(x1, qhi[s], sx2);
                sy[0] = mfma_f16(y0, qhi[s], sy[0]);
                sy2 = mfma_f16(y1, qhi[s], sy2);
                sx2 = mfma_f16(x0, qlo[s], sx2);
                sy2 = mfma_f16(y0, qlo[s], sy2);
            }
            sx[0] += sx2;
            sy[0] += sy2;
        }
    };

    // ---- one pair: online softmax and PV, given its logits ----------------------------------
    // A pair index at or past npairs is a no-op: its token window is empty, so every logit
    // is -inf, no reference moves, p = 0 and the V values are zero.
    auto finish = [&](Raw& r, int k, const f32x4 (&sx)[NT], const f32x4 (&sy)[NT]) {
        const int pgA = pg0 + 2 * min(k, npairs - 1);
        const bool hasB = pgA + 1 < pg1;
        const int hi_k = k < npairs ? hi : lo;
        const bool full = MQ ? (pgA * kPageTokens >= max(lo, tile_lo)) && hasB &&
                                   ((pgA + 2) * kPageTokens <= min(hi_k, tile_hi))
                             : (pgA * kPageTokens >= lo) && hasB && ((pgA + 2) * kPageTokens <= hi_k);

        float z[NT][8];
#pragma unroll
        for (int u = 0; u < NT; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) { z[u][e] = sx[u][e] * zscale; z[u][4 + e] = sy[u][e] * zscale; }
        if constexpr (kKcb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) { z[0][e] *= r.kn0[e]; z[0][4 + e] *= r.kn1[e]; }
        }
        if constexpr (CAP) {   // cap * tanh(x / cap), evaluated in base-2 units
#pragma unroll
            for (int u = 0; u < NT; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float t = fast_exp2(2.0f * kLog2e * (z[u][e] * inv_cap_l2));
                    z[u][e] = cap_l2 * (1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + t));
                }
        }
        if (alibi) {   // + slope * (j - q_pos) for the lane's tokens j = tok0 .. tok0 + 7
            const int tok0 = (pgA + ln.v_sel) * kPageTokens + ln.v_pos0;
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                const float base = slope_l2[u] * (float)(tok0 - q_pos[u]);
#pragma unroll
                for (int e = 0; e < 8; ++e) z[u][e] += base + slope_l2[u] * (float)e;
            }
        }
        float vn[8];   // V norms (codebook V)
        if constexpr (kVcb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) { vn[e] = r.vn0[e]; vn[4 + e] = r.vn1[e]; }
        }
        // Tokens outside [lo, hi) (and a missing second page) are selected out, never
        // multiplied: their logits become -inf and their V values zero.  A query of a chunk
        // also drops the keys outside its own causal window (logits only: those tokens hold
        // real data).  Only pairs at the ends of a range can be partial; the test is uniform
        // over the wave.
        if (!full) {
            const int tok0 = (pgA + ln.v_sel) * kPageTokens + ln.v_pos0;
            uint32_t vmask = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = tok0 + e;
                const bool ok = (t >= lo) && (t < hi_k) && (ln.v_sel == 0 || hasB);
                vmask |= (ok ? 1u : 0u) << e;
#pragma unroll
                for (int u = 0; u < NT; ++u)
                    z[u][e] = (ok && (!MQ || (t >= row_lo[u] && t < row_hi[u]))) ? z[u][e] : -INFINITY;
            }
            if constexpr (kVcb) {
                // table levels are always finite, so zero norms (possibly NaN in unused slots)
                // make the masked P' exactly 0
#pragma unroll
                for (int e = 0; e < 8; ++e) vn[e] = ((vmask >> e) & 1u) ? vn[e] : 0.0f;
            } else if constexpr (FMT == KVD_BF16) {
                uint32_t mk[4];   // 16-bit lane masks of the eight V k-slots
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    mk[i] = (((vmask >> (2 * i)) & 1u) ? 0x0000FFFFu : 0u) |
                            (((vmask >> (2 * i + 1)) & 1u) ? 0xFFFF0000u : 0u);
#pragma unroll
                for (int t = 0; t < VT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) r.v[t][i] &= mk[i];
            } else {
                uint32_t mb[2];   // byte masks of the eight V codes (code 0 is +0.0)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    mb[h] = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        mb[h] |= (((vmask >> (4 * h + e)) & 1u) ? 0xFFu : 0u) << (8 * e);
                }
#pragma unroll
                for (int t = 0; t < VT; ++t) { r.v[t][0] &= mb[0]; r.v[t][1] &= mb[1]; }
            }
        }
        // maxima over the lane's eight tokens; m_true is reduced over the row's four lane
        // groups only once, at the end of the walk
        float mloc[NT];
        bool grow = false;
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            mloc[u] = z[u][0];
#pragma unroll
            for (int e = 1; e < 8; ++e) mloc[u] = fmaxf(mloc[u], z[u][e]);
            m_true[u] = fmaxf(m_true[u], mloc[u]);
            grow = grow || mloc[u] > m_run[u] + kLazyLog2;
        }
        // Lazy rescaling: the reference max m_run (and, for the codebook formats, the V-norm
        // reference sig_run) only moves when some query's new logits exceed it by more than
        // 2^kLazyLog2 (or a norm exceeds it kLazySig-fold), so P stays <= 2^8 (P' <= 2^12) and
        // the accumulator rescale is skipped on almost every pair.  The choice is wave-uniform
        // (a ballot of the lanes' own tests); only a rescale needs the maxima over the row's
        // four lane groups, which keep m_run and sig_run the same in all of them.  With several
        // query tiles, a tile moves its reference only when its own logits ask for it, exactly
        // as a one-tile walk would.
        float vloc = 0.0f;
        if constexpr (kVcb) {
#pragma unroll
            for (int e = 0; e < 8; ++e) vloc = fmaxf(vloc, vn[e]);
            grow = grow || (vloc > sig_run * kLazySig);
        }
        // (chunks of queries: maxima are clamped to -FLT_MAX where they enter a difference: a
        // query row that has not seen a key yet keeps m = -inf, and -inf - -inf would be NaN;
        // with one query per sequence every computed pair holds a key of the range)
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            [[maybe_unused]] float fsig = 1.0f;   // sigma_old / sigma_new (codebook V)
            if constexpr (kVcb) {
                vloc = max_over_groups(vloc);
                const float sig_new = fmaxf(sig_run, vloc);
                inv_sig = __builtin_amdgcn_rcpf(sig_new);
                fsig = sig_run * inv_sig;
                sig_run = sig_new;
            }
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                if (NT > 1 && __builtin_amdgcn_ballot_w64(mloc[u] > m_run[u] + kLazyLog2) == 0)
                    continue;
                const float m_new = fmaxf(m_run[u], max_over_groups(mloc[u]));
                float f = MQ ? fast_exp2(fmaxf(m_run[u], -FLT_MAX) - fmaxf(m_new, -FLT_MAX))
                             : fast_exp2(m_run[u] - m_new);
                l_run[u] *= f;
                if constexpr (kVcb) f *= fsig;
#pragma unroll
                for (int t = 0; t < VT; ++t) oacc[u][t] *= f;
                m_run[u] = m_new;
            }
        }
        float pe[NT][8];
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            float psum = 0.0f;
            const float m_ref = MQ ? fmaxf(m_run[u], -FLT_MAX) : m_run[u];
#pragma unroll
            for (int e = 0; e < 8; ++e) { pe[u][e] = fast_exp2(z[u][e] - m_ref); psum += pe[u][e]; }
            l_run[u] += psum;
        }

        if constexpr (kVcb) {
            // P' = p * vnorm / sigma, rounded once to fp16
            u32x4 pb;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f16x2 h = {(_Float16)(pe[0][2 * i] * (vn[2 * i] * inv_sig)),
                                 (_Float16)(pe[0][2 * i + 1] * (vn[2 * i + 1] * inv_sig))};
                pb[i] = __builtin_bit_cast(uint32_t, h);
            }
#pragma unroll
            for (int t = 0; t < VT; ++t)
                oacc[0][t] = mfma_f16(v_operand<FMT, D>(r, t, lds_bytes, vbase), pb, oacc[0][t]);
        } else {
            u32x4 phi[NT], plo[NT];
#pragma unroll
            for (int u = 0; u < NT; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t a = __float_as_uint(pe[u][2 * i]), c = __float_as_uint(pe[u][2 * i + 1]);
                    const uint32_t ah = a & 0xFFFF0000u, ch = c & 0xFFFF0000u;
                    phi[u][i] = (a >> 16) | ch;
                    bf16x2 l = {(__bf16)(pe[u][2 * i] - __uint_as_float(ah)),
                                (__bf16)(pe[u][2 * i + 1] - __uint_as_float(ch))};
                    plo[u][i] = __builtin_bit_cast(uint32_t, l);
                }
            // (one V operand per tile t serves all NT query tiles)
#pragma unroll
            for (int t = 0; t < VT; ++t) {
                const u32x4 vop = v_operand<FMT, D>(r, t, lds_bytes, vbase);
#pragma unroll
                for (int u = 0; u < NT; ++u) {
                    oacc[u][t] = mfma_bf16(vop, phi[u], oacc[u][t]);
                    oacc[u][t] = mfma_bf16(vop, plo[u], oacc[u][t]);
                }
            }
        }
    };

    auto compute = [&](Raw& r, int k) {
        f32x4 sx[NT], sy[NT];
        qk(r, sx, sy);
        finish(r, k, sx, sy);
    };

    // Codebook formats (8 waves, two per SIMD): the hardware issues from the older of a SIMD's
    // two waves first, so waves 4-7 fall behind waves 0-3.  The pair start with opposite
    // priorities and swap them at every partition boundary they cross.  The condition is
    // wave-uniform; pairs past the end cross nothing.
    bool prio_hi = (wave >> 2) & 1;
    if constexpr (kVcb) {
        if (prio_hi) __builtin_amdgcn_s_setprio(1);
    }
    auto partition_boundary = [&](int k) {
        if constexpr (kVcb) {
            const int tend = (pg0 + 2 * k + 2) * kPageTokens;   // first token after pair k
            if (k < npairs && tend >= part_end) {
                prio_hi = !prio_hi;
                if (prio_hi) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
                part_end = min(hi, part_end + p.part_size);
            }
        }
    };

    // ---- streaming walk over the wave's pairs ------------------------------------------
    // PF pairs are always in flight: buffer i holds pair k + i; after computing it, the same
    // buffer is refilled with pair k + i + PF.  Pair indices past the end are clamped to the
    // wave's last pair (its pages are already cached), so every load stays inside the
    // attended pages, and computes past the end are no-ops; the loop body is one basic block
    // with no early exit, so the loads stay in flight across the back-edge.
    if (live) {
        Raw buf[PF];
        int ida[PF], idb[PF];   // block-table ids of the pair each buffer is loaded with next
        const int klast = npairs - 1;
        // (issue order here must match the loop body's: buffer 0 first, K before V)
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            int pa, pb;
            size_t ha, hb;
            fetch_ids(min(i, klast), pa, pb);
            heads(pa, pb, ha, hb);
            __builtin_amdgcn_sched_barrier(0);
            load_pair<FMT, D>(buf[i], p, ln, ha, hb);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < PF; ++i) fetch_ids(min(PF + i, klast), ida[i], idb[i]);
        // The scheduling barriers keep each refill after the compute that frees its buffer:
        // vmcnt retires in issue order, so a refill hoisted above an older pair's compute
        // would make that compute wait for every younger load too.
#pragma unroll 1
        for (int k = 0; k < npairs; k += PF) {
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                compute(buf[i], k + i);
                if (si.split) partition_boundary(k + i);
                __builtin_amdgcn_sched_barrier(0);
                size_t ha, hb;
                heads(ida[i], idb[i], ha, hb);
                load_pair<FMT, D>(buf[i], p, ln, ha, hb);
                fetch_ids(min(k + i + 2 * PF, klast), ida[i], idb[i]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // ---- results ---------------------------------------------------------------------------
    // Split sequences: each wave's run gives a triple per query row -- m = the exact max logit
    // in base-2 units, l = the sum taken relative to it, o = O / l in output units (no
    // reference choice affects them; a row that saw no key of the run: m = -inf, l = 0, o = 0;
    // a wave with no run gives that too).  The workgroup's waves stage them in LDS and merge
    // them with the LSE rule into one triple for the workgroup's kW consecutive runs, written
    // to its slot plo + xb: a quarter (an eighth for the codebook formats) of the workspace
    // traffic of one triple per run, and of the reduce's reads.
    if (si.split) {
        const float osc = kVcb ? oscale * sig_run : oscale;
        if constexpr (kVcb) __syncthreads();   // the staging rows reuse the tables
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            const float mt = max_over_groups(m_true[u]);
            float lt = l_run[u] + __shfl_xor(l_run[u], 16);
            lt += __shfl_xor(lt, 32);
            const float sc = lt > 0.0f ? osc / lt : 0.0f;
            const float lx = lt > 0.0f ? lt * fast_exp2(m_run[u] - mt) : 0.0f;
            if (tlive[u]) {
                const int rr = kMaxGroup * u + n;
                if (j == 0) {
                    sm_m[wave][rr] = mt;
                    sm_l[wave][rr] = lx;
                }
#pragma unroll
                for (int t = 0; t < VT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sm_o[wave][rr * SD + 16 * t + 4 * j + r] = oacc[u][t][r] * sc;
            }
        }
        const bool wg_bad = __syncthreads_or(bad_ids ? 1 : 0) != 0;
        for (int i = tid; i < g * D; i += kThr) {
            const int r = i / D, d = i % D;
            float M = sm_m[0][r];
#pragma unroll
            for (int w = 1; w < kW; ++w) M = fmaxf(M, sm_m[w][r]);
            float wsum = 0.0f, acc = 0.0f;
#pragma unroll
            for (int w = 0; w < kW; ++w) {   // l > 0 implies a finite m, so M is finite too
                const float lw = sm_l[w][r];
                const float sc = lw > 0.0f ? lw * fast_exp2(sm_m[w][r] - M) : 0.0f;
                wsum += sc;
                acc += sm_o[w][r * SD + d] * sc;
            }
            const size_t slot = row_index(r) * p.P + run_slot;
            p.ws_o[slot * D + d] = wg_bad ? __builtin_nanf("") : (wsum > 0.0f ? acc / wsum : 0.0f);
            if (d == 0) {
                p.ws_m[slot] = M;
                p.ws_l[slot] = wsum;
            }
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        l_run[u] += __shfl_xor(l_run[u], 16);
        l_run[u] += __shfl_xor(l_run[u], 32);
    }
    if constexpr (kVcb) oscale *= sig_run;

    // unsplit: merge the waves through LDS, then write the final rows (the codebook formats'
    // merge rows reuse the tables, so every wave must have finished its walk first)
    if constexpr (kVcb) __syncthreads();
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        if (tlive[u]) {
            const int rr = kMaxGroup * u + n;
            if (j == 0) {
                sm_m[wave][rr] = m_run[u];
                sm_l[wave][rr] = l_run[u];
            }
#pragma unroll
            for (int t = 0; t < VT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sm_o[wave][rr * SD + 16 * t + 4 * j + r] = oacc[u][t][r] * oscale;
        }
    }
    const bool wg_bad = __syncthreads_or(bad_ids ? 1 : 0) != 0;
    for (int i = tid; i < g * D; i += kThr) {
        const int r = i / D, d = i % D;
        float M = sm_m[0][r];
#pragma unroll
        for (int w = 1; w < kW; ++w) M = fmaxf(M, sm_m[w][r]);
        float wsum = 0.0f, acc = 0.0f;
#pragma unroll
        for (int w = 0; w < kW; ++w) {
            const float sc = fast_exp2(sm_m[w][r] - M);   // 0 for waves without tokens
            wsum += sm_l[w][r] * sc;
            acc += sm_o[w][r * SD + d] * sc;
        }
        float o = acc / wsum;
        if (wg_bad) o = __builtin_nanf("");
        if constexpr (kVcb) lds.row[i] = o;
        else p.out[row_index(r) * D + d] = o;
    }
    if constexpr (kVcb) {   // inverse rotation of the final rows: diag(s) H o / sqrt(D)
        __syncthreads();
        fwht_rows<D>(lds.row, g, tid, kThr);
        const float rs = 1.0f / sqrtf((float)D);
        for (int i = tid; i < g * D; i += kThr)
            p.out[row_index(i / D) * D + i % D] = lds.row[i] * p.sign[i % D] * rs;
    }
}

// ------------------------------------------------------------------------------------------
// phase 2: log-sum-exp merge of the partition triples
// ------------------------------------------------------------------------------------------
// One wave per (query head, sequence x query of the chunk); lane l owns output elements
// E*l .. E*l + E - 1 (E = D / 64).  The partition kernel wrote one triple per workgroup of kW
// runs, at slots plo .. plo + blocks - 1 (run_blocks).  Triples are taken KB at a time (KB = 16 when a row has
// at most 32 of them, else 64): lane i < KB takes the (m, l) of triple base + i and every lane
// loads its slice of all KB outputs, so a block costs one memory round trip.  The block's
// weights are computed lane-parallel and broadcast with v_readlane; blocks after the first
// rescale the running sums to the new maximum (online LSE).  The short block spares a typical
// row (4 to 16 triples) the loads of 48 or more clamped duplicate slots (with one triple per
// run, 16 per row: C4 call 193.8 -> 192.3 us).
template <int FMT, int D>
__global__ __launch_bounds__(64) void reduce_kernel(const LaunchParams p) {
    constexpr bool kVcb = v_codebook<FMT>();   // partial outputs are in the rotated domain
    constexpr int E = D / 64;
    const int hq = blockIdx.x, bi = blockIdx.y, b = bi / p.nq, lane = threadIdx.x;
    const SeqInfo si = seq_info<true>(p, b);
    if (si.bad || si.L == 0 || !si.split) return;
    constexpr int kW = waves_per_group(FMT);      // runs per workgroup, merged into one triple
    const RunBlocks rb = run_blocks(p, si, kW);
    const int p0 = rb.plo, n = rb.n;              // first slot, triples of the sequence
    const size_t row = (size_t)bi * p.Hq + hq;    // out / workspace row (b, query, head)
    const float* ms = p.ws_m + row * p.P + p0;
    const float* ls = p.ws_l + row * p.P + p0;
    const float* os = p.ws_o + (row * p.P + p0) * D + E * lane;

    float M = -INFINITY, wsum = 0.0f, acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    auto merge_block = [&](auto kb, int base) {
        constexpr int KB = decltype(kb)::value;
        // indices past the end are clamped (their loads stay in bounds) and weighted 0
        const int q = min(base + lane, n - 1);
        const float mq = ms[q], lq = ls[q];
        float v[KB][E];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            const int qq = min(base + u, n - 1);
#pragma unroll
            for (int e = 0; e < E; ++e) v[u][e] = os[(size_t)qq * D + e];
        }
        __builtin_amdgcn_sched_barrier(0);   // keep all of the block's loads ahead of any use
        const bool in = lane < KB && base + lane < n;
        float mb = in ? mq : -INFINITY;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) mb = fmaxf(mb, __shfl_xor(mb, o));
        const float Mn = fmaxf(M, mb);
        // 0 on the first block (M = -inf); the clamp keeps a block in which this query row
        // has no key yet (m = -inf everywhere) from producing -inf - -inf
        const float sc = fast_exp2(fmaxf(M, -FLT_MAX) - fmaxf(Mn, -FLT_MAX));
        const float w = (in && lq > 0.0f) ? lq * fast_exp2(mq - Mn) : 0.0f;   // l = 0: no key
        wsum = wsum * sc + w;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] *= sc;
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += wu * v[u][e];
        }
        M = Mn;
    };
    if (n <= 32) {
#pragma unroll 1
        for (int base = 0; base < n; base += 16) merge_block(std::integral_constant<int, 16>{}, base);
    } else {
#pragma unroll 1
        for (int base = 0; base < n; base += 64) merge_block(std::integral_constant<int, 64>{}, base);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) wsum += __shfl_xor(wsum, o);
    const float inv = 1.0f / wsum;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= inv;

    if constexpr (kVcb) {   // diag(s) H o / sqrt(D): butterflies in registers, then lanes
        static_assert(E == 2, "codebook formats are built for head_dim 128");
        const float a0 = acc[0], a1 = acc[1];
        acc[0] = a0 + a1;
        acc[1] = a0 - a1;
#pragma unroll
        for (int h = 1; h < 64; h <<= 1) {   // elements d and d + 2h live in lanes l and l ^ h
            const bool upper = (lane & h) != 0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float other = __shfl_xor(acc[e], h);
                acc[e] = upper ? other - acc[e] : acc[e] + other;
            }
        }
        const float rs = 1.0f / sqrtf((float)D);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] *= p.sign[E * lane + e] * rs;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) p.out[row * D + E * lane + e] = acc[e];
}

// ------------------------------------------------------------------------------------------
// test export: dequantised gather
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_kernel(const GatherParams p) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= p.n * p.D) return;
    const int t = p.t0 + i / p.D, d = i % p.D;
    const int page = t / kPageTokens, pos = t % kPageTokens;
    const int phys = p.bt[(size_t)p.seq * p.max_blocks + page];
    if (phys < 0 || phys >= p.pool) {
        p.out[i] = __builtin_nanf("");
        return;
    }
    const size_t head = (size_t)phys * p.Hkv + p.kv_head;
    const uint8_t* ch = p.cache + head * p.chunk;
    float val;
    if (p.fmt == KVD_BF16) {
        const size_t off = p.is_v ? (size_t)d * 16 + pos : ((size_t)(d / 8) * 16 + pos) * 8 + d % 8;
        val = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(ch)[off]);
    } else if (p.fmt == KVD_FP8_E4M3 || (p.fmt == KVD_TURBO8 && !p.is_v)) {
        const size_t off = p.is_v ? (size_t)d * 16 + pos : ((size_t)(d / 16) * 16 + pos) * 16 + d % 16;
        const uint32_t w = reinterpret_cast<const uint32_t*>(ch)[off / 4];
        const u32x2 bf = fp8x4_to_bf16(w);
        const int e = off % 4;
        const uint32_t pair = bf[e / 2];
        val = bf16_bits_to_f32((e & 1) ? (pair >> 16) : (pair & 0xFFFFu));
        // FP8: scales [2][Hkv]; Turbo8: the [Hkv] K scales
        val *= p.fmt == KVD_TURBO8 ? p.scales[p.kv_head]
                                   : p.scales[(p.is_v ? p.Hkv : 0) + p.kv_head];
    } else {
        uint32_t idx;
        if (p.is_v) {
            const uint32_t w = reinterpret_cast<const uint32_t*>(ch + (size_t)d * 8)[pos / 8];
            idx = (w >> (4 * (pos % 8))) & 15u;
        } else if (p.fmt == KVD_TURBO4) {
            const uint32_t w = reinterpret_cast<const uint32_t*>(ch + ((size_t)(d / 32) * 16 + pos) * 16)[(d % 32) / 8];
            idx = (w >> (4 * (d % 8))) & 15u;
        } else {
            const uint32_t* g3 = reinterpret_cast<const uint32_t*>(ch + ((size_t)(d / 32) * 16 + pos) * 12);
            const int e = d % 32;
            idx = (tri_field(g3[0], g3[1], g3[2], e / 8) >> (3 * (e % 8))) & 7u;
        }
        // levels: 2^kbits K then 16 V (Turbo8: the 16 V levels); the page's 16 fp32 norms
        // follow the chunk's indices
        const bool t8 = p.fmt == KVD_TURBO8;
        const int kl = t8 ? 0 : 1 << p.kbits;
        const float lvl = p.codebook[(p.is_v ? kl : 0) + idx];
        val = reinterpret_cast<const float*>(ch + p.chunk - 64)[pos] * lvl;
    }
    p.out[i] = val;
}

// ------------------------------------------------------------------------------------------
// test export: the partition kernel's own MFMA operands of page pairs
// ------------------------------------------------------------------------------------------
// 512 threads (eight waves), the same table build as the partition kernel's codebook formats;
// wave w of workgroup x takes page pair pair0 + 8x + w of one (sequence, KV head) (pages 2k and
// 2k + 1 of the sequence), loads it with load_pair and the lane map of the partition kernel and
// forms the QK and PV operands with k_operands / v_operand.  Record of lane l (D + 16 words):
// for each QK step s: x0, x1, y0, y1; for each PV tile t: v, then four zero words; then K norms
// (8 floats of the lane's eight softmax tokens), V norms (8), zero where the format has none.
// A pair whose block table entry lies outside the pool writes all-ones records.
template <int FMT, int D>
__global__ __launch_bounds__(512) void operand_kernel(const OperandParams op) {
    constexpr bool kKcb = k_codebook<FMT>();
    constexpr bool kVcb = v_codebook<FMT>();
    constexpr int KS = D / 32, VT = D / 16, W = operand_words(D);
    __shared__ u32x4 lut[kVcb ? (v_table_base<FMT>() + kVTableBytes) / 16 : 1];
    const LaunchParams& p = op.lp;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const char* const lds_bytes = reinterpret_cast<const char*>(lut);
    if constexpr (kVcb) {
        const Levels lv = load_levels<FMT>(p.codebook, p.kbits, tid);
        fill_tables<FMT, 512>(reinterpret_cast<char*>(lut), tid, lv, pow2_normaliser(lv.kmax),
                              pow2_normaliser(lv.vmax));
        __syncthreads();
    }
    const int k = blockIdx.x * 8 + wave;
    if (k >= op.npairs) return;
    const int pair = op.pair0 + k;
    const LaneMap ln = lane_map(lane);
    const uint32_t kbase = (uint32_t)(lane & (kLutCopies - 1)) * 4u;
    const uint32_t vbase = (uint32_t)(lane & (kLutCopies - 1)) * 4u | (uint32_t)(v_table_base<FMT>() & 0x10000);
    uint32_t* rec = op.out + ((size_t)k * 64 + lane) * W;
    const int32_t* btrow = p.bt + (size_t)op.seq * p.max_blocks;
    const int pa = btrow[2 * pair], pb = btrow[2 * pair + 1];
    if (pa < 0 || pa >= p.pool || pb < 0 || pb >= p.pool) {
        for (int i = 0; i < W; ++i) rec[i] = 0xFFFFFFFFu;
        return;
    }
    PairRaw<FMT, D> r;
    load_pair<FMT, D>(r, p, ln, (size_t)pa * p.Hkv + op.kv_head, (size_t)pb * p.Hkv + op.kv_head);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        u32x4 x[4];
        k_operands<FMT, D>(r, s, lds_bytes, kbase, x[0], x[1], x[2], x[3]);
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(rec + 16 * s + 4 * i) = x[i];
    }
#pragma unroll
    for (int t = 0; t < VT; ++t) {
        *reinterpret_cast<u32x4*>(rec + D / 2 + 8 * t) = v_operand<FMT, D>(r, t, lds_bytes, vbase);
        *reinterpret_cast<u32x4*>(rec + D / 2 + 8 * t + 4) = u32x4{0u, 0u, 0u, 0u};
    }
    f32x4 nrm[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if constexpr (kKcb) { nrm[0] = r.kn0; nrm[1] = r.kn1; }
    if constexpr (kVcb) { nrm[2] = r.vn0; nrm[3] = r.vn1; }
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<f32x4*>(rec + D + 4 * i) = nrm[i];
}

template <int FMT, int D>
hipError_t launch_operands_t(const OperandParams& p, hipStream_t s) {
    return launch_kernel(operand_kernel<FMT, D>, dim3((p.npairs + 7) / 8), dim3(512), s, p);
}

// Pairs in flight per wave.  With every wave of the chip streaming random pages, fewer
// outstanding requests read HBM more efficiently.  FP8 32K partition kernel, A/B on one GPU:
// 195.6 us at one pair in flight (8 KB per wave) against 204.0 us at two; three pairs ran
// 1.4% slower than two, four slower still.  Turbo8 (FP8 K) 32K: 80.9 against 85.1 us.  BF16
// (16 KB per pair) runs the same at one or two.  Turbo4 / Turbo3 are bound by compute latency
// and need the second pair to cover it (one pair: 1.5-3% slower).
template <int FMT, bool WIDE>
constexpr int prefetch_depth() {
    return FMT == KVD_FP8_E4M3 || FMT == KVD_TURBO8 || WIDE ? 1 : 2;
}

template <int FMT, int D>
hipError_t launch_partitions_t(const LaunchParams& p, bool wide, dim3 grid, hipStream_t s) {
    constexpr int PF = prefetch_depth<FMT, false>();
    const dim3 block(64 * waves_per_group(FMT));
    if (p.nq > 1) {
        if constexpr (tile_pairs_built(FMT, true, false)) {
            // a chunk of queries with more than 16 rows per KV head: two query tiles per wave
            // (FP8 C4 shape with 8 queries per sequence, 64 rows per KV head: 367 us per call
            // with one tile per wave, 271 us with two at one pair in flight, 257 us at two)
            constexpr int PFQ = FMT == KVD_BF16 ? 1 : 2;
            if (p.nt == 2)
                return p.softcap > 0.0f ? launch_kernel(partition_kernel<FMT, D, true, PFQ, true, false, 2>, grid, block, s, p)
                                        : launch_kernel(partition_kernel<FMT, D, false, PFQ, true, false, 2>, grid, block, s, p);
        }
        return p.softcap > 0.0f ? launch_kernel(partition_kernel<FMT, D, true, PF, true, false, 1>, grid, block, s, p)
                                : launch_kernel(partition_kernel<FMT, D, false, PF, true, false, 1>, grid, block, s, p);
    }
    if constexpr (wide_layout_built(FMT, D, false)) {
        constexpr int PFW = prefetch_depth<FMT, true>();
        if (wide)
            return p.softcap > 0.0f ? launch_kernel(partition_kernel<FMT, D, true, PFW, false, true, 1>, grid, block, s, p)
                                    : launch_kernel(partition_kernel<FMT, D, false, PFW, false, true, 1>, grid, block, s, p);
    }
    if constexpr (tile_pairs_built(FMT, false, false)) {
        // two query tiles per wave (the second tile's registers leave BF16 one pair in flight)
        constexpr int PF2 = FMT == KVD_BF16 ? 1 : 2;
        if (p.nt == 2)
            return p.softcap > 0.0f ? launch_kernel(partition_kernel<FMT, D, true, PF2, false, false, 2>, grid, block, s, p)
                                    : launch_kernel(partition_kernel<FMT, D, false, PF2, false, false, 2>, grid, block, s, p);
    }
    return p.softcap > 0.0f ? launch_kernel(partition_kernel<FMT, D, true, PF, false, false, 1>, grid, block, s, p)
                            : launch_kernel(partition_kernel<FMT, D, false, PF, false, false, 1>, grid, block, s, p);
}
template <int FMT, int D>
hipError_t launch_reduce_t(const LaunchParams& p, hipStream_t s) {
    return launch_kernel(reduce_kernel<FMT, D>, dim3(p.Hq, p.B * p.nq), dim3(64), s, p);
}

// Workspace of the allocation-free entry point.  The host-side name `scratch` is a stand-in,
// not a device address: host code uses only the pointer hipGetSymbolAddress returns for the
// current device (each GPU holds its own copy of the array, at its own address).
static __device__ __align__(256) unsigned char scratch[kNoAllocWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];

}  // namespace

hipError_t noalloc_workspace(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // with the device current; two threads racing here store the same address
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_partitions(int fmt, bool wide, const LaunchParams& p, dim3 grid, hipStream_t s) {
    switch (fmt) {
        case KVD_BF16: return p.D == 64 ? launch_partitions_t<KVD_BF16, 64>(p, wide, grid, s)
                                        : launch_partitions_t<KVD_BF16, 128>(p, wide, grid, s);
        case KVD_FP8_E4M3: return p.D == 64 ? launch_partitions_t<KVD_FP8_E4M3, 64>(p, wide, grid, s)
                                            : launch_partitions_t<KVD_FP8_E4M3, 128>(p, wide, grid, s);
        case KVD_TURBO4: return launch_partitions_t<KVD_TURBO4, 128>(p, wide, grid, s);
        case KVD_TURBO8: return launch_partitions_t<KVD_TURBO8, 128>(p, wide, grid, s);
        default: return launch_partitions_t<KVD_TURBO3, 128>(p, wide, grid, s);
    }
}

hipError_t launch_reduce(int fmt, const LaunchParams& p, hipStream_t s) {
    switch (fmt) {
        case KVD_BF16: return p.D == 64 ? launch_reduce_t<KVD_BF16, 64>(p, s)
                                        : launch_reduce_t<KVD_BF16, 128>(p, s);
        case KVD_FP8_E4M3: return p.D == 64 ? launch_reduce_t<KVD_FP8_E4M3, 64>(p, s)
                                            : launch_reduce_t<KVD_FP8_E4M3, 128>(p, s);
        case KVD_TURBO4: return launch_reduce_t<KVD_TURBO4, 128>(p, s);
        case KVD_TURBO8: return launch_reduce_t<KVD_TURBO8, 128>(p, s);
        default: return launch_reduce_t<KVD_TURBO3, 128>(p, s);
    }
}

hipError_t launch_operands(int fmt, const OperandParams& p, hipStream_t s) {
    switch (fmt) {
        case KVD_BF16: return p.lp.D == 64 ? launch_operands_t<KVD_BF16, 64>(p, s)
                                           : launch_operands_t<KVD_BF16, 128>(p, s);
        case KVD_FP8_E4M3: return p.lp.D == 64 ? launch_operands_t<KVD_FP8_E4M3, 64>(p, s)
                                               : launch_operands_t<KVD_FP8_E4M3, 128>(p, s);
        case KVD_TURBO4: return launch_operands_t<KVD_TURBO4, 128>(p, s);
        case KVD_TURBO8: return launch_operands_t<KVD_TURBO8, 128>(p, s);
        default: return launch_operands_t<KVD_TURBO3, 128>(p, s);
    }
}

hipError_t launch_gather(const GatherParams& p, hipStream_t s) {
    const int total = p.n * p.D;
    return launch_kernel(gather_kernel, dim3((total + 255) / 256), dim3(256), s, p);
}

}  // namespace kvd
