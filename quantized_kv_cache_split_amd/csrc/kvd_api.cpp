// C-ABI host layer: argument checks, workspace sizing and kernel launches (include/kvdecode.h).
//
// Mirrors the host side of turboquant-rs 0.4.1 src/cache/cuda/attention.rs: refuse bad
// arguments before anything runs, size the partitions as ceil(len / partition size), launch
// the partition kernel and then the reduce, and report a launch failure.  Unlike that wrapper
// it allocates nothing: the partial buffers live in a caller-provided workspace.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvd_internal.h"
#include "kvdecode.h"

namespace {

using kvd::LaunchParams;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Bytes of one (page, KV head) chunk; codebook-stored K or V end with the page's 16 fp32
// per-token norms (64 bytes).
int64_t k_chunk_bytes(int fmt, int d) {
    switch (fmt) {
        case KVD_BF16: return 32LL * d;
        case KVD_FP8_E4M3:
        case KVD_TURBO8: return 16LL * d;   // Turbo8 K is stored as FP8 K
        case KVD_TURBO4: return 8LL * d + 64;
        default: return 6LL * d + 64;
    }
}
int64_t v_chunk_bytes(int fmt, int d) {
    return fmt == KVD_BF16 ? 32LL * d : (fmt == KVD_FP8_E4M3 ? 16LL * d : 8LL * d + 64);
}

// Formats that read a scale array: FP8 ([2][Hkv]) and Turbo8 ([Hkv] K scales).
bool needs_scales(int fmt) { return fmt == KVD_FP8_E4M3 || fmt == KVD_TURBO8; }

struct Plan {
    int mode;        // kvd::PartMode
    int part_size;   // tokens
    int P;           // partitions per sequence kept in the workspace (0 = no split possible)
    size_t off_l, off_o, bytes;
};

// Queries per sequence (a chunk at the last positions; 0 means 1).
int queries(const kvd_dims* d) { return d->queries_per_seq > 1 ? d->queries_per_seq : 1; }

// Query rows per KV head (queries x group) and the MFMA tiles of up to kMaxGroup rows they fill.
int64_t query_rows(const kvd_dims* d) {
    return (int64_t)queries(d) * (d->num_q_heads / d->num_kv_heads);
}
int query_tiles(const kvd_dims* d) {
    return (int)((query_rows(d) + kvd::kMaxGroup - 1) / kvd::kMaxGroup);
}
// Query tiles one wave computes (two where a KV head has several tiles and the format has the
// two-tile build), and the work units per KV head.
int tiles_per_unit(const kvd_dims* d, int fmt) {
    return query_tiles(d) >= 2 && kvd::tile_pairs_built(fmt, queries(d) > 1, false) ? 2 : 1;
}
int units_per_head(const kvd_dims* d, int fmt) {
    const int nt = tiles_per_unit(d, fmt);
    return (query_tiles(d) + nt - 1) / nt;
}

// Compute units of the current device (256 on MI355X when the query fails).
int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        return 256;
    return cus;
}

// Tokens each wave of the partition kernel walks (its run), and the kernel's layout.  A wave
// pays a fixed start-up (query staging, the block-table -> page-load latency chain, filling its
// load pipeline) and leaves a tail when it ends, so runs should be long; the chip should also
// be covered in one round.  For a batch whose sequences were all max_context_len long the
// automatic choice gives each sequence (and work unit) as many whole run blocks as one round
// of workgroups holds, and spreads the sequence's page pairs over those blocks' waves (runs of
// whole page pairs; a workgroup's runs cover at least one partition, its workspace slot).
// Splitting the batch's pairs evenly over the wave slots instead left a few workgroups for a
// second round whenever the units do not divide the slots: 6 x 32K calls FP8 98.4 -> 80.6
// us, Turbo4 84.5 -> 59.1, BF16 194.5 -> 144.9 us with the whole-block rule; power-of-two
// batches get the same runs either way.  With
// a mean_context_len hint below max_context_len (a ragged batch) it splits the batch's mean
// work over 2.5 rounds of the slots instead: sequences end at different times, and about 2.5
// waves of work per slot let the dispatcher even them out (ragged 64 x U{1..32K} BF16 batch,
// runs of 1 / 2 / 3 / 4 partitions, i.e. 5.2 / 2.6 / 1.8 / 1.5 rounds: 500.9 / 490.8 / 499.8 /
// 508.0 us per partition launch on MI355X).  Where
// the wide layout is built (one workgroup per CU) it is taken if runs of at most kMaxRunWide
// partitions cover the chip in one round; otherwise runs are capped at kMaxRunUniform
// partitions, or kMaxRun for ragged batches, whose real work is smaller and which do better
// with short runs (uniform FP8 16 x 32K with 8 queries per sequence, runs of 4 / 8 / 16
// partitions: 256.2 / 242.6 / 250.4 us per call).  Runs other than
// one partition need partition boundaries on even pages (partition size a multiple of 32).  A
// wave that computes two query tiles counts as two slots' work, so its runs are twice as long
// (FP8 / BF16 16 x 32K with 64 query heads on one KV head, runs of 1 / 2 partitions: 52.4 /
// 49.6 and 74.1 / 65.9 us per call).  An explicit partitions_per_wave R gives runs of R
// partitions in the two-workgroup layout.
//
// XCD skew.  In the BF16 / FP8 walks over random pages the odd XCDs of MI355X read more slowly
// than the even ones (wave timelines of FP8 16 x 32K: even XCDs end their walks after 166-170
// us, odd ones after 179-180 us, whichever KV heads they read; BF16 16 x 32K: 312-324 against
// 346-353 us).  When the automatic choice covers the chip in one round with a single query
// tile per KV head, runs of even run blocks (which the grid order puts on the even XCDs) are
// made run_skew_permille / 1000 longer and those of odd blocks as much shorter, in whole page
// pairs and never below one partition.  Measured optimum: 31-45 per mille in the two-workgroup
// layout (FP8 16 x 32K call 193.6 -> 190.3 us at 31, 193.5 at 100), 70 in the wide one (BF16
// 16 x 32K 368 -> 357.4 us; 360.9 at 31, 360.0 at 100).
//
// Early skew.  When such a grid holds exactly two workgroups per CU (two-workgroup layout),
// the workgroups each CU receives second (the grid's second half) end about 4 us after those
// it receives first.  Then both runs of the block pairs the grid dispatches first are made
// early_skew_permille / 1000 longer and those of the other pairs as much shorter (an even
// number of pairs, so a full sequence still ends with its last pair).  Measured on FP8 16 x 32K
// (single query, and 2 queries per sequence): 31 per mille (64 tokens on 2048-token runs),
// calls 190.1 -> 189.1 us and 192.6 -> 191.4 us; 16: 189.6 and 192.1; 47: 191.6 and 194.2;
// 62: 193.4 and 196.2.
constexpr int64_t run_skew_permille(bool wide) { return wide ? 70 : 31; }
// Small uniform batches: runs shorter than a partition (a workgroup's runs still cover one)
// fill the device where one-partition runs left most of it idle, and below this many pairs
// per run one workgroup per CU beats two (calls at 32K, runs as chosen / one partition:
// FP8 1 x 32K 24.2 / 30.8 us, 2 x 32K 34.6 us against 36.0 with two workgroups per CU and
// half the run, Turbo4 1 x 32K 25.5 / 40.7 us, BF16 1 x 32K 35.3 / 37.6 us).
constexpr int64_t kMinPairsTwoPerCu = 16;
constexpr int64_t early_skew_permille = 31;
struct RunChoice {
    int64_t run_tokens;   // narrowed to int32 once the caller has checked the token range
    bool wide;
    int64_t skew;         // LaunchParams::run_skew
    int64_t early;        // LaunchParams::early_skew
};
// Run blocks of a split sequence whose attended range starts in its first partition and spans
// `span` tokens (the kernels' run_blocks).
int64_t run_blocks(int64_t span, int64_t run_tokens, int64_t skew, int waves) {
    if (skew == 0) {
        const int64_t runs = (span + run_tokens - 1) / run_tokens;
        return (runs + waves - 1) / waves;
    }
    const int64_t two = 2 * waves * run_tokens;
    const int64_t q = span / two, rem = span - q * two;
    return 2 * q + (rem == 0 ? 0 : rem <= waves * (run_tokens + skew) ? 1 : 2);
}
RunChoice choose_run(const kvd_dims* d, const Plan& pl, int fmt) {
    const int ps = pl.part_size;
    if (!pl.P || ps % (2 * kvd::kPageTokens) != 0) return {ps, false, 0, 0};
    const int64_t pair_tokens = 2 * kvd::kPageTokens;
    int64_t tokens;
    bool wide = false;
    if (d->partitions_per_wave > 0) {
        tokens = (int64_t)d->partitions_per_wave * ps;
    } else {
        const bool ragged = d->mean_context_len > 0 && d->mean_context_len < d->max_context_len;
        const int64_t len = ragged ? d->mean_context_len : d->max_context_len;
        const int64_t pairs = (len + pair_tokens - 1) / pair_tokens;
        const int64_t units = (int64_t)d->num_kv_heads * units_per_head(d, fmt) * d->num_seqs;
        auto run_for = [&](bool w) -> int64_t {
            int64_t slots = (int64_t)device_cus() * kvd::waves_per_cu(w) / tiles_per_unit(d, fmt);
            int64_t rp;   // pairs per wave
            if (ragged) {
                slots = slots * 5 / 2;                                // 2.5 rounds of work
                rp = (pairs * units + slots - 1) / slots;
            } else {
                // as many whole run blocks per sequence as one round of workgroups holds, the
                // sequence spread over their waves
                const int64_t kw = kvd::waves_per_group(fmt);
                auto whole_blocks = [&](int64_t sl) {
                    int64_t per_seq = sl / kw / units;
                    if (per_seq < 1) per_seq = 1;
                    return (pairs + per_seq * kw - 1) / (per_seq * kw);
                };
                rp = whole_blocks(slots);
                // two workgroups per CU pay off only with runs of at least kMinPairsTwoPerCu
                // pairs; below that one per CU, with runs twice as long
                if (rp < kMinPairsTwoPerCu && slots / kw == 2LL * device_cus())
                    rp = whole_blocks(slots / 2);
                // a block's kw runs cover at least one partition (its workspace slot)
                const int64_t lo = (ps + kw * pair_tokens - 1) / (kw * pair_tokens);
                return (rp < lo ? lo : rp) * pair_tokens;
            }
            return rp * pair_tokens < ps ? ps : rp * pair_tokens;
        };
        if (!ragged && tiles_per_unit(d, fmt) == 1 &&
            kvd::wide_layout_built(fmt, d->head_dim, queries(d) > 1)) {
            const int64_t t = run_for(true);
            if (t <= (int64_t)kvd::kMaxRunWide * ps) {
                wide = true;
                tokens = t;
            }
        }
        if (!wide) {
            tokens = run_for(false);
            const int64_t cap = (int64_t)(ragged ? kvd::kMaxRun : kvd::kMaxRunUniform) * ps;
            if (tokens > cap) tokens = cap;
        }
    }
    const int64_t span = (int64_t)pl.P * ps;
    if (tokens > span) tokens = span;
    // Runs that one workgroup covers with room to spare would leave some of its waves without
    // pairs (Turbo 64 x 4K: 8 waves x 1024 tokens for a 4096-token context): the span is
    // spread over the workgroup's waves instead, in whole page pairs (at least a partition per
    // workgroup; per run for ragged batches).
    const int64_t kw = kvd::waves_per_group(fmt);
    if (d->partitions_per_wave == 0 && tokens * kw > span) {
        const bool rag = d->mean_context_len > 0 && d->mean_context_len < d->max_context_len;
        const int64_t floor_tok =
            rag ? ps : (ps + kw * pair_tokens - 1) / (kw * pair_tokens) * pair_tokens;
        int64_t even = (span + kw * pair_tokens - 1) / (kw * pair_tokens) * pair_tokens;
        if (even < floor_tok) even = floor_tok;
        if (even < tokens) tokens = even;
    }
    int64_t skew = 0;
    const bool ragged = d->mean_context_len > 0 && d->mean_context_len < d->max_context_len;
    if (d->partitions_per_wave == 0 && !ragged && (fmt == KVD_BF16 || fmt == KVD_FP8_E4M3) &&
        units_per_head(d, fmt) == 1 &&
        span >= 2 * kvd::waves_per_group(fmt) * tokens) {
        const int64_t pairs = tokens / pair_tokens;
        const int64_t sp = (pairs * run_skew_permille(wide) + 500) / 1000;
        if (sp > 0 && (pairs - sp) * pair_tokens >= ps) skew = sp * pair_tokens;
        if (skew) {   // no skew whose extra block would need a second round of workgroups
            int64_t bs = run_blocks(span, tokens, skew, kvd::waves_per_group(fmt));
            bs += bs & 1;
            const int64_t units = (int64_t)d->num_kv_heads * units_per_head(d, fmt) * d->num_seqs;
            const int64_t wgs = (int64_t)device_cus() * kvd::waves_per_cu(wide) /
                                tiles_per_unit(d, fmt) / kvd::waves_per_group(fmt);
            if (bs * units > wgs) skew = 0;
        }
    }
    int64_t early = 0;
    if (skew && !wide) {
        int64_t blocks = run_blocks(span, tokens, skew, kvd::waves_per_group(fmt));
        blocks += blocks & 1;
        const int64_t wgs = blocks * d->num_kv_heads * units_per_head(d, fmt) * d->num_seqs;
        const int64_t pairs = tokens / pair_tokens;
        const int64_t ep = (pairs * early_skew_permille + 500) / 1000;
        if (blocks % 4 == 0 && wgs == 2LL * device_cus() && ep > 0 &&
            tokens - skew - ep * pair_tokens >= ps)
            early = ep * pair_tokens;
    }
    return {tokens, wide, skew, early};
}

// Partition mode, partition size and partitions per sequence kept in the workspace (0 = no
// split possible) for d's partition_size.
struct Parts {
    int mode, part_size, P;
};
Parts partitions(const kvd_dims* d) {
    if (d->partition_size == -1) return {kvd::kPartNever, d->max_context_len, 0};
    if (d->partition_size == 0) {
        const int ps = kvd::kAutoPartition;
        return {kvd::kPartAuto, ps,
                d->max_context_len >= kvd::kAutoSplitMin
                    ? (int)(((int64_t)d->max_context_len + ps - 1) / ps) : 0};
    }
    return {kvd::kPartFixed, d->partition_size,
            (int)(((int64_t)d->max_context_len + d->partition_size - 1) / d->partition_size)};
}

// Shape checks that hold for every format.
int check_shape(const kvd_dims* d) {
    if (!d) return KVD_ERR_NULL;
    if (d->num_seqs < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1) return KVD_ERR_SHAPE;
    if (d->num_q_heads % d->num_kv_heads != 0) return KVD_ERR_SHAPE;
    if (d->head_dim != 64 && d->head_dim != 128) return KVD_ERR_SHAPE;
    if (d->block_size != kvd::kPageTokens) return KVD_ERR_SHAPE;
    if (d->max_blocks_per_seq < 1 || d->num_pool_blocks < 1) return KVD_ERR_SHAPE;
    if (d->max_context_len < 1 ||
        (int64_t)d->max_context_len > (int64_t)kvd::kPageTokens * d->max_blocks_per_seq)
        return KVD_ERR_SHAPE;
    const int ps = d->partition_size;
    if (!(ps == 0 || ps == -1 || (ps > 0 && ps % kvd::kPageTokens == 0))) return KVD_ERR_SHAPE;
    if (d->num_seqs > 65535 || d->num_kv_heads > 65535) return KVD_ERR_SHAPE;   // grid limits
    if (d->partitions_per_wave < 0 || d->mean_context_len < 0) return KVD_ERR_SHAPE;
    if (d->queries_per_seq < 0 || d->queries_per_seq > 65535) return KVD_ERR_SHAPE;
    if ((int64_t)d->num_seqs * queries(d) > 65535) return KVD_ERR_SHAPE;   // reduce grid rows
    if ((int64_t)queries(d) > d->max_context_len) return KVD_ERR_SHAPE;   // positions >= 0
    // query / output rows [B][n_q][Hq] are counted in int32
    if ((int64_t)d->num_seqs * queries(d) * d->num_q_heads > 0x7FFFFFFFLL) return KVD_ERR_SHAPE;
    // the workspace (fp32 m, l and D outputs per row and partition) must stay addressable
    const unsigned __int128 slots = (unsigned __int128)((int64_t)d->num_seqs * queries(d)) *
                                    (uint64_t)d->num_q_heads * (uint64_t)partitions(d).P;
    if (slots * (uint64_t)(d->head_dim + 2) * sizeof(float) > ((unsigned __int128)1 << 62))
        return KVD_ERR_SHAPE;
    return KVD_OK;
}

// Checks shared by every entry point that takes a format: the format itself, then the shape.
int check_dims(const kvd_dims* d, int fmt) {
    if (!d) return KVD_ERR_NULL;
    if (fmt < KVD_BF16 || fmt > KVD_TURBO8) return KVD_ERR_FORMAT;
    const int st = check_shape(d);
    if (st != KVD_OK) return st;
    if (fmt >= KVD_TURBO4 && d->head_dim != 128) return KVD_ERR_SHAPE;
    return KVD_OK;
}

// Workspace plan of dims that passed check_shape.
Plan make_plan(const kvd_dims* d) {
    Plan pl{};
    const Parts pa = partitions(d);
    pl.mode = pa.mode;
    pl.part_size = pa.part_size;
    pl.P = pa.P;
    const size_t rows = (size_t)d->num_seqs * queries(d) * d->num_q_heads * pl.P;
    const size_t ml = round_up(rows * sizeof(float), 256);
    pl.off_l = ml;
    pl.off_o = 2 * ml;
    pl.bytes = pl.P ? 2 * ml + round_up(rows * d->head_dim * sizeof(float), 256) : 0;
    return pl;
}

enum Phases { kPhase1 = 1, kPhase2 = 2 };

int run(int phases, const kvd_dims* d, const void* q, const void* k_cache, const void* v_cache,
        const int32_t* block_table, const int32_t* context_lens, int fmt, const float* scales,
        const float* codebook, const float* sign_pattern, float softmax_scale,
        const int32_t* window, float softcap, const float* alibi, float* out, void* workspace,
        size_t workspace_bytes, void* stream) {
    int st = check_dims(d, fmt);
    if (st != KVD_OK) return st;
    if (!q || !k_cache || !v_cache || !block_table || !context_lens || !out) return KVD_ERR_NULL;
    if (needs_scales(fmt) && !scales) return KVD_ERR_NULL;
    if (fmt >= KVD_TURBO4 && (!codebook || !sign_pattern)) return KVD_ERR_NULL;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
        !aligned(block_table, 4) || !aligned(context_lens, 4) || (window && !aligned(window, 4)) ||
        (scales && !aligned(scales, 16)) || (codebook && !aligned(codebook, 4)) ||
        (sign_pattern && !aligned(sign_pattern, 4)) || (alibi && !aligned(alibi, 4)))
        return KVD_ERR_ALIGN;
    if (!(softcap >= 0.0f) || !(softmax_scale == softmax_scale)) return KVD_ERR_SHAPE;
    const Plan pl = make_plan(d);
    if (pl.bytes) {
        if (!workspace) return KVD_ERR_WORKSPACE;
        if (workspace_bytes < pl.bytes) return KVD_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return KVD_ERR_ALIGN;
    }
    if (d->num_seqs == 0) return KVD_OK;

    LaunchParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint8_t*>(k_cache);
    p.v = static_cast<const uint8_t*>(v_cache);
    p.bt = block_table;
    p.ctx = context_lens;
    p.win = window;
    p.scales = scales;
    p.codebook = codebook;
    p.sign = sign_pattern;
    p.alibi = alibi;
    p.out = out;
    char* ws = static_cast<char*>(workspace);
    p.ws_m = pl.bytes ? reinterpret_cast<float*>(ws) : nullptr;
    p.ws_l = pl.bytes ? reinterpret_cast<float*>(ws + pl.off_l) : nullptr;
    p.ws_o = pl.bytes ? reinterpret_cast<float*>(ws + pl.off_o) : nullptr;
    p.k_chunk = k_chunk_bytes(fmt, d->head_dim);
    p.v_chunk = v_chunk_bytes(fmt, d->head_dim);
    p.B = d->num_seqs;
    p.Hq = d->num_q_heads;
    p.Hkv = d->num_kv_heads;
    p.g = d->num_q_heads / d->num_kv_heads;
    p.nq = queries(d);
    p.qt = query_tiles(d);
    p.nt = tiles_per_unit(d, fmt);
    p.qg = units_per_head(d, fmt);
    p.D = d->head_dim;
    p.max_blocks = d->max_blocks_per_seq;
    p.pool = d->num_pool_blocks;
    p.max_ctx = d->max_context_len;
    p.part_size = pl.part_size;
    p.P = pl.P;
    p.kbits = fmt == KVD_TURBO3 ? 3 : 4;
    const RunChoice rc = choose_run(d, pl, fmt);
    const int waves = kvd::waves_per_group(fmt);
    // run blocks of a sequence, at most (skewed runs: an even number of them)
    int64_t blocks = pl.P ? run_blocks((int64_t)pl.P * pl.part_size, rc.run_tokens, rc.skew, waves)
                          : 0;
    if (rc.skew) blocks += blocks & 1;
    // token indices of every run a workgroup can name must fit in int32
    if (pl.P && (int64_t)pl.P * pl.part_size + (rc.skew ? 2 : 1) * waves * (rc.run_tokens + rc.skew) >
                    0x7FFFFFFFLL)
        return KVD_ERR_SHAPE;
    // When every split sequence is one workgroup's walk (a single run block), nothing is merged
    // across workgroups: a call of both phases takes the kernel's unsplit path, whose waves
    // merge in LDS and write the final rows, with no workspace traffic and no reduce launch
    // (BF16 32 x 4K: call 100.0 -> 95.3 us).
    const bool one_block = pl.P && blocks == 1 && phases == (kPhase1 | kPhase2);
    p.part_mode = pl.P && !one_block ? pl.mode : kvd::kPartNever;
    p.run_tokens = (int32_t)rc.run_tokens;
    p.run_skew = (int32_t)rc.skew;
    p.early_skew = (int32_t)rc.early;
    p.run_pairs = (int32_t)(blocks / 2);
    p.softmax_scale = softmax_scale;
    p.softcap = softcap;

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (phases & kPhase1) {
        // `waves` waves per workgroup, one run per wave
        const int64_t px = pl.P ? blocks : 1;
        const int64_t wgs = (int64_t)px * d->num_kv_heads * p.qg * d->num_seqs;
        if (wgs > 0x7FFFFFFF) return KVD_ERR_SHAPE;
        const dim3 grid((unsigned)wgs);
        e = kvd::launch_partitions(fmt, rc.wide, p, grid, s);
        if (e != hipSuccess) return KVD_ERR_HIP;
    }
    if ((phases & kPhase2) && pl.P && !one_block) {
        e = kvd::launch_reduce(fmt, p, s);
        if (e != hipSuccess) return KVD_ERR_HIP;
    }
    return KVD_OK;
}

}  // namespace

extern "C" {

size_t kvd_workspace_bytes(const kvd_dims* dims) {
    if (check_shape(dims) != KVD_OK) return 0;
    return make_plan(dims).bytes;
}

int kvd_decode_attn_paged(const kvd_dims* d, const void* q, const void* k, const void* v,
                          const int32_t* bt, const int32_t* ctx, int fmt, const float* scales,
                          const float* codebook, const float* sign, float softmax_scale,
                          const int32_t* window, float softcap, const float* alibi, float* out,
                          void* ws, size_t ws_bytes, void* stream) {
    return run(kPhase1 | kPhase2, d, q, k, v, bt, ctx, fmt, scales, codebook, sign,
               softmax_scale, window, softcap, alibi, out, ws, ws_bytes, stream);
}

int kvd_decode_attn_paged_noalloc(const kvd_dims* d, const void* q, const void* k, const void* v,
                                  const int32_t* bt, const int32_t* ctx, int fmt,
                                  const float* scales, const float* codebook, const float* sign,
                                  float softmax_scale, const int32_t* window, float softcap,
                                  const float* alibi, float* out, void* stream) {
    int st = check_dims(d, fmt);
    if (st != KVD_OK) return st;
    if (make_plan(d).bytes > kvd::kNoAllocWorkspaceBytes) return KVD_ERR_WORKSPACE;
    void* ws = nullptr;
    if (kvd::noalloc_workspace(&ws) != hipSuccess) return KVD_ERR_HIP;
    return run(kPhase1 | kPhase2, d, q, k, v, bt, ctx, fmt, scales, codebook, sign,
               softmax_scale, window, softcap, alibi, out, ws, kvd::kNoAllocWorkspaceBytes,
               stream);
}

int kvd_decode_partitions(const kvd_dims* d, const void* q, const void* k, const void* v,
                          const int32_t* bt, const int32_t* ctx, int fmt, const float* scales,
                          const float* codebook, const float* sign, float softmax_scale,
                          const int32_t* window, float softcap, const float* alibi, float* out,
                          void* ws, size_t ws_bytes, void* stream) {
    return run(kPhase1, d, q, k, v, bt, ctx, fmt, scales, codebook, sign, softmax_scale,
               window, softcap, alibi, out, ws, ws_bytes, stream);
}

int kvd_reduce_partitions(const kvd_dims* d, const void* q, const void* k, const void* v,
                          const int32_t* bt, const int32_t* ctx, int fmt, const float* scales,
                          const float* codebook, const float* sign, float softmax_scale,
                          const int32_t* window, float softcap, const float* alibi, float* out,
                          void* ws, size_t ws_bytes, void* stream) {
    return run(kPhase2, d, q, k, v, bt, ctx, fmt, scales, codebook, sign, softmax_scale,
               window, softcap, alibi, out, ws, ws_bytes, stream);
}

int kvd_dequant_gather(const kvd_dims* d, int fmt, int is_v, const void* cache,
                       const float* scales, const float* codebook, const int32_t* block_table,
                       int32_t seq, int32_t kv_head, int32_t token_begin, int32_t n_tokens,
                       float* out, void* stream) {
    int st = check_dims(d, fmt);
    if (st != KVD_OK) return st;
    if (!cache || !block_table || !out) return KVD_ERR_NULL;
    if (needs_scales(fmt) && !scales) return KVD_ERR_NULL;
    if (fmt >= KVD_TURBO4 && !codebook) return KVD_ERR_NULL;
    if (!aligned(cache, 16) || !aligned(out, 4) || !aligned(block_table, 4) ||
        (scales && !aligned(scales, 4)))
        return KVD_ERR_ALIGN;
    if (seq < 0 || seq >= d->num_seqs || kv_head < 0 || kv_head >= d->num_kv_heads ||
        token_begin < 0 || n_tokens < 0 ||
        (int64_t)token_begin + n_tokens > (int64_t)kvd::kPageTokens * d->max_blocks_per_seq)
        return KVD_ERR_SHAPE;
    if ((int64_t)n_tokens * d->head_dim > 0x7FFFFFFF) return KVD_ERR_SHAPE;
    if (n_tokens == 0) return KVD_OK;
    kvd::GatherParams p{};
    p.cache = static_cast<const uint8_t*>(cache);
    p.scales = scales;
    p.codebook = codebook;
    p.bt = block_table;
    p.out = out;
    p.fmt = fmt;
    p.is_v = is_v ? 1 : 0;
    p.chunk = is_v ? v_chunk_bytes(fmt, d->head_dim) : k_chunk_bytes(fmt, d->head_dim);
    p.Hkv = d->num_kv_heads;
    p.D = d->head_dim;
    p.max_blocks = d->max_blocks_per_seq;
    p.pool = d->num_pool_blocks;
    p.seq = seq;
    p.kv_head = kv_head;
    p.t0 = token_begin;
    p.n = n_tokens;
    p.kbits = fmt == KVD_TURBO3 ? 3 : 4;
    return kvd::launch_gather(p, static_cast<hipStream_t>(stream)) == hipSuccess ? KVD_OK
                                                                                 : KVD_ERR_HIP;
}

int kvd_dequant_operands(const kvd_dims* d, int fmt, const void* k_cache, const void* v_cache,
                         const float* scales, const float* codebook, const int32_t* block_table,
                         int32_t seq, int32_t kv_head, int32_t pair_begin, int32_t n_pairs,
                         uint32_t* out, void* stream) {
    int st = check_dims(d, fmt);
    if (st != KVD_OK) return st;
    if (!k_cache || !v_cache || !block_table || !out) return KVD_ERR_NULL;
    if (needs_scales(fmt) && !scales) return KVD_ERR_NULL;
    if (fmt >= KVD_TURBO4 && !codebook) return KVD_ERR_NULL;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
        !aligned(block_table, 4) || (scales && !aligned(scales, 16)) ||
        (codebook && !aligned(codebook, 4)))
        return KVD_ERR_ALIGN;
    if (seq < 0 || seq >= d->num_seqs || kv_head < 0 || kv_head >= d->num_kv_heads ||
        pair_begin < 0 || n_pairs < 0 ||
        2 * ((int64_t)pair_begin + n_pairs) > (int64_t)d->max_blocks_per_seq)
        return KVD_ERR_SHAPE;
    if (n_pairs == 0) return KVD_OK;
    kvd::OperandParams op{};
    LaunchParams& p = op.lp;
    p.k = static_cast<const uint8_t*>(k_cache);
    p.v = static_cast<const uint8_t*>(v_cache);
    p.bt = block_table;
    p.scales = scales;
    p.codebook = codebook;
    p.k_chunk = k_chunk_bytes(fmt, d->head_dim);
    p.v_chunk = v_chunk_bytes(fmt, d->head_dim);
    p.B = d->num_seqs;
    p.Hq = d->num_q_heads;
    p.Hkv = d->num_kv_heads;
    p.g = d->num_q_heads / d->num_kv_heads;
    p.D = d->head_dim;
    p.max_blocks = d->max_blocks_per_seq;
    p.pool = d->num_pool_blocks;
    p.max_ctx = d->max_context_len;
    p.kbits = fmt == KVD_TURBO3 ? 3 : 4;
    op.out = out;
    op.seq = seq;
    op.kv_head = kv_head;
    op.pair0 = pair_begin;
    op.npairs = n_pairs;
    return kvd::launch_operands(fmt, op, static_cast<hipStream_t>(stream)) == hipSuccess
               ? KVD_OK : KVD_ERR_HIP;
}

int kvd_append_kv(const kvd_dims* d, int fmt, const float* k_new, const float* v_new,
                  const int32_t* block_table, const int32_t* positions, int32_t n_new,
                  void* k_cache, void* v_cache, const float* scales, const float* codebook,
                  const float* sign_pattern, void* stream) {
    int st = check_dims(d, fmt);
    if (st != KVD_OK) return st;
    if (n_new < 0) return KVD_ERR_SHAPE;
    if (!k_new || !v_new || !block_table || !positions || !k_cache || !v_cache) return KVD_ERR_NULL;
    if (needs_scales(fmt) && !scales) return KVD_ERR_NULL;
    if (fmt >= KVD_TURBO4 && (!codebook || !sign_pattern)) return KVD_ERR_NULL;
    if (!aligned(k_new, 8) || !aligned(v_new, 8) || !aligned(block_table, 4) ||
        !aligned(positions, 4) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        (scales && !aligned(scales, 4)) || (codebook && !aligned(codebook, 4)) ||
        (sign_pattern && !aligned(sign_pattern, 4)))
        return KVD_ERR_ALIGN;
    // one workgroup per (sequence, page slot, KV head); T new tokens touch at most
    // ceil(T / 16) + 1 pages of a sequence
    const int64_t ps = ((int64_t)n_new + kvd::kPageTokens - 1) / kvd::kPageTokens + 1;
    if ((int64_t)d->num_seqs * ps * d->num_kv_heads > 0x7FFFFFFFLL) return KVD_ERR_SHAPE;
    if (d->num_seqs == 0 || n_new == 0) return KVD_OK;
    kvd::AppendParams p{};
    p.k_new = k_new;
    p.v_new = v_new;
    p.bt = block_table;
    p.pos = positions;
    p.k = static_cast<uint8_t*>(k_cache);
    p.v = static_cast<uint8_t*>(v_cache);
    p.scales = scales;
    p.codebook = codebook;
    p.sign = sign_pattern;
    p.k_chunk = k_chunk_bytes(fmt, d->head_dim);
    p.v_chunk = v_chunk_bytes(fmt, d->head_dim);
    p.fmt = fmt;
    p.B = d->num_seqs;
    p.T = n_new;
    p.Hkv = d->num_kv_heads;
    p.D = d->head_dim;
    p.max_blocks = d->max_blocks_per_seq;
    p.pool = d->num_pool_blocks;
    p.kbits = fmt == KVD_TURBO3 ? 3 : 4;
    p.ps = (int32_t)ps;
    return kvd::launch_append(p, static_cast<hipStream_t>(stream)) == hipSuccess ? KVD_OK
                                                                                : KVD_ERR_HIP;
}

int kvd_read_probe(const void* buf, size_t buf_bytes, const int32_t* chunk_ids, int64_t n_chunks,
                   int32_t chunk_bytes, int32_t waves_per_cu, int32_t loads_in_flight,
                   uint32_t* sink, size_t sink_bytes, void* stream) {
    if (!buf || !chunk_ids || !sink) return KVD_ERR_NULL;
    if (!aligned(buf, 16) || !aligned(chunk_ids, 4) || !aligned(sink, 4)) return KVD_ERR_ALIGN;
    if (chunk_bytes < 1024 || (chunk_bytes & (chunk_bytes - 1)) != 0 || n_chunks < 0 ||
        buf_bytes < (size_t)chunk_bytes || waves_per_cu < 4 || waves_per_cu > 32 ||
        waves_per_cu % 4 != 0 || !(loads_in_flight == 1 || loads_in_flight == 2 ||
                                   loads_in_flight == 4 || loads_in_flight == 8 ||
                                   loads_in_flight == 16))
        return KVD_ERR_SHAPE;
    const int blocks = device_cus() * waves_per_cu / 4;
    if (sink_bytes < (size_t)blocks * 4 * 64 * sizeof(uint32_t)) return KVD_ERR_WORKSPACE;
    if (n_chunks == 0) return KVD_OK;
    kvd::ProbeParams p{};
    p.buf = static_cast<const uint8_t*>(buf);
    p.ids = chunk_ids;
    p.sink = sink;
    p.n = n_chunks;
    p.buf_bytes = (int64_t)buf_bytes;
    p.log2_pieces = 0;
    while ((1024 << p.log2_pieces) < chunk_bytes) ++p.log2_pieces;
    return kvd::launch_read_probe(p, blocks, loads_in_flight, static_cast<hipStream_t>(stream)) ==
                   hipSuccess ? KVD_OK : KVD_ERR_HIP;
}

const char* kvd_status_str(int status) {
    switch (status) {
        case KVD_OK: return "ok";
        case KVD_ERR_NULL: return "a required pointer is NULL";
        case KVD_ERR_SHAPE: return "unsupported or inconsistent dimensions";
        case KVD_ERR_FORMAT: return "unknown kv format";
        case KVD_ERR_ALIGN: return "a pointer is not aligned as required";
        case KVD_ERR_WORKSPACE: return "workspace missing or too small";
        case KVD_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

}  // extern "C"
