// Drives every entry point of the C-ABI layer (include/kvdecode.h) on the host, with the device
// side replaced by recording stubs (launch_stub.cpp), for a build under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Fixed cases check each documented error path; a seeded sweep
// then feeds dims drawn from edge values (negative, zero, powers of two and their neighbours,
// INT32_MAX and its neighbours) to every entry point and checks, for each accepted call, that
// the launch the layer would make stays inside what the kernels assume: grid sizes, workspace
// slots inside the workspace, run lengths, chunk sizes, token ranges.  Any failed check prints
// the case and exits 1; the sanitizers abort on the first memory or UB error.
//
// usage: abi_sweep [iterations] [seed]
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvdecode.h"
#include "launch_stub.h"

namespace {

int failures = 0;
char where[512];
long accepted[7];   // sweep calls that reached a launch, by stub::Kind
long skewed;        // checked partition launches with skewed runs
long early;         // ... of which also with early-skewed block pairs
long single;        // checked decode launches whose sequences are one run block each

#define CHECK(cond)                                                                            \
    do {                                                                                       \
        if (!(cond)) {                                                                         \
            fprintf(stderr, "FAIL %s:%d: %s [%s]\n", __FILE__, __LINE__, #cond, where);        \
            if (++failures > 20) exit(1);                                                      \
        }                                                                                      \
    } while (0)

// Device pointers are never dereferenced by the host layer; these stand-ins are 1 MiB aligned
// (or 2 bytes off) and point at unmapped low memory, so a host dereference would fault.
void* fake(uintptr_t k) { return reinterpret_cast<void*>((k + 1) * 0x100000); }
void* misaligned(uintptr_t k) { return reinterpret_cast<void*>((k + 1) * 0x100000 + 2); }

uint64_t rng_state;
uint64_t next() {   // xorshift64*
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1DULL;
}
int pick(const int* v, int n) { return v[next() % (uint64_t)n]; }

const int kEdges[] = {INT32_MIN, INT32_MIN + 1, -65536, -17, -2, -1, 0, 1, 2, 3, 15, 16, 17,
                      31, 32, 33, 63, 64, 65, 127, 128, 129, 511, 512, 513, 1023, 1024, 1025,
                      4096, 32768, 65535, 65536, 65537, 1 << 20, (1 << 27) - 1, 1 << 27,
                      1 << 28, INT32_MAX - 511, INT32_MAX - 16, INT32_MAX - 1, INT32_MAX};
const int kNE = sizeof(kEdges) / sizeof(kEdges[0]);

// A field value: usually a plausible one, sometimes an edge value.
int field(const int* plausible, int n) {
    return next() % 4 == 0 ? pick(kEdges, kNE) : pick(plausible, n);
}

kvd_dims random_dims() {
    static const int seqs[] = {0, 1, 2, 3, 8, 16, 64, 255, 4096, 65535};
    static const int qh[] = {1, 4, 8, 16, 32, 64, 128, 256};
    static const int kvh[] = {1, 2, 4, 8, 16};
    static const int hd[] = {64, 128, 128};
    static const int bs[] = {16, 16, 16, 32};
    static const int mb[] = {1, 2, 7, 64, 65, 2048, 4096, 1 << 20};
    static const int pool[] = {1, 16, 4096, 1 << 20};
    static const int ctx[] = {1, 15, 16, 17, 1000, 1023, 1024, 1025, 32768, 65536};
    static const int ps[] = {0, 0, -1, 16, 32, 48, 256, 512, 4096};
    static const int ppw[] = {0, 0, 1, 2, 3, 8, 1000};
    static const int nq[] = {0, 1, 1, 2, 7, 16, 64};
    static const int mean[] = {0, 0, 1, 500, 16384, 32768, 65536};
    kvd_dims d;
    d.num_seqs = field(seqs, 10);
    d.num_q_heads = field(qh, 8);
    d.num_kv_heads = field(kvh, 5);
    d.head_dim = field(hd, 3);
    d.block_size = field(bs, 4);
    d.max_blocks_per_seq = field(mb, 8);
    d.num_pool_blocks = field(pool, 4);
    d.max_context_len = field(ctx, 10);
    if (next() % 2 && d.max_blocks_per_seq > 0 && d.max_blocks_per_seq < (1 << 27))
        d.max_context_len = 16 * d.max_blocks_per_seq - (int)(next() % 16);   // often valid
    d.partition_size = field(ps, 9);
    d.partitions_per_wave = field(ppw, 7);
    d.queries_per_seq = field(nq, 7);
    d.mean_context_len = field(mean, 7);
    return d;
}

void describe(const kvd_dims& d, int fmt, const char* entry) {
    snprintf(where, sizeof(where),
             "%s fmt=%d B=%d Hq=%d Hkv=%d D=%d bs=%d mb=%d pool=%d L=%d ps=%d ppw=%d nq=%d mean=%d",
             entry, fmt, d.num_seqs, d.num_q_heads, d.num_kv_heads, d.head_dim, d.block_size,
             d.max_blocks_per_seq, d.num_pool_blocks, d.max_context_len, d.partition_size,
             d.partitions_per_wave, d.queries_per_seq, d.mean_context_len);
}

int64_t k_chunk(int fmt, int D) {
    switch (fmt) {
        case KVD_BF16: return 32LL * D;
        case KVD_FP8_E4M3: case KVD_TURBO8: return 16LL * D;
        case KVD_TURBO4: return 8LL * D + 64;
        default: return 6LL * D + 64;
    }
}
int64_t v_chunk(int fmt, int D) {
    return fmt == KVD_BF16 ? 32LL * D : fmt == KVD_FP8_E4M3 ? 16LL * D : 8LL * D + 64;
}

// Arguments of one decode call; everything valid unless a case changes it.
struct Call {
    const kvd_dims* d;
    const void *q, *k, *v;
    const int32_t *bt, *ctx;
    int fmt;
    const float *scales, *codebook, *sign;
    float scale;
    const int32_t* window;
    float softcap;
    const float* alibi;
    float* out;
    void* ws;
    size_t ws_bytes;
};
Call base_call(const kvd_dims* d, int fmt) {
    Call c;
    c.d = d;
    c.q = fake(1);
    c.k = fake(2);
    c.v = fake(3);
    c.bt = static_cast<const int32_t*>(fake(4));
    c.ctx = static_cast<const int32_t*>(fake(5));
    c.fmt = fmt;
    c.scales = static_cast<const float*>(fake(6));
    c.codebook = static_cast<const float*>(fake(7));
    c.sign = static_cast<const float*>(fake(8));
    c.scale = 0.088f;
    c.window = nullptr;
    c.softcap = 0.0f;
    c.alibi = nullptr;
    c.out = static_cast<float*>(fake(9));
    c.ws = fake(10);
    c.ws_bytes = SIZE_MAX;
    return c;
}
typedef int (*DecodeFn)(const kvd_dims*, const void*, const void*, const void*, const int32_t*,
                        const int32_t*, int, const float*, const float*, const float*, float,
                        const int32_t*, float, const float*, float*, void*, size_t, void*);
int call(DecodeFn f, const Call& c) {
    return f(c.d, c.q, c.k, c.v, c.bt, c.ctx, c.fmt, c.scales, c.codebook, c.sign, c.scale,
             c.window, c.softcap, c.alibi, c.out, c.ws, c.ws_bytes, nullptr);
}

// What the partition and reduce launches of an accepted decode call must satisfy.
void check_decode_launch(const kvd_dims& d, int fmt, const char* base, size_t ws_bytes,
                         bool phase1, bool phase2) {
    const stub::Record& r = stub::rec;
    const kvd::LaunchParams& p = r.lp;
    const int64_t nq = d.queries_per_seq > 1 ? d.queries_per_seq : 1;
    const int64_t g = d.num_q_heads / d.num_kv_heads;
    const int64_t qt = (nq * g + 15) / 16;
    // BF16 / FP8 with several tiles per KV head: two tiles per work unit
    const int64_t nt = (qt >= 2 && (fmt == KVD_BF16 || fmt == KVD_FP8_E4M3)) ? 2 : 1;
    const int64_t units = (qt + nt - 1) / nt;
    if (d.num_seqs == 0) {
        CHECK(r.calls[stub::kPartitions] == 0 && r.calls[stub::kReduce] == 0);
        return;
    }
    CHECK(r.calls[stub::kPartitions] == (phase1 ? 1 : 0));
    CHECK(r.calls[stub::kReduce] <= (phase2 && p.P > 0 ? 1 : 0));
    if (!phase1) CHECK(r.calls[stub::kReduce] == (phase2 && p.P > 0 ? 1 : 0));
    if (!r.calls[stub::kPartitions] && !r.calls[stub::kReduce]) return;
    CHECK(r.fmt == fmt);
    CHECK(p.B == d.num_seqs && p.Hq == d.num_q_heads && p.Hkv == d.num_kv_heads);
    CHECK(p.g == g && p.nq == nq && p.qt == qt && p.nt == nt && p.qg == units && p.D == d.head_dim);
    CHECK(p.k_chunk == k_chunk(fmt, d.head_dim) && p.v_chunk == v_chunk(fmt, d.head_dim));
    CHECK(p.kbits == (fmt == KVD_TURBO3 ? 3 : 4));
    CHECK(p.max_ctx == d.max_context_len && p.max_blocks == d.max_blocks_per_seq);
    const int waves = fmt >= KVD_TURBO4 ? 8 : 4;
    if (p.P > 0) {
        CHECK(p.part_size > 0 && (int64_t)p.P * p.part_size >= d.max_context_len);
        CHECK((int64_t)(p.P - 1) * p.part_size < d.max_context_len);
        // a workgroup's runs cover at least one partition (its workspace slot); explicit
        // partitions_per_wave and ragged batches: whole partitions
        CHECK((int64_t)waves * p.run_tokens >= p.part_size && p.run_tokens > 0);
        if (d.partitions_per_wave > 0 ||
            (d.mean_context_len > 0 && d.mean_context_len < d.max_context_len))
            CHECK(p.run_tokens >= p.part_size);
        CHECK(p.run_tokens <= (int64_t)p.P * p.part_size);
        CHECK(p.run_tokens == p.part_size || p.run_tokens % 32 == 0);
        CHECK((int64_t)p.P * p.part_size + (int64_t)waves * p.run_tokens <= INT32_MAX);
        // every slot a run writes lies inside the workspace, each array in its own region
        const int64_t rows = (int64_t)d.num_seqs * nq * d.num_q_heads;
        const char* ws = base;
        const char* m = reinterpret_cast<const char*>(p.ws_m);
        const char* l = reinterpret_cast<const char*>(p.ws_l);
        const char* o = reinterpret_cast<const char*>(p.ws_o);
        const unsigned __int128 slots = (unsigned __int128)rows * (uint64_t)p.P;
        CHECK(m == ws && l > m && o > l);
        CHECK((unsigned __int128)(l - m) >= slots * 4);
        CHECK((unsigned __int128)(o - l) >= slots * 4);
        CHECK((unsigned __int128)(o - ws) + slots * (uint64_t)d.head_dim * 4 <= ws_bytes);
        CHECK((reinterpret_cast<uintptr_t>(o) & 255) == 0 && (reinterpret_cast<uintptr_t>(l) & 255) == 0);
    } else {
        CHECK(p.part_mode == kvd::kPartNever);
    }
    if (r.calls[stub::kPartitions]) {
        // run blocks per sequence: W runs of T tokens each, or with a skew s > 0 alternately
        // W runs of T + s and W of T - s, an even number of blocks; with an early skew e > 0
        // as well, the grid is two workgroups per CU and holds an even number of block pairs,
        // half of them e tokens longer per run and half e shorter
        int64_t px = 1;
        if (p.P > 0) {
            const int64_t span = (int64_t)p.P * p.part_size, T = p.run_tokens, sk = p.run_skew;
            if (sk == 0) {
                px = ((span + T - 1) / T + waves - 1) / waves;
            } else {
                CHECK(sk > 0 && sk % 32 == 0 && T - sk >= p.part_size && T % 32 == 0);
                CHECK(units == 1 && (fmt == KVD_BF16 || fmt == KVD_FP8_E4M3));
                CHECK(d.partitions_per_wave == 0 &&
                      !(d.mean_context_len > 0 && d.mean_context_len < d.max_context_len));
                const int64_t two = 2 * waves * T, q = span / two, rem = span - q * two;
                px = 2 * q + (rem == 0 ? 0 : rem <= waves * (T + sk) ? 1 : 2);
                px += px & 1;
                CHECK(px / 2 * two >= span);
                CHECK(p.run_pairs == px / 2);
                ++skewed;
                if (p.early_skew != 0) {
                    const int64_t e = p.early_skew;
                    const int cus = stub::device_cus > 0 ? stub::device_cus : 256;
                    CHECK(e > 0 && e % 32 == 0 && T - sk - e >= p.part_size && !r.wide);
                    CHECK(px % 4 == 0 &&
                          px * d.num_kv_heads * units * d.num_seqs == 2LL * cus);
                    ++early;
                }
            }
            if (sk == 0) CHECK(p.early_skew == 0);
            CHECK(span + (sk ? 2 : 1) * waves * (T + sk) <= 0x7FFFFFFFLL);
        } else {
            CHECK(p.run_skew == 0 && p.early_skew == 0);
        }
        CHECK((int64_t)r.grid.x == px * d.num_kv_heads * units * d.num_seqs);
        // both phases with one run block per sequence: the unsplit path, no reduce
        const bool one_block = phase2 && p.P > 0 && px == 1;
        CHECK(r.calls[stub::kReduce] == (phase2 && p.P > 0 && !one_block ? 1 : 0));
        if (p.P > 0) CHECK((p.part_mode == kvd::kPartNever) == one_block);
        if (one_block) ++single;
        CHECK(r.grid.x >= 1 && r.grid.x <= 0x7FFFFFFFu && r.grid.y == 1 && r.grid.z == 1);
        CHECK(!r.wide || (fmt == KVD_BF16 && d.head_dim == 128 && nq == 1 && nt == 1));
    }
}

// ---- fixed cases -------------------------------------------------------------------------

kvd_dims valid_dims() {
    kvd_dims d;
    memset(&d, 0, sizeof(d));
    d.num_seqs = 4;
    d.num_q_heads = 32;
    d.num_kv_heads = 8;
    d.head_dim = 128;
    d.block_size = 16;
    d.max_blocks_per_seq = 2048;
    d.num_pool_blocks = 8192;
    d.max_context_len = 32768;
    return d;
}

// The automatic run choice on uniform batches of 256-CU devices: the FP8 16 x 32K batch takes
// runs of 2048 tokens, the XCD skew (64 tokens) and the early skew (64), 512 workgroups (two
// per CU); batches of 6 sequences (48 units) fit one round of workgroups; batches of 1 or 2
// sequences take runs shorter than a partition and one workgroup per CU.
void run_choice_cases() {
    struct Case {
        int fmt, seqs, hq, ctx;
        int64_t run_tokens, skew, early, max_wgs;
    };
    const Case cases[] = {
        {KVD_FP8_E4M3, 16, 64, 32768, 2048, 64, 64, 512},
        {KVD_FP8_E4M3, 6, 64, 32768, 832, 32, 0, 512},
        {KVD_TURBO4, 6, 32, 32768, 832, 0, 0, 256},
        {KVD_TURBO4, 8, 32, 32768, 1024, 0, 0, 256},
        {KVD_BF16, 6, 64, 32768, 1664, 0, 0, 256},
        {KVD_TURBO4, 64, 32, 4096, 512, 0, 0, 512},
        {KVD_FP8_E4M3, 1, 64, 32768, 256, 0, 0, 256},
        {KVD_FP8_E4M3, 2, 64, 32768, 512, 0, 0, 256},
        {KVD_FP8_E4M3, 4, 64, 32768, 512, 0, 0, 512},
        {KVD_TURBO4, 1, 32, 32768, 128, 0, 0, 256},
        {KVD_BF16, 1, 64, 32768, 256, 0, 0, 256},
    };
    for (const Case& k : cases) {
        kvd_dims* d = static_cast<kvd_dims*>(malloc(sizeof(kvd_dims)));
        *d = valid_dims();
        d->num_seqs = k.seqs;
        d->num_q_heads = k.hq;
        d->max_context_len = k.ctx;
        d->num_pool_blocks = 1 << 20;
        describe(*d, k.fmt, "run choice");
        Call c = base_call(d, k.fmt);
        c.ws_bytes = kvd_workspace_bytes(d);
        stub::reset();
        CHECK(call(kvd_decode_partitions, c) == KVD_OK);
        const kvd::LaunchParams& p = stub::rec.lp;
        CHECK(p.run_tokens == k.run_tokens && p.run_skew == k.skew && p.early_skew == k.early);
        CHECK((int64_t)stub::rec.grid.x <= k.max_wgs);
        check_decode_launch(*d, k.fmt, static_cast<const char*>(c.ws), c.ws_bytes, true, false);
        free(d);
    }
}

void fixed_cases() {
    run_choice_cases();
    for (int s = -8; s <= 2; ++s) CHECK(kvd_status_str(s) != nullptr && kvd_status_str(s)[0]);
    snprintf(where, sizeof(where), "null dims");
    CHECK(kvd_workspace_bytes(nullptr) == 0);
    kvd_dims* heap = static_cast<kvd_dims*>(malloc(sizeof(kvd_dims)));   // exact size: ASan
    *heap = valid_dims();                                                 // sees any overread
    for (int fmt = KVD_BF16; fmt <= KVD_TURBO8; ++fmt) {
        describe(*heap, fmt, "fixed");
        Call c = base_call(heap, fmt);
        c.d = nullptr;
        CHECK(call(kvd_decode_attn_paged, c) == KVD_ERR_NULL);
        c.d = heap;
        const size_t need = kvd_workspace_bytes(heap);
        CHECK(need > 0);
        c.ws_bytes = need;
        stub::reset();
        CHECK(call(kvd_decode_attn_paged, c) == KVD_OK);
        check_decode_launch(*heap, fmt, static_cast<const char*>(c.ws), need, true, true);
        stub::reset();
        CHECK(call(kvd_decode_partitions, c) == KVD_OK);
        check_decode_launch(*heap, fmt, static_cast<const char*>(c.ws), need, true, false);
        stub::reset();
        CHECK(call(kvd_reduce_partitions, c) == KVD_OK);
        check_decode_launch(*heap, fmt, static_cast<const char*>(c.ws), need, false, true);
        c.ws_bytes = need - 1;
        CHECK(call(kvd_decode_attn_paged, c) == KVD_ERR_WORKSPACE);
        c.ws_bytes = need;
        c.ws = nullptr;
        CHECK(call(kvd_decode_attn_paged, c) == KVD_ERR_WORKSPACE);
        c.ws = misaligned(10);
        CHECK(call(kvd_decode_attn_paged, c) == KVD_ERR_ALIGN);
        c = base_call(heap, fmt);
        c.q = misaligned(1);
        CHECK(call(kvd_decode_attn_paged, c) == KVD_ERR_ALIGN);
        c = base_call(heap, fmt);
        c.scale = NAN;
        CHECK(call(kvd_decode_attn_paged, c) == KVD_ERR_SHAPE);
        c = base_call(heap, fmt);
        c.softcap = -1.0f;
        CHECK(call(kvd_decode_attn_paged, c) == KVD_ERR_SHAPE);
        c.softcap = NAN;
        CHECK(call(kvd_decode_attn_paged, c) == KVD_ERR_SHAPE);
        c = base_call(heap, fmt);
        c.scales = nullptr;
        CHECK(call(kvd_decode_attn_paged, c) ==
              (fmt == KVD_FP8_E4M3 || fmt == KVD_TURBO8 ? KVD_ERR_NULL : KVD_OK));
        c = base_call(heap, fmt);
        c.codebook = nullptr;
        CHECK(call(kvd_decode_attn_paged, c) == (fmt >= KVD_TURBO4 ? KVD_ERR_NULL : KVD_OK));
        // the allocation-free entry point: the library's workspace, refused past its size
        stub::reset();
        CHECK(kvd_decode_attn_paged_noalloc(heap, c.q, c.k, c.v, c.bt, c.ctx, fmt, c.scales,
                                            static_cast<const float*>(fake(7)), c.sign, c.scale,
                                            nullptr, 0.0f, nullptr, c.out, nullptr) == KVD_OK);
        check_decode_launch(*heap, fmt, static_cast<const char*>(stub::noalloc_address),
                            KVD_NOALLOC_WORKSPACE_BYTES, true, true);
        kvd_dims big = *heap;
        big.num_seqs = 512;
        big.num_q_heads = 64;
        describe(big, fmt, "noalloc too big");
        CHECK(kvd_workspace_bytes(&big) > KVD_NOALLOC_WORKSPACE_BYTES);
        CHECK(kvd_decode_attn_paged_noalloc(&big, c.q, c.k, c.v, c.bt, c.ctx, fmt, c.scales,
                                            static_cast<const float*>(fake(7)), c.sign, c.scale,
                                            nullptr, 0.0f, nullptr, c.out, nullptr) ==
              KVD_ERR_WORKSPACE);
    }
    for (int fmt : {-1, 5, 100, INT32_MIN}) {
        describe(*heap, fmt, "bad format");
        Call c = base_call(heap, fmt);
        CHECK(call(kvd_decode_attn_paged, c) == KVD_ERR_FORMAT);
    }
    // device query failure: the layer assumes 256 compute units
    stub::device_cus = 0;
    stub::reset();
    uint32_t* sink = static_cast<uint32_t*>(fake(11));
    snprintf(where, sizeof(where), "probe, failed device query");
    CHECK(kvd_read_probe(fake(12), 1 << 30, static_cast<const int32_t*>(fake(13)), 1000, 4096, 8,
                         8, sink, SIZE_MAX, nullptr) == KVD_OK);
    CHECK(stub::rec.blocks == 256 * 8 / 4 && stub::rec.loads_in_flight == 8);
    CHECK(stub::rec.pp.log2_pieces == 2);
    stub::device_cus = 256;
    CHECK(kvd_read_probe(fake(12), 1 << 30, static_cast<const int32_t*>(fake(13)), 1000, 4096, 8,
                         8, sink, 512 * 64 * 4 - 1, nullptr) == KVD_ERR_WORKSPACE);
    free(heap);
}

// ---- sweep -------------------------------------------------------------------------------

void sweep_one() {
    kvd_dims* d = static_cast<kvd_dims*>(malloc(sizeof(kvd_dims)));
    *d = random_dims();
    const int fmts[] = {-1, 0, 1, 2, 3, 4, 5};
    const int fmt = fmts[next() % 7];
    describe(*d, fmt, "workspace_bytes");
    const size_t need = kvd_workspace_bytes(d);
    describe(*d, fmt, "decode");
    Call c = base_call(d, fmt);
    if (next() % 3 == 0) c.window = static_cast<const int32_t*>(fake(14));
    if (next() % 3 == 0) c.alibi = static_cast<const float*>(fake(15));
    if (next() % 4 == 0) c.softcap = 30.0f;
    stub::reset();
    const int st = call(kvd_decode_attn_paged, c);
    CHECK(st == KVD_OK || st == KVD_ERR_SHAPE || st == KVD_ERR_FORMAT);
    if (st == KVD_OK) {
        accepted[stub::kPartitions] += stub::rec.calls[stub::kPartitions];
        accepted[stub::kReduce] += stub::rec.calls[stub::kReduce];
        check_decode_launch(*d, fmt, static_cast<const char*>(c.ws), need ? need : SIZE_MAX, true, true);
        c.ws_bytes = need;
        stub::reset();
        CHECK(call(kvd_decode_attn_paged, c) == KVD_OK);
        if (need > 0) {
            check_decode_launch(*d, fmt, static_cast<const char*>(c.ws), need, true, true);
            c.ws_bytes = need - 1;
            CHECK(call(kvd_decode_attn_paged, c) == KVD_ERR_WORKSPACE);
        }
        stub::reset();
        const int sn = kvd_decode_attn_paged_noalloc(d, c.q, c.k, c.v, c.bt, c.ctx, fmt, c.scales,
                                                     c.codebook, c.sign, c.scale, c.window,
                                                     c.softcap, c.alibi, c.out, nullptr);
        CHECK(sn == (need <= KVD_NOALLOC_WORKSPACE_BYTES ? KVD_OK : KVD_ERR_WORKSPACE));
        if (sn == KVD_OK)
            check_decode_launch(*d, fmt, static_cast<const char*>(stub::noalloc_address),
                                KVD_NOALLOC_WORKSPACE_BYTES, true, true);
    } else if (fmt >= 0 && fmt <= 4) {
        CHECK(st == KVD_ERR_SHAPE);
    }

    // dequant gather: a token range of one (sequence, KV head)
    {
        const int seq = pick(kEdges, kNE) % 5, head = (int)(next() % 9) - 1;
        const int t0 = next() % 2 ? (int)(next() % 64) : pick(kEdges, kNE);
        const int n = next() % 2 ? (int)(next() % 300) : pick(kEdges, kNE);
        const int is_v = (int)(next() % 2);
        describe(*d, fmt, "gather");
        stub::reset();
        const int sg = kvd_dequant_gather(d, fmt, is_v, fake(2), c.scales, c.codebook, c.bt, seq,
                                          head, t0, n, c.out, nullptr);
        if (sg == KVD_OK && stub::rec.calls[stub::kGather]) {
            accepted[stub::kGather]++;
            const kvd::GatherParams& g = stub::rec.gp;
            CHECK(g.seq >= 0 && g.seq < d->num_seqs && g.kv_head >= 0 && g.kv_head < d->num_kv_heads);
            CHECK(g.t0 >= 0 && g.n > 0 && (int64_t)g.t0 + g.n <= 16LL * d->max_blocks_per_seq);
            CHECK(g.chunk == (is_v ? v_chunk(fmt, d->head_dim) : k_chunk(fmt, d->head_dim)));
            CHECK((int64_t)g.n * g.D <= INT32_MAX);
        }
    }
    // operand export: page pairs of one (sequence, KV head)
    {
        const int seq = (int)(next() % 4), head = (int)(next() % 9);
        const int p0 = next() % 2 ? (int)(next() % 40) : pick(kEdges, kNE);
        const int np = next() % 2 ? (int)(next() % 40) : pick(kEdges, kNE);
        describe(*d, fmt, "operands");
        stub::reset();
        const int so = kvd_dequant_operands(d, fmt, fake(2), fake(3), c.scales, c.codebook, c.bt,
                                            seq, head, p0, np,
                                            static_cast<uint32_t*>(fake(9)), nullptr);
        if (so == KVD_OK && stub::rec.calls[stub::kOperands]) {
            accepted[stub::kOperands]++;
            const kvd::OperandParams& o = stub::rec.op;
            CHECK(o.pair0 >= 0 && o.npairs > 0 &&
                  2 * ((int64_t)o.pair0 + o.npairs) <= d->max_blocks_per_seq);
            CHECK(o.seq < d->num_seqs && o.kv_head < d->num_kv_heads);
        }
    }
    // append: n_new tokens per sequence
    {
        const int n_new = next() % 2 ? (int)(next() % 100) : pick(kEdges, kNE);
        describe(*d, fmt, "append");
        stub::reset();
        const int sa = kvd_append_kv(d, fmt, static_cast<const float*>(fake(16)),
                                     static_cast<const float*>(fake(17)), c.bt,
                                     static_cast<const int32_t*>(fake(18)), n_new, fake(2),
                                     fake(3), c.scales, c.codebook, c.sign, nullptr);
        if (sa == KVD_OK && stub::rec.calls[stub::kAppend]) {
            accepted[stub::kAppend]++;
            const kvd::AppendParams& a = stub::rec.ap;
            CHECK(a.T == n_new && a.T > 0 && a.ps == ((int64_t)n_new + 15) / 16 + 1);
            CHECK((int64_t)a.B * a.ps * a.Hkv <= INT32_MAX);
            CHECK(a.k_chunk == k_chunk(fmt, d->head_dim) && a.v_chunk == v_chunk(fmt, d->head_dim));
        }
        if (n_new < 0) CHECK(sa != KVD_OK);
    }
    // read probe
    {
        const int cb = next() % 2 ? 1024 << (next() % 4) : pick(kEdges, kNE);
        const int wpc = next() % 2 ? 4 * (int)(next() % 9) : pick(kEdges, kNE);
        const int lif = next() % 2 ? 1 << (next() % 6) : pick(kEdges, kNE);
        const int64_t n = next() % 2 ? (int64_t)(next() % 100000) : (int64_t)pick(kEdges, kNE);
        const size_t buf_bytes = next() % 2 ? (size_t)1 << (next() % 40) : SIZE_MAX;
        snprintf(where, sizeof(where), "probe cb=%d wpc=%d lif=%d n=%lld", cb, wpc, lif, (long long)n);
        stub::reset();
        const int sp = kvd_read_probe(fake(12), buf_bytes, static_cast<const int32_t*>(fake(13)),
                                      n, cb, wpc, lif, static_cast<uint32_t*>(fake(11)),
                                      (size_t)256 * 32 / 4 * 256 * 4, nullptr);
        if (sp == KVD_OK && stub::rec.calls[stub::kProbe]) {
            accepted[stub::kProbe]++;
            const kvd::ProbeParams& p = stub::rec.pp;
            CHECK((1024LL << p.log2_pieces) == cb && p.n == n && n > 0);
            CHECK(stub::rec.blocks == 256 * wpc / 4);
            CHECK((size_t)cb <= buf_bytes);
        }
    }
    free(d);
}

}  // namespace

int main(int argc, char** argv) {
    const long iters = argc > 1 ? atol(argv[1]) : 100000;
    rng_state = argc > 2 ? strtoull(argv[2], nullptr, 10) : 0x9E3779B97F4A7C15ULL;
    if (!rng_state) rng_state = 1;
    fixed_cases();
    for (long i = 0; i < iters; ++i) sweep_one();
    if (failures) {
        fprintf(stderr, "%d failed checks\n", failures);
        return 1;
    }
    printf("abi_sweep: %ld sweep cases, all checks passed; launches reached: partitions %ld, "
           "reduce %ld, gather %ld, operands %ld, append %ld, probe %ld; skewed runs %ld, "
           "early-skewed %ld, one-block %ld\n", iters,
           accepted[stub::kPartitions], accepted[stub::kReduce], accepted[stub::kGather],
           accepted[stub::kOperands], accepted[stub::kAppend], accepted[stub::kProbe], skewed,
           early, single);
    return 0;
}
