// Internal interface between the C-ABI host layer (kvd_api.cpp) and the HIP kernels
// (kvd_kernels.hip).  Not installed; the public contract is include/kvdecode.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvd {

constexpr int kPageTokens = 16;     // tokens per page (block_size)
constexpr int kAutoPartition = 512; // partition size of the automatic split
constexpr int kAutoSplitMin = 1024; // automatic split only from this many attended tokens
constexpr int kMaxGroup = 16;       // query heads one MFMA tile (one wave) handles
constexpr int kMaxRun = 4;          // cap on the automatic partitions-per-wave choice (ragged)
constexpr int kMaxRunUniform = 8;   // ... for a batch of equal lengths
// Wide layout of the partition kernel: one 4-wave workgroup per CU (one wave per SIMD; its LDS
// area of 137 KB keeps a second workgroup off the CU), with runs of up to kMaxRunWide
// partitions.  Built for
// single-query BF16 at head_dim 128, where the random-page stream reads faster with half the
// waves (BF16 16 x 32K: 380 against 390 us per call); the host takes it only when such runs
// cover the chip in one round (a large ragged batch balances better with short runs).
constexpr int kMaxRunWide = 8;
constexpr bool wide_layout_built(int fmt, int d, bool mq) { return fmt == 0 && d == 128 && !mq; }
// Query tiles per wave: BF16 / FP8 in the two-workgroup layout also have a build in which one
// wave computes two 16-row query tiles of a KV head (more than 16 rows per KV head: query
// groups above 16, e.g. MQA, or a chunk of queries times the group), so the tiles share every
// page load and dequantisation.
constexpr bool tile_pairs_built(int fmt, bool /*mq: both builds*/, bool wide) {
    return (fmt == 0 || fmt == 1) && !wide;
}
// Waves per workgroup of the partition kernel: 4 for BF16 / FP8 (two workgroups per CU), 8 for
// the codebook formats (sharing conflict-free codebook tables: 132 KB for Turbo4 / Turbo3, 141 KB
// of LDS with the query rows, one workgroup per CU; 64 KB for Turbo8).  Measured on Turbo4 / Turbo3: twelve waves per workgroup
// (three per SIMD, one page pair in flight) ran 1-4% slower than eight with two pairs in flight.
constexpr int waves_per_group(int fmt) { return fmt >= 2 ? 8 : 4; }
// Waves per SIMD the partition kernel is compiled for (its register budget: 512 / this).
constexpr int waves_per_simd(bool wide) { return wide ? 1 : 2; }
// Resident waves per CU the automatic run choice fills (Turbo8 could hold two workgroups per
// CU, but sixteen waves read its random pages more slowly than eight).
constexpr int waves_per_cu(bool wide) { return wide ? 4 : 8; }
// Rows of the per-wave LDS merge area of the BF16 / FP8 partition kernel (the unsplit merge
// uses the first kMaxGroup).  Its size is what holds the kernel at two workgroups per CU
// (68.9 KB each at D = 128) or one in the wide layout (137 KB).
constexpr int stage_rows(int d, bool wide) { return (wide ? 8192 : 4096) / d; }

enum PartMode : int32_t { kPartAuto = 0, kPartFixed = 1, kPartNever = 2 };

// Partition workspace of the allocation-free entry point: a device array inside the library,
// one per GPU (KVD_NOALLOC_WORKSPACE_BYTES in include/kvdecode.h).
constexpr size_t kNoAllocWorkspaceBytes = (size_t)128 << 20;

// Everything a kernel needs, passed by value as the kernel argument.
struct LaunchParams {
    const uint16_t* q;        // bf16 [B][Hq][D]
    const uint8_t* k;         // K pool
    const uint8_t* v;         // V pool
    const int32_t* bt;        // [B][max_blocks]
    const int32_t* ctx;       // [B]
    const int32_t* win;       // [B] or nullptr
    const float* scales;      // fp8 [2][Hkv]; turbo8 [Hkv] K scales; else unused (the
                              // codebook norms sit inside the cache chunks)
    const float* codebook;    // turbo levels (K then V; turbo8: V only)
    const float* sign;        // turbo [D]
    const float* alibi;       // [Hq] ALiBi slopes or nullptr
    float* out;               // [B][Hq][D]
    float* ws_m;              // [B][Hq][P]
    float* ws_l;              // [B][Hq][P]
    float* ws_o;              // [B][Hq][P][D]
    int64_t k_chunk;          // bytes per (page, KV head), K
    int64_t v_chunk;          // bytes per (page, KV head), V
    int32_t B, Hq, Hkv, g, D;
    int32_t nq;               // queries per sequence (a chunk at the last positions; 1 = decode)
    int32_t qt;               // query tiles per KV head: ceil(nq * g / kMaxGroup)
    int32_t nt;               // query tiles per work unit (1, or 2: tile_pairs_built)
    int32_t qg;               // work units per KV head: ceil(qt / nt)
    int32_t max_blocks, pool, max_ctx;
    int32_t part_mode;        // PartMode
    int32_t part_size;        // tokens per partition (split sequences)
    int32_t P;                // partitions per sequence in the workspace / grid
    int32_t kbits;            // turbo K index width (4 or 3)
    int32_t run_tokens;       // tokens of one wave's run (split sequences), >= part_size
    int32_t run_skew;         // 0, or tokens added to the runs of even run blocks and taken
                              // from those of odd ones (a multiple of 32; see run_blocks)
    int32_t early_skew;       // 0, or tokens added to every run of the block pairs the grid
                              // dispatches first and taken from the others (run_skew > 0 only)
    int32_t run_pairs;        // run block pairs per sequence in the grid (early_skew > 0)
    float softmax_scale;
    float softcap;
};

struct GatherParams {
    const uint8_t* cache;
    const float* scales;
    const float* codebook;
    const int32_t* bt;
    float* out;
    int64_t chunk;
    int32_t fmt, is_v, Hkv, D, max_blocks, pool, seq, kv_head, t0, n, kbits;
};

// Arguments of the operand export: the partition kernel's load and dequantisation code run on
// page pairs pair0 .. pair0 + npairs - 1 of one (sequence, KV head); lp carries the cache,
// scales, codebook, block table and sizes exactly as a decode launch does.
struct OperandParams {
    LaunchParams lp;
    uint32_t* out;            // [npairs][64 lanes][D + 16] words
    int32_t seq, kv_head, pair0, npairs;
};
// 32-bit words the operand export writes per (pair, lane): QK operands (x0 x1 y0 y1 per step,
// D / 2 words), PV operands (v0 v1 per tile, D / 2 words), then 16 norm words.
constexpr int operand_words(int d) { return d + 16; }

// Arguments of the KV append (quantize-on-write) kernel.
struct AppendParams {
    const float* k_new;       // [B][T][Hkv][D] fp32
    const float* v_new;
    const int32_t* bt;        // [B][max_blocks]
    const int32_t* pos;       // [B] token index of each sequence's first new token
    uint8_t* k;               // K pool
    uint8_t* v;               // V pool
    const float* scales;      // FP8: [2][Hkv]; Turbo8: [Hkv] K scales (read); else unused
    const float* codebook;    // codebook formats: K levels then 16 V levels (Turbo8: V levels)
    const float* sign;        // codebook formats: [D]
    int64_t k_chunk, v_chunk;
    int32_t fmt, B, T, Hkv, D, max_blocks, pool, kbits;
    int32_t ps;               // page slots per sequence: pages one sequence's T new tokens touch, at most
};

// Arguments of the HBM read probe (kvd_read_probe).
struct ProbeParams {
    const uint8_t* buf;
    const int32_t* ids;       // chunk indices, read in this order
    uint32_t* sink;           // one word per lane of every wave
    int64_t n;                // chunks to read
    int64_t buf_bytes;
    int32_t log2_pieces;      // chunk = 1 KB << log2_pieces
};

// Launches `kernel` (which takes one parameter struct by value) and returns the status of this
// launch alone.  hipGetLastError() after a triple-chevron launch would also report an error
// left pending by any earlier, unrelated runtime call on the thread (the caller's, or another
// library's) and blame this launch for it.
template <typename Params>
inline hipError_t launch_kernel(void (*kernel)(Params), dim3 grid, dim3 block, hipStream_t s,
                                const Params& p) {
    void* args[] = {const_cast<Params*>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, s);
}

// Launchers (kvd_kernels.hip, kvd_append.hip).  Return hipSuccess or the launch error.
hipError_t launch_partitions(int fmt, bool wide, const LaunchParams& p, dim3 grid, hipStream_t s);
hipError_t launch_reduce(int fmt, const LaunchParams& p, hipStream_t s);
hipError_t launch_gather(const GatherParams& p, hipStream_t s);
hipError_t launch_operands(int fmt, const OperandParams& p, hipStream_t s);

// Device address of the library's static workspace array on the current device (looked up
// with hipGetSymbolAddress on the first call per device, then cached).
hipError_t noalloc_workspace(void** ptr);
hipError_t launch_append(const AppendParams& p, hipStream_t s);
hipError_t launch_read_probe(const ProbeParams& p, int blocks, int loads_in_flight, hipStream_t s);

}  // namespace kvd
