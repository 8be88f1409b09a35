// KV append (quantize-on-write) for the paged cache on gfx950: stores new tokens in the layout
// the decode kernels read (include/kvdecode.h documents both).
//
// Formats as in the attention.rs README "KV Cache Formats" table (BF16, FP8 E4M3, and Turbo8,
// Turbo4 and Turbo3 with the Walsh-Hadamard rotation; Turbo8 writes K as FP8 and V as Turbo4
// does); the rotated-codebook recipe is the one the compressed-cache workload states: sign
// flip, orthonormal Walsh-Hadamard transform, fp32 L2 norm stored per token, nearest Lloyd-Max
// level per coordinate, little-endian bit packing (turboquant-rs 0.4.1
// src/cache/cuda/attention.rs reads exactly these: packed indices, per-token scales, a sign
// pattern and a codebook).
//
// Page-tiled: one workgroup (16 waves) per (sequence, page, KV head) that receives new tokens.
// The V layout is transposed (one row per head element, 16 token slots per row) and the 4-bit
// formats pack two tokens per byte, so a token alone owns no whole store unit.  The workgroup
// therefore assembles the page's K and V chunks in LDS -- starting from the chunk's current
// bytes when only part of the page is new -- encodes its new tokens into that image (wave w
// takes token slot w; lane l owns head elements 2l and 2l + 1 at D = 128, or l at D = 64) and
// writes both chunks back with 16-byte stores.  No other workgroup of the call touches the same
// (page, KV head), so no global atomics are needed.
//
// Every decision that picks a code is taken exactly:
//   BF16   round to nearest even on the fp32 bit pattern; NaN -> 0x7FC0;
//   FP8    q = x / scale in one correctly rounded fp32 division, then round to nearest even
//          OCP E4M3FN on the bit pattern, saturating to +-448; NaN -> 0x7F;
//   Turbo  the Hadamard butterflies in fp64 (exact for fp32 inputs: every partial sum of 128
//          fp32 values with +-1 weights fits the 53-bit significand unless their exponents
//          differ by more than 22 binades), r = y / sqrt(D); the norm is an fp64 sum of the
//          squares taken as a pairwise tree (adjacent elements, then adjacent lanes by xor
//          shuffles), its square root rounded to fp32; u = r / norm (fp64) and the index counts
//          the level midpoints (c_k + c_{k+1}) / 2 strictly below u (a tie takes the lower
//          level) -- a binary search over the ascending midpoints, computed once per workgroup
//          in fp64 (exact: the sum of two fp32 levels fits the fp64 significand).
#include <math.h>

#include "kvd_internal.h"
#include "kvdecode.h"

namespace kvd {
namespace {

constexpr int kAppendWaves = 16;   // one per token slot of a page
constexpr int kImageBytes = 2 * 32 * 128;   // largest K + V chunk pair (BF16, D = 128)

__device__ __forceinline__ uint32_t bf16_rne(float x) {
    const uint32_t b = __float_as_uint(x);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// fp32 -> OCP E4M3FN code, round to nearest even, saturating to +-448.
__device__ __forceinline__ uint32_t e4m3fn_rne(float q) {
    const uint32_t b = __float_as_uint(q);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return 0x7Fu;                  // NaN
    if (a >= 0x43E00000u) return sign | 0x7Eu;          // |q| >= 448 (and infinity)
    if (a < 0x3C800000u)                                // |q| < 2^-6: multiples of 2^-9
        return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;   // exponent | 3 mantissa bits
    r -= (127u - 7u) << 3;                                  // rebias
    return sign | (r < 0x7Eu ? r : 0x7Eu);
}

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
    const uint64_t u = __double_as_longlong(v);
    const uint32_t lo = __shfl_xor((uint32_t)u, m), hi = __shfl_xor((uint32_t)(u >> 32), m);
    return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

// Number of midpoints mid[0 .. n) (ascending) strictly below u, n < 16.
__device__ __forceinline__ uint32_t count_below(const double* mid, int n, double u) {
    uint32_t idx = 0;
#pragma unroll
    for (int step = 8; step >= 1; step >>= 1)
        if ((int)idx + step <= n && u > mid[idx + step - 1]) idx += step;
    return idx;
}

// One token vector (this lane's part of it) into the LDS image of its page: K chunk at byte 0,
// V chunk at byte k_chunk.  A codebook-stored token's fp32 norm goes to its slot of the 16
// norms after the chunk's indices (chunk_bytes - 64).
// mids: the level midpoints of K (row 0) and V (row 1), fp64, in LDS.
__device__ __forceinline__ void encode_token(const AppendParams& p, int which, const float* src,
                                             uint8_t* chunk, const double (*mids)[16],
                                             int t, int hk, int lane) {
    const bool t8 = p.fmt == KVD_TURBO8;
    const bool fp8 = p.fmt == KVD_FP8_E4M3 || (t8 && which == 0);   // Turbo8 K is FP8 K
    if (p.fmt == KVD_BF16 || fp8) {
        // FP8: scales [2][Hkv]; Turbo8: the [Hkv] K scales
        const float scale = !fp8 ? 1.0f : t8 ? p.scales[hk] : p.scales[which * p.Hkv + hk];
        for (int d = lane; d < p.D; d += 64) {
            const float x = src[d];
            if (p.fmt == KVD_BF16) {
                const uint16_t c = (uint16_t)bf16_rne(x);
                uint16_t* c16 = reinterpret_cast<uint16_t*>(chunk);
                if (which == 0) c16[((d / 8) * kPageTokens + t) * 8 + d % 8] = c;   // [D/8][16][8]
                else c16[d * kPageTokens + t] = c;                                   // [D][16]
            } else {
                const uint8_t c = (uint8_t)e4m3fn_rne(__fdiv_rn(x, scale));
                if (which == 0) chunk[((d / 16) * kPageTokens + t) * 16 + d % 16] = c;  // [D/16][16][16]
                else chunk[d * kPageTokens + t] = c;                                     // [D][16]
            }
        }
        return;
    }

    // ---- rotated codebook (D = 128): lane owns elements e0 = 2 lane, e1 = 2 lane + 1 ----
    const int e0 = 2 * lane;
    const float x0 = src[e0], x1 = src[e0 + 1];
    double y0 = (double)(x0 * p.sign[e0]), y1 = (double)(x1 * p.sign[e0 + 1]);
    {   // stage h = 1 inside the lane, then h = 2 .. 64 across lanes (partner lane ^ h / 2)
        const double a = y0, c = y1;
        y0 = a + c;
        y1 = a - c;
    }
#pragma unroll
    for (int h = 2; h < 128; h <<= 1) {
        const int m = h >> 1;
        const double o0 = shfl_xor_f64(y0, m), o1 = shfl_xor_f64(y1, m);
        const bool upper = (e0 & h) != 0;
        y0 = upper ? o0 - y0 : y0 + o0;
        y1 = upper ? o1 - y1 : y1 + o1;
    }
    const double rs = sqrt(128.0);
    const double r0 = y0 / rs, r1 = y1 / rs;
    double n2 = (double)x0 * (double)x0 + (double)x1 * (double)x1;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) n2 += shfl_xor_f64(n2, m);
    const float norm = (float)sqrt(n2);
    const double nd = (double)norm;
    const double u0 = nd > 0.0 ? r0 / nd : 0.0, u1 = nd > 0.0 ? r1 / nd : 0.0;

    const int nmid = (which ? 16 : 1 << p.kbits) - 1;
    const uint32_t i0 = count_below(mids[which], nmid, u0), i1 = count_below(mids[which], nmid, u1);
    if (lane == 0)   // after the chunk's indices
        reinterpret_cast<float*>(chunk + (which ? p.v_chunk : p.k_chunk) - 64)[t] = norm;

    if (which == 1) {   // V [D][8 B]: nibble t of rows e0 and e0 + 1 (words shared with the
                        // other waves' tokens: clear, then set, with LDS atomics)
        uint32_t* words = reinterpret_cast<uint32_t*>(chunk);
        const int sh = 4 * (t % 8);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            uint32_t* w = words + (e0 + k) * 2 + t / 8;
            atomicAnd(w, ~(0xFu << sh));
            atomicOr(w, (k ? i1 : i0) << sh);
        }
    } else if (p.kbits == 4) {   // K [D/32][16][16 B]: the lane's byte, indices e0, e0+1
        chunk[((e0 / 32) * kPageTokens + t) * 16 + (e0 % 32) / 2] = (uint8_t)(i0 | (i1 << 4));
    } else {   // K [D/32][16][12 B]: 32 3-bit indices per group, 6 bits per lane
        const int g = e0 / 32, pos6 = 6 * (lane % 16);     // bit offset inside the group
        const uint32_t v6 = i0 | (i1 << 3);
        uint32_t w[3] = {0u, 0u, 0u};
        const int wk = pos6 / 32, off = pos6 % 32;
        w[wk] = v6 << off;
        if (off > 26) w[wk + 1] = v6 >> (32 - off);
#pragma unroll
        for (int m = 1; m < 16; m <<= 1)
#pragma unroll
            for (int k = 0; k < 3; ++k) w[k] |= __shfl_xor(w[k], m);
        const int lg = lane % 16;
        if (lg < 3) {
            uint32_t* dst = reinterpret_cast<uint32_t*>(chunk + (g * kPageTokens + t) * 12);
            dst[lg] = lg == 0 ? w[0] : (lg == 1 ? w[1] : w[2]);
        }
    }
}

// Grid: B * p.ps * Hkv workgroups, KV head fastest, then the page slot s, then the sequence:
// page slot s of sequence b is page floor(first / 16) + s, first = max(positions[b], 0).
__global__ __launch_bounds__(64 * kAppendWaves) void append_kernel(const AppendParams p) {
    __shared__ uint4 image4[kImageBytes / 16];
    __shared__ double mids[2][16];   // codebook level midpoints: K (row 0), V (row 1)
    uint8_t* const image = reinterpret_cast<uint8_t*>(image4);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t wg = blockIdx.x;
    const int hk = (int)(wg % p.Hkv);
    const int s = (int)((wg / p.Hkv) % p.ps);
    const int b = (int)(wg / ((int64_t)p.Hkv * p.ps));
    const int64_t pos = p.pos[b];
    const int64_t first = pos > 0 ? pos : 0, end = pos + p.T;   // new tokens [first, end)
    if (first >= end) return;
    const int64_t pg = first / kPageTokens + s;
    if (pg * kPageTokens >= end) return;                       // past the new tokens
    if (pg >= p.max_blocks) return;                            // no page for them
    const int phys = p.bt[(size_t)b * p.max_blocks + pg];
    if (phys < 0 || phys >= p.pool) return;                    // not a pool page
    const int t_lo = (int)((first > pg * kPageTokens ? first : pg * kPageTokens) - pg * kPageTokens);
    const int t_hi = (int)((end < (pg + 1) * kPageTokens ? end : (pg + 1) * kPageTokens) - pg * kPageTokens);
    const size_t head = (size_t)phys * p.Hkv + hk;
    uint8_t* const kdst = p.k + head * p.k_chunk;
    uint8_t* const vdst = p.v + head * p.v_chunk;
    const int nk = (int)(p.k_chunk / 16), nv = (int)(p.v_chunk / 16);

    // 1. the page's current bytes, unless every slot of it is new; the codebook midpoints
    if (t_lo > 0 || t_hi < kPageTokens) {
        for (int i = tid; i < nk + nv; i += 64 * kAppendWaves)
            image4[i] = i < nk ? reinterpret_cast<const uint4*>(kdst)[i]
                               : reinterpret_cast<const uint4*>(vdst)[i - nk];
    }
    if (p.fmt >= KVD_TURBO4 && tid < 32) {   // levels: 2^kbits K then 16 V (Turbo8: 16 V)
        const int which = tid >> 4, k = tid & 15;
        const int kl = p.fmt == KVD_TURBO8 ? 0 : 1 << p.kbits;
        const int n = which ? 16 : kl;
        const float* lv = p.codebook + (which ? kl : 0);
        if (k + 1 < n) mids[which][k] = ((double)lv[k] + (double)lv[k + 1]) / 2.0;
    }
    __syncthreads();

    // 2. encode the new tokens of the page into the image: wave w takes slot w
    const int t = wave;
    if (t >= t_lo && t < t_hi) {
        const int64_t i = pg * kPageTokens + t - pos;            // index among the call's tokens
        const size_t row = ((size_t)b * p.T + (size_t)i) * p.Hkv + hk;
        encode_token(p, 0, p.k_new + row * p.D, image, mids, t, hk, lane);
        encode_token(p, 1, p.v_new + row * p.D, image + p.k_chunk, mids, t, hk, lane);
    }
    __syncthreads();

    // 3. both chunks back, 16 bytes per store
    for (int i = tid; i < nk + nv; i += 64 * kAppendWaves) {
        if (i < nk) reinterpret_cast<uint4*>(kdst)[i] = image4[i];
        else reinterpret_cast<uint4*>(vdst)[i - nk] = image4[i];
    }
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
    const int64_t blocks = (int64_t)p.B * p.ps * p.Hkv;
    return launch_kernel(append_kernel, dim3((unsigned)blocks), dim3(64 * kAppendWaves), s, p);
}

}  // namespace kvd
