// HIP kernels for single-query decode attention over a paged KV cache on gfx950 (MI355X).
//
// Two phases, as in turboquant-rs 0.4.1 src/cache/cuda/attention.rs ("partitioned attention +
// reduce"; 512-token partitions; fp32 per-partition max, sum and output) and the attention.rs
// README (Split-K decode for every cache format from 1024 tokens on, one shared float reduce):
//
//   partition_kernel<FMT, D>  one workgroup (4 waves) per (partition, KV head, sequence).
//       Each wave walks pairs of 16-token pages.  Per pair it
//         - loads K and V of both pages with 16-byte (or narrower, for the packed V rows)
//           coalesced loads straight into MFMA operand registers;
//         - computes S^T = K Q^T for the 32 tokens x 16 query slots (the GQA group, zero
//           padded) with v_mfma_f32_16x16x32_{bf16,f16}, dequantising FP8 / codebook indices
//           in registers on the way (FP8 -> bf16 is exact; codebook levels come from a 16-entry
//           fp16 table in LDS);
//         - runs an fp32 online softmax in the base-2 domain (max across the four 16-lane
//           groups by cross-lane shuffles);
//         - accumulates O^T += V^T P^T with the same MFMA, P fed as bf16 hi + lo halves (BF16,
//           FP8: ~2^-16 relative) or as fp16 p * vnorm / running-max(vnorm) (codebook formats).
//       The MFMA output layout of S^T (lane = query, 4 lane groups x 4 rows = 16 tokens) is
//       exactly the B-operand layout of P^T for the PV product once the two pages are
//       interleaved as below, so no data moves between the QK and PV products.
//       The four waves merge their (max, sum, output) through LDS; the workgroup writes its
//       partition triple to the workspace, or the final row when the sequence is not split.
//   reduce_kernel<FMT, D>    one workgroup per (query head, sequence): LSE merge of the
//       partition triples, then (codebook formats) the inverse rotation diag(s) H / sqrt(D).
//   gather_kernel            test export: dequantised values through the block table with the
//       same page addressing, index unpacking and FP8 decode as the attention kernel.
//
// MFMA 16x16x32 operand layout used throughout (lane = 0..63, n = lane % 16, j = lane / 16):
//   A operand: row n, 8 consecutive k-slots of group j;  B operand: column n, same k-slots;
//   C/D: column n, rows 4j..4j+3.
// Token placement for one page pair (pages A, B): QK tile X row m holds token
//   (page m/8, slot 8*((m/4)%2) + m%4), tile Y the slot 4 higher; after the QK product lane
//   (n, j) then holds query n's logits for tokens (page j/2, slots 8*(j%2) + e), e = 0..7,
//   which is also the k-slot order of group j in the PV product.
#include <math.h>

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

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

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

__device__ __forceinline__ float wave_max16x(float v) {   // max over the 4 lane groups
    v = fmaxf(v, __shfl_xor(v, 16));
    return fmaxf(v, __shfl_xor(v, 32));
}

// 4 E4M3FN codes (little-endian bytes of w) -> 4 bf16 in two packed pairs.  Exact: every
// E4M3FN value is a bf16 value.  gfx950 decodes OCP E4M3FN natively.
__device__ __forceinline__ u32x2 fp8x4_to_bf16(uint32_t w) {
    bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// 8 4-bit indices (index e at bits 4e of w) -> 8 fp16 table values as 4 packed pairs.
__device__ __forceinline__ u32x4 lut_nib8(const _Float16* lut, uint32_t w) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f16x2 h = {lut[(w >> (8 * i)) & 15u], lut[(w >> (8 * i + 4)) & 15u]};
        r[i] = __builtin_bit_cast(uint32_t, h);
    }
    return r;
}
// 8 3-bit indices (index e at bits 3e of the low 24 bits of f) -> 8 fp16 table values.
__device__ __forceinline__ u32x4 lut_tri8(const _Float16* lut, uint32_t f) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f16x2 h = {lut[(f >> (6 * i)) & 7u], lut[(f >> (6 * i + 3)) & 7u]};
        r[i] = __builtin_bit_cast(uint32_t, h);
    }
    return r;
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
    int L, lo;
    bool bad, split;
};

// Attended range [lo, L) of sequence b and whether it is split into partitions.
__device__ __forceinline__ SeqInfo seq_info(const LaunchParams& p, int b) {
    SeqInfo s;
    int L = p.ctx[b];
    const int W = p.win ? p.win[b] : 0;
    s.bad = (L < 0) || (L > p.max_ctx) || (W < 0);
    if (s.bad) L = 0;
    s.L = L;
    s.lo = (W > 0 && L > W) ? L - W : 0;
    const int span = L - s.lo;
    s.split = p.part_mode == kPartFixed ? true
            : (p.part_mode == kPartNever ? false : span >= kAutoSplitMin);
    return s;
}

// ------------------------------------------------------------------------------------------
// phase 1: partitioned attention
// ------------------------------------------------------------------------------------------
template <int FMT, int D>
__global__ __launch_bounds__(kThreads, 2) void partition_kernel(const LaunchParams p) {
    constexpr bool kTurbo = (FMT == KVD_TURBO4 || FMT == KVD_TURBO3);
    constexpr int KS = D / 32;   // QK MFMA steps (k = 32 head elements each)
    constexpr int VT = D / 16;   // PV MFMA tiles (16 head elements each)
    static_assert(!kTurbo || D == 128, "codebook formats are built for head_dim 128");

    __shared__ float sm_m[kWaves][kMaxGroup];
    __shared__ float sm_l[kWaves][kMaxGroup];
    __shared__ float sm_o[kWaves][kMaxGroup][D];
    __shared__ float sm_row[kTurbo ? kMaxGroup * D : 1];   // query rotation / output rotation
    __shared__ float sm_rowscale[kMaxGroup];
    __shared__ _Float16 sm_lut[2][16];
    __shared__ float sm_lutscale[2];

    const int part = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, j = lane >> 4;
    const int g = p.g;
    const SeqInfo si = seq_info(p, b);
    float* out_rows = p.out + ((size_t)b * p.Hq + (size_t)hk * g) * D;

    if (si.bad || si.L == 0) {
        if (part == 0) {
            const float v = si.bad ? __builtin_nanf("") : 0.0f;
            for (int i = tid; i < g * D; i += kThreads) out_rows[i] = v;
        }
        return;
    }
    int lo, hi;
    if (!si.split) {
        if (part != 0) return;
        lo = si.lo;
        hi = si.L;
    } else {
        lo = max(si.lo, part * p.part_size);
        hi = min(si.L, (part + 1) * p.part_size);
        if (lo >= hi) return;
    }

    // ---- query operand (B of the QK product): lane (n, j), step s -------------------------
    const int qn = min(n, g - 1);          // clamp the address; rows n >= g are zeroed
    const bool qlive = n < g;
    const uint16_t* qrow = p.q + ((size_t)b * p.Hq + (size_t)hk * g + qn) * D;
    u32x4 qop[KS];
    float zscale;           // logit -> base-2 softmax argument (without per-token factors)
    float oscale = 1.0f;    // accumulator -> output units (FP8 V scale / codebook scales)

    if constexpr (kTurbo) {
        // codebook tables (fp16, scaled by a power of two so the largest level is in [0.5, 1))
        if (wave == 0) {
            const int kl = 1 << p.kbits;
            const int which = lane >> 4, idx = lane & 15;
            float c = 0.0f;
            if (which == 0 && idx < kl) c = p.codebook[idx];
            if (which == 1) c = p.codebook[kl + idx];
            float mx = fabsf(c);
            mx = fmaxf(mx, __shfl_xor(mx, 1));
            mx = fmaxf(mx, __shfl_xor(mx, 2));
            mx = fmaxf(mx, __shfl_xor(mx, 4));
            mx = fmaxf(mx, __shfl_xor(mx, 8));
            const float sc = pow2_normaliser(mx);
            if (which < 2) sm_lut[which][idx] = (_Float16)(c * sc);
            if (which < 2 && idx == 0) sm_lutscale[which] = sc;
        }
        // q_rot = H (s * q): rows of the group in LDS, then the butterfly
        for (int i = tid; i < g * D; i += kThreads) {
            const int r = i / D, d = i % D;
            const uint16_t qb = p.q[((size_t)b * p.Hq + (size_t)hk * g + r) * D + d];
            sm_row[i] = bf16_bits_to_f32(qb) * p.sign[d];
        }
        __syncthreads();
        fwht_rows<D>(sm_row, g, tid, kThreads);
        for (int r = wave; r < g; r += kWaves) {       // per-row power-of-two normaliser
            float mx = fmaxf(fabsf(sm_row[r * D + lane]), fabsf(sm_row[r * D + 64 + lane]));
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
            if (lane == 0) sm_rowscale[r] = pow2_normaliser(mx);
        }
        __syncthreads();
        const float qs = sm_rowscale[qn];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int d0 = 32 * j + 8 * s;
            u32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f16x2 h = {(_Float16)(sm_row[qn * D + d0 + 2 * i] * qs),
                           (_Float16)(sm_row[qn * D + d0 + 2 * i + 1] * qs)};
                w[i] = qlive ? __builtin_bit_cast(uint32_t, h) : 0u;
            }
            qop[s] = w;
        }
        zscale = p.softmax_scale * kLog2e / (qs * sm_lutscale[0] * sqrtf((float)D));
        oscale = 1.0f / sm_lutscale[1];
    } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int d0 = (FMT == KVD_BF16) ? 32 * s + 8 * j : 64 * (s / 2) + 16 * j + 8 * (s % 2);
            const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + d0);
            qop[s] = qlive ? w : u32x4{0u, 0u, 0u, 0u};
        }
        zscale = p.softmax_scale * kLog2e;
        if constexpr (FMT == KVD_FP8_E4M3) {
            zscale *= p.scales[hk];
            oscale = p.scales[p.Hkv + hk];
        }
    }
    const bool capped = p.softcap > 0.0f;
    const float inv_cap = capped ? 1.0f / p.softcap : 0.0f;

    // ---- main loop over page pairs -------------------------------------------------------
    const int pg0 = lo / kPageTokens, pg1 = (hi - 1) / kPageTokens + 1;
    const int npairs = (pg1 - pg0 + 1) >> 1;
    const int32_t* btrow = p.bt + (size_t)b * p.max_blocks;
    const int a_sel = n >> 3;                              // QK A row n: page of its token
    const int a_pos = 8 * ((n >> 2) & 1) + (n & 3);        // slot of its tile-X token
    const int v_sel = j >> 1;                              // PV / softmax: page of group j
    const int v_pos0 = 8 * (j & 1);                        // first slot of group j

    f32x4 oacc[VT];
#pragma unroll
    for (int i = 0; i < VT; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.0f;
    float sig_run = 1.17549435e-38f;   // running max of V norms (codebook formats)
    bool bad_ids = false;

#pragma unroll 1
    for (int k = wave; k < npairs; k += kWaves) {
        const int pgA = pg0 + 2 * k, pgB = pgA + 1;
        const bool hasB = pgB < pg1;
        int physA = btrow[pgA];
        int physB = hasB ? btrow[pgB] : physA;
        if (physA < 0 || physA >= p.pool) { bad_ids = true; physA = 0; }
        if (physB < 0 || physB >= p.pool) { bad_ids = true; physB = 0; }
        const bool full = (pgA * kPageTokens >= lo) && hasB && ((pgB + 1) * kPageTokens <= hi);

        const size_t headA = (size_t)physA * p.Hkv + hk, headB = (size_t)physB * p.Hkv + hk;
        const uint8_t* kch = p.k + (a_sel ? headB : headA) * p.k_chunk;
        const uint8_t* vch = p.v + (v_sel ? headB : headA) * p.v_chunk;

        // ---- QK: S^T tiles X and Y ----
        f32x4 sx = {0.f, 0.f, 0.f, 0.f}, sy = {0.f, 0.f, 0.f, 0.f};
        if constexpr (FMT == KVD_BF16) {
            u32x4 kx[KS], ky[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const uint8_t* base = kch + 1024 * s + 256 * j + 16 * a_pos;
                kx[s] = *reinterpret_cast<const u32x4*>(base);
                ky[s] = *reinterpret_cast<const u32x4*>(base + 64);
            }
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                sx = mfma_bf16(kx[s], qop[s], sx);
                sy = mfma_bf16(ky[s], qop[s], sy);
            }
        } else if constexpr (FMT == KVD_FP8_E4M3) {
            u32x4 kx[KS / 2], ky[KS / 2];
#pragma unroll
            for (int i = 0; i < KS / 2; ++i) {
                const uint8_t* base = kch + 1024 * i + 256 * j + 16 * a_pos;
                kx[i] = *reinterpret_cast<const u32x4*>(base);
                ky[i] = *reinterpret_cast<const u32x4*>(base + 64);
            }
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int i = s / 2, h = s % 2;
                const u32x2 ax0 = fp8x4_to_bf16(kx[i][2 * h]), ax1 = fp8x4_to_bf16(kx[i][2 * h + 1]);
                const u32x2 ay0 = fp8x4_to_bf16(ky[i][2 * h]), ay1 = fp8x4_to_bf16(ky[i][2 * h + 1]);
                sx = mfma_bf16(u32x4{ax0[0], ax0[1], ax1[0], ax1[1]}, qop[s], sx);
                sy = mfma_bf16(u32x4{ay0[0], ay0[1], ay1[0], ay1[1]}, qop[s], sy);
            }
        } else if constexpr (FMT == KVD_TURBO4) {
            const uint8_t* base = kch + 256 * j + 16 * a_pos;
            const u32x4 kx = *reinterpret_cast<const u32x4*>(base);
            const u32x4 ky = *reinterpret_cast<const u32x4*>(base + 64);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                sx = mfma_f16(lut_nib8(sm_lut[0], kx[s]), qop[s], sx);
                sy = mfma_f16(lut_nib8(sm_lut[0], ky[s]), qop[s], sy);
            }
        } else {  // KVD_TURBO3
            const uint32_t* bx = reinterpret_cast<const uint32_t*>(kch + 192 * j + 12 * a_pos);
            const uint32_t* by = reinterpret_cast<const uint32_t*>(kch + 192 * j + 12 * (a_pos + 4));
            const uint32_t x0 = bx[0], x1 = bx[1], x2 = bx[2];
            const uint32_t y0 = by[0], y1 = by[1], y2 = by[2];
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                sx = mfma_f16(lut_tri8(sm_lut[0], tri_field(x0, x1, x2, s)), qop[s], sx);
                sy = mfma_f16(lut_tri8(sm_lut[0], tri_field(y0, y1, y2, s)), qop[s], sy);
            }
        }

        // ---- V operand loads (A of the PV product): tile i, row d = 16 i + n ----
        u32x4 vop[VT];
        if constexpr (FMT == KVD_BF16) {
#pragma unroll
            for (int i = 0; i < VT; ++i)
                vop[i] = *reinterpret_cast<const u32x4*>(vch + (16 * i + n) * 32 + 2 * v_pos0);
        } else if constexpr (FMT == KVD_FP8_E4M3) {
#pragma unroll
            for (int i = 0; i < VT; ++i) {
                const u32x2 w = *reinterpret_cast<const u32x2*>(vch + (16 * i + n) * 16 + v_pos0);
                const u32x2 a0 = fp8x4_to_bf16(w[0]), a1 = fp8x4_to_bf16(w[1]);
                vop[i] = u32x4{a0[0], a0[1], a1[0], a1[1]};
            }
        } else {
#pragma unroll
            for (int i = 0; i < VT; ++i) {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(vch + (16 * i + n) * 8 + v_pos0 / 2);
                vop[i] = lut_nib8(sm_lut[1], w);
            }
        }

        // per-token factors (codebook formats): norms of group j's eight tokens
        float kn[8], vn[8];
        if constexpr (kTurbo) {
            const size_t nbase = ((v_sel ? headB : headA) * kPageTokens + v_pos0);
            const f32x4 k0 = *reinterpret_cast<const f32x4*>(p.scales + nbase);
            const f32x4 k1 = *reinterpret_cast<const f32x4*>(p.scales + nbase + 4);
            const size_t voff = (size_t)p.pool * p.Hkv * kPageTokens;
            const f32x4 v0 = *reinterpret_cast<const f32x4*>(p.scales + voff + nbase);
            const f32x4 v1 = *reinterpret_cast<const f32x4*>(p.scales + voff + nbase + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kn[e] = k0[e]; kn[4 + e] = k1[e];
                vn[e] = v0[e]; vn[4 + e] = v1[e];
            }
        }

        // ---- logits, mask, online softmax ----
        float z[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { z[e] = sx[e]; z[4 + e] = sy[e]; }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = z[e] * zscale;
            if constexpr (kTurbo) x *= kn[e];
            if (capped) {   // cap * tanh(x_nat / cap), in the base-2 domain
                const float y = x * (1.0f / kLog2e) * inv_cap;
                const float t = fast_exp2(2.0f * kLog2e * y);
                x = p.softcap * kLog2e * (1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + t));
            }
            z[e] = x;
        }
        uint32_t vmask = 0xFFu;
        if (!full) {
            const int tok0 = (pgA + v_sel) * kPageTokens + v_pos0;
            vmask = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = tok0 + e;
                const bool ok = (t >= lo) && (t < hi) && (v_sel == 0 || hasB);
                vmask |= (ok ? 1u : 0u) << e;
                z[e] = ok ? z[e] : -INFINITY;
            }
        }
        float mloc = z[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mloc = fmaxf(mloc, z[e]);
        mloc = wave_max16x(mloc);
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = fast_exp2(m_run - m_new);
        float pe[8], psum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) { pe[e] = fast_exp2(z[e] - m_new); psum += pe[e]; }
        l_run = l_run * alpha + psum;
        m_run = m_new;

        // ---- P operand and PV ----
        if constexpr (kTurbo) {
            float vloc = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                vn[e] = ((vmask >> e) & 1u) ? vn[e] : 0.0f;
                vloc = fmaxf(vloc, vn[e]);
            }
            vloc = wave_max16x(vloc);
            const float sig_new = fmaxf(sig_run, vloc);
            const float f = alpha * (sig_run / sig_new);
            sig_run = sig_new;
            const float inv_sig = 1.0f / sig_new;
            u32x4 pop;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f16x2 h = {(_Float16)(pe[2 * i] * vn[2 * i] * inv_sig),
                           (_Float16)(pe[2 * i + 1] * vn[2 * i + 1] * inv_sig)};
                pop[i] = __builtin_bit_cast(uint32_t, h);
            }
            if (!full) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t mk = (((vmask >> (2 * i)) & 1u) ? 0x0000FFFFu : 0u) |
                                        (((vmask >> (2 * i + 1)) & 1u) ? 0xFFFF0000u : 0u);
#pragma unroll
                    for (int t = 0; t < VT; ++t) vop[t][i] &= mk;
                }
            }
#pragma unroll
            for (int t = 0; t < VT; ++t) oacc[t] = mfma_f16(vop[t], pop, oacc[t] * f);
        } else {
            u32x4 phi, plo;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t a = __float_as_uint(pe[2 * i]), c = __float_as_uint(pe[2 * i + 1]);
                const uint32_t ah = a & 0xFFFF0000u, ch = c & 0xFFFF0000u;
                phi[i] = (a >> 16) | ch;
                bf16x2 l = {(__bf16)(pe[2 * i] - __uint_as_float(ah)),
                            (__bf16)(pe[2 * i + 1] - __uint_as_float(ch))};
                plo[i] = __builtin_bit_cast(uint32_t, l);
            }
            if (!full) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t mk = (((vmask >> (2 * i)) & 1u) ? 0x0000FFFFu : 0u) |
                                        (((vmask >> (2 * i + 1)) & 1u) ? 0xFFFF0000u : 0u);
#pragma unroll
                    for (int t = 0; t < VT; ++t) vop[t][i] &= mk;
                }
            }
#pragma unroll
            for (int t = 0; t < VT; ++t) {
                f32x4 acc = oacc[t] * alpha;
                acc = mfma_bf16(vop[t], phi, acc);
                oacc[t] = mfma_bf16(vop[t], plo, acc);
            }
        }
    }

    // ---- merge the four waves --------------------------------------------------------------
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if constexpr (kTurbo) oscale *= sig_run;
    if (qlive) {
        if (j == 0) {
            sm_m[wave][n] = m_run;
            sm_l[wave][n] = l_run;
        }
#pragma unroll
        for (int t = 0; t < VT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) sm_o[wave][n][16 * t + 4 * j + r] = oacc[t][r] * oscale;
    }
    const bool wg_bad = __syncthreads_or(bad_ids ? 1 : 0) != 0;

    const size_t row0 = (size_t)b * p.Hq + (size_t)hk * g;
    for (int i = tid; i < g * D; i += kThreads) {
        const int r = i / D, d = i % D;
        float M = sm_m[0][r];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][r]);
        float wsum = 0.0f, acc = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float sc = fast_exp2(sm_m[w][r] - M);
            wsum += sm_l[w][r] * sc;
            acc += sm_o[w][r][d] * sc;
        }
        float o = acc / wsum;
        if (wg_bad) o = __builtin_nanf("");
        if (si.split) {
            const size_t slot = (row0 + r) * p.P + part;
            p.ws_o[slot * D + d] = o;
            if (d == 0) {
                p.ws_m[slot] = M;
                p.ws_l[slot] = wsum;
            }
        } else if constexpr (kTurbo) {
            sm_row[i] = o;
        } else {
            out_rows[i] = o;
        }
    }
    if constexpr (kTurbo) {
        if (!si.split) {   // inverse rotation of the final rows: diag(s) H o / sqrt(D)
            __syncthreads();
            fwht_rows<D>(sm_row, g, tid, kThreads);
            const float rs = 1.0f / sqrtf((float)D);
            for (int i = tid; i < g * D; i += kThreads) out_rows[i] = sm_row[i] * p.sign[i % D] * rs;
        }
    }
}

// ------------------------------------------------------------------------------------------
// phase 2: log-sum-exp merge of the partition triples
// ------------------------------------------------------------------------------------------
template <int FMT, int D>
__global__ __launch_bounds__(D) void reduce_kernel(const LaunchParams p) {
    constexpr bool kTurbo = (FMT == KVD_TURBO4 || FMT == KVD_TURBO3);
    __shared__ float sm[D];
    const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const SeqInfo si = seq_info(p, b);
    if (si.bad || si.L == 0 || !si.split) return;
    const int p0 = si.lo / p.part_size, p1 = (si.L - 1) / p.part_size;
    const size_t row = (size_t)b * p.Hq + hq;
    const float* ms = p.ws_m + row * p.P;
    const float* ls = p.ws_l + row * p.P;
    const float* os = p.ws_o + row * p.P * D;
    float M = -INFINITY;
    for (int q = p0; q <= p1; ++q) M = fmaxf(M, ms[q]);
    float wsum = 0.0f, acc = 0.0f;
    for (int q = p0; q <= p1; ++q) {
        const float w = ls[q] * fast_exp2(ms[q] - M);
        wsum += w;
        acc += w * os[(size_t)q * D + d];
    }
    float o = acc / wsum;
    if constexpr (kTurbo) {
        sm[d] = o;
        __syncthreads();
        fwht_rows<D>(sm, 1, d, D);
        o = sm[d] * p.sign[d] * (1.0f / sqrtf((float)D));
    }
    p.out[row * D + d] = o;
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
    } else if (p.fmt == KVD_FP8_E4M3) {
        const size_t off = p.is_v ? (size_t)d * 16 + pos : ((size_t)(d / 16) * 16 + pos) * 16 + d % 16;
        const uint32_t w = reinterpret_cast<const uint32_t*>(ch)[off / 4];
        const u32x2 bf = fp8x4_to_bf16(w);
        const int e = off % 4;
        const uint32_t pair = bf[e / 2];
        val = bf16_bits_to_f32((e & 1) ? (pair >> 16) : (pair & 0xFFFFu));
        val *= p.scales[(p.is_v ? p.Hkv : 0) + p.kv_head];
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
        const int kl = 1 << p.kbits;
        const float lvl = p.codebook[(p.is_v ? kl : 0) + idx];
        const size_t nb = (size_t)(p.is_v ? p.pool : 0) * p.Hkv * kPageTokens + head * kPageTokens + pos;
        val = p.scales[nb] * lvl;
    }
    p.out[i] = val;
}

template <int FMT, int D>
hipError_t launch_partitions_t(const LaunchParams& p, dim3 grid, hipStream_t s) {
    hipLaunchKernelGGL((partition_kernel<FMT, D>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}
template <int FMT, int D>
hipError_t launch_reduce_t(const LaunchParams& p, hipStream_t s) {
    hipLaunchKernelGGL((reduce_kernel<FMT, D>), dim3(p.Hq, p.B), dim3(D), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_partitions(int fmt, const LaunchParams& p, dim3 grid, hipStream_t s) {
    switch (fmt) {
        case KVD_BF16: return p.D == 64 ? launch_partitions_t<KVD_BF16, 64>(p, grid, s)
                                        : launch_partitions_t<KVD_BF16, 128>(p, grid, s);
        case KVD_FP8_E4M3: return p.D == 64 ? launch_partitions_t<KVD_FP8_E4M3, 64>(p, grid, s)
                                            : launch_partitions_t<KVD_FP8_E4M3, 128>(p, grid, s);
        case KVD_TURBO4: return launch_partitions_t<KVD_TURBO4, 128>(p, grid, s);
        default: return launch_partitions_t<KVD_TURBO3, 128>(p, grid, s);
    }
}

hipError_t launch_reduce(int fmt, const LaunchParams& p, hipStream_t s) {
    switch (fmt) {
        case KVD_BF16: return p.D == 64 ? launch_reduce_t<KVD_BF16, 64>(p, s)
                                        : launch_reduce_t<KVD_BF16, 128>(p, s);
        case KVD_FP8_E4M3: return p.D == 64 ? launch_reduce_t<KVD_FP8_E4M3, 64>(p, s)
                                            : launch_reduce_t<KVD_FP8_E4M3, 128>(p, s);
        case KVD_TURBO4: return launch_reduce_t<KVD_TURBO4, 128>(p, s);
        default: return launch_reduce_t<KVD_TURBO3, 128>(p, s);
    }
}

hipError_t launch_gather(const GatherParams& p, hipStream_t s) {
    const int total = p.n * p.D;
    hipLaunchKernelGGL(gather_kernel, dim3((total + 255) / 256), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace kvd
