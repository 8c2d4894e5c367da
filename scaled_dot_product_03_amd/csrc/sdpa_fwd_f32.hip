// gfx950 fused attention forward, fp32 inputs and fp32 arithmetic (the high-precision path).
//
// Same operation and conventions as the bf16 kernel -- the four attention steps of the
// "jax-gpu-05-attention-gpu" codelab, section 1, with index-generated causal / sliding-window
// masks, T5 or full additive bias and GQA head sharing -- but computed with fp32 FMAs and
// full-precision expf, for workloads stored in fp32 (the codelab's fp32 inputs, section 3).
// It favours exactness over speed: one lane per query row, 64 rows per workgroup; key tiles
// staged in LDS are split over the waves of the workgroup (8; 4 at D = 256), each wave keeping its own
// online softmax (max, sum, output) over its keys; the eight partial results of a row are
// merged in wave order at the end, so the summation order is fixed.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sdpa_params.h"

namespace sdpa {

constexpr int kRowsF32 = 64;       // query rows per workgroup: one per lane of every wave
// waves per workgroup, each taking an equal share of every key tile; at D = 256 four (one wave
// per SIMD, so the 256 output registers of a lane fit the register file)
template <int D> constexpr int waves_f32() { return D == 256 ? 4 : 8; }
template <int D> constexpr int keys_f32() { return D <= 64 ? 64 : 32; }   // keys per tile

// keeps the compiler from moving loads across this point (bounds the registers that loads
// hoisted ahead of their use would hold)
__device__ __forceinline__ void load_fence() { asm volatile("" ::: "memory"); }

template <int D, int MASK, int BIAS>
__global__ __launch_bounds__(kRowsF32 * waves_f32<D>()) void sdpa_fwd_f32_kernel(const FwdParams p) {
    constexpr int NW = waves_f32<D>();
    constexpr int KT = keys_f32<D>();
    constexpr int KW = KT / NW;                 // keys of a tile per wave
    constexpr int NT = kRowsF32 * NW;           // threads
    constexpr int QP = D + 4;                   // Q row pitch in LDS (16-byte aligned rows)
    constexpr bool QREG = D <= 64;              // Q row held in registers (else read from LDS)
    constexpr int VC = D < 32 ? D : 32;         // head-dim chunk of one P.V step
    __shared__ __attribute__((aligned(16))) float qs[kRowsF32 * QP];
    __shared__ __attribute__((aligned(16))) float kvs[2 * KT * D];   // K tile, V tile; then merge
    __shared__ float mls[2][NW][kRowsF32];
    // T5 bias by relative position rel = key - query, clamped to +-kSat (the bucket is constant
    // beyond): t5r[kSat + rel]
    constexpr bool IS_T5 = BIAS == BIAS_T5 || BIAS == BIAS_T5U;
    constexpr int kSat = BIAS == BIAS_T5U ? kT5USat : kT5Sat;
    __shared__ float t5r[IS_T5 ? 2 * kSat + 1 : 1];
    static_assert(NW * NW * kRowsF32 <= 2 * KT * D, "merge area");
    float* ks = kvs;
    float* vs = kvs + KT * D;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.z, hq = blockIdx.y, kvh = hq / p.G;
    const int Sq = p.Sq, Sk = p.Sk;
    const int q0 = blockIdx.x * kRowsF32;
    const int i = q0 + lane;
    const bool row_ok = i < Sq;
    const int pos = i + p.off;

    const size_t q_row = (size_t)p.Hq * D, kv_row = (size_t)p.Hkv * D;
    const float* qg = (const float*)p.q + ((size_t)b * Sq * p.Hq + hq) * D;
    const float* kg = (const float*)p.k + ((size_t)b * Sk * p.Hkv + kvh) * D;
    const float* vg = (const float*)p.v + ((size_t)b * Sk * p.Hkv + kvh) * D;

    for (int e = tid; e < kRowsF32 * D; e += NT) {
        const int r = e / D, d = e % D;
        qs[r * QP + d] = (q0 + r < Sq) ? qg[(size_t)(q0 + r) * q_row + d] : 0.f;
    }
    if constexpr (IS_T5) {
        const float* tb = (const float*)p.bias + (size_t)hq * kT5Buckets;
        for (int r = tid; r < 2 * kSat + 1; r += NT)
            t5r[r] = tb[BIAS == BIAS_T5U ? t5u_bucket(r - kSat) : t5_bucket(r - kSat)];
    }
    const float slope = BIAS == BIAS_ALIBI ? ((const float*)p.bias)[hq] : 0.f;
    __syncthreads();
    const float* qrow = qs + lane * QP;
    float q[QREG ? D : 1];
    if constexpr (QREG) {
#pragma unroll
        for (int d = 0; d < D; ++d) q[d] = qrow[d];
    }

    // key range of the 64-row block
    const int pa = q0 + p.off, pb = min(q0 + kRowsF32, Sq) - 1 + p.off;
    int khi = Sk - 1, klo = 0;
    if constexpr (MASK != MASK_NONE) khi = min(khi, pb);
    if constexpr (MASK == MASK_SLIDING) klo = max(0, pa - p.window + 1);

    // this wave's running max, sum and output over its share of the keys
    float o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = 0.f;
    float m = -INFINITY, l = 0.f;
    const int jlo = pos - p.window;     // sliding window: keys after jlo
    const float* brow = nullptr;
    if constexpr (BIAS == BIAS_FULL)
        brow = (const float*)p.bias + (((size_t)b * p.Hq + hq) * Sq + (row_ok ? i : 0)) * (size_t)Sk;

    for (int j0 = (klo / KT) * KT; j0 <= khi; j0 += KT) {
        __syncthreads();
        for (int e = tid; e < KT * D; e += NT) {
            const int j = j0 + e / D;
            ks[e] = (j < Sk) ? kg[(size_t)j * kv_row + e % D] : 0.f;
            vs[e] = (j < Sk) ? vg[(size_t)j * kv_row + e % D] : 0.f;
        }
        __syncthreads();

        // keys wave * KW .. wave * KW + KW - 1 of the tile: Q.K for all of them, eight head-dim
        // columns at a time (each dot product summed in ascending d)
        const float* kw = ks + wave * KW * D;
        const float* vw = vs + wave * KW * D;
        float acc[KW];
#pragma unroll
        for (int jj = 0; jj < KW; ++jj) acc[jj] = 0.f;
#pragma unroll
        for (int c = 0; c < D / 8; ++c) {
            float qc[8];
            if constexpr (QREG) {
#pragma unroll
                for (int t = 0; t < 8; ++t) qc[t] = q[8 * c + t];
            } else {
                const float4 a0 = *(const float4*)(qrow + 8 * c), a1 = *(const float4*)(qrow + 8 * c + 4);
                qc[0] = a0.x; qc[1] = a0.y; qc[2] = a0.z; qc[3] = a0.w;
                qc[4] = a1.x; qc[5] = a1.y; qc[6] = a1.z; qc[7] = a1.w;
            }
#pragma unroll
            for (int jj = 0; jj < KW; ++jj) {
                const float4 k0 = *(const float4*)(kw + jj * D + 8 * c);
                const float4 k1 = *(const float4*)(kw + jj * D + 8 * c + 4);
                float a = acc[jj];
                a = fmaf(qc[0], k0.x, a); a = fmaf(qc[1], k0.y, a);
                a = fmaf(qc[2], k0.z, a); a = fmaf(qc[3], k0.w, a);
                a = fmaf(qc[4], k1.x, a); a = fmaf(qc[5], k1.y, a);
                a = fmaf(qc[6], k1.z, a); a = fmaf(qc[7], k1.w, a);
                acc[jj] = a;
            }
            load_fence();
        }
        float sc[KW];
        float mt = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < KW; ++jj) {
            const int j = j0 + wave * KW + jj;
            float x = acc[jj] * p.scale;
            if constexpr (IS_T5) x += t5r[kSat + min(max(j - pos, -kSat), kSat)];
            if constexpr (BIAS == BIAS_ALIBI) x -= slope * fabsf((float)(j - pos));
            // (keys past the end read the last key's bias and are hidden below)
            if constexpr (BIAS == BIAS_FULL) x += brow[min(j, Sk - 1)];
            bool vis = j < Sk;
            if constexpr (MASK != MASK_NONE) vis = vis && (j <= pos);
            if constexpr (MASK == MASK_SLIDING) vis = vis && (j > jlo);
            sc[jj] = vis ? x : -INFINITY;
            mt = fmaxf(mt, sc[jj]);
        }
        load_fence();
        if (mt > m) {
            // a larger max: rescale what this wave has summed (an unchanged max would scale by
            // exactly 1, so that case skips the multiplications)
            const float alpha = expf(m - mt);
            l *= alpha;
#pragma unroll
            for (int d = 0; d < D; ++d) o[d] *= alpha;
            m = mt;
        }
        if (m != -INFINITY) {
#pragma unroll
            for (int jj = 0; jj < KW; ++jj) {
                const float pj = expf(sc[jj] - m);
                l += pj;
#pragma unroll
                for (int c = 0; c < D / VC; ++c) {
#pragma unroll
                    for (int t = 0; t < VC / 4; ++t) {
                        const float4 v4 = *(const float4*)(vw + jj * D + c * VC + 4 * t);
                        float* oo = o + c * VC + 4 * t;
                        oo[0] = fmaf(pj, v4.x, oo[0]); oo[1] = fmaf(pj, v4.y, oo[1]);
                        oo[2] = fmaf(pj, v4.z, oo[2]); oo[3] = fmaf(pj, v4.w, oo[3]);
                    }
                    load_fence();
                }
            }
        }
    }

    // Merge the waves' partial results of each row in wave order: weights exp(m_w - M) with
    // M the largest m_w; a row that sees no key (every m_w = -inf) gets O = 0, LSE = -inf.
    __syncthreads();
    mls[0][wave][lane] = m;
    mls[1][wave][lane] = l;
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < NW; ++u) M = fmaxf(M, mls[0][u][lane]);
    float a[NW];
    float L = 0.f;
#pragma unroll
    for (int u = 0; u < NW; ++u) {
        a[u] = (M == -INFINITY) ? 0.f : expf(mls[0][u][lane] - M);
        L = fmaf(a[u], mls[1][u][lane], L);
    }
    const float inv = (L > 0.f) ? 1.f / L : 0.f;
    float* og = (float*)p.out + ((size_t)b * Sq + (row_ok ? i : 0)) * q_row + (size_t)hq * D;
#pragma unroll
    for (int c = 0; c < D / NW; ++c) {
        // columns c * NW .. c * NW + NW - 1: every wave stores its partials, wave w sums column
        // c * NW + w over the waves
#pragma unroll
        for (int dd = 0; dd < NW; ++dd) kvs[(wave * NW + dd) * kRowsF32 + lane] = o[c * NW + dd];
        __syncthreads();
        float r = 0.f;
#pragma unroll
        for (int u = 0; u < NW; ++u) r = fmaf(a[u], kvs[(u * NW + wave) * kRowsF32 + lane], r);
        if (row_ok) og[c * NW + wave] = r * inv;
        __syncthreads();
    }
    if (row_ok && wave == 0)
        p.lse[((size_t)b * p.Hq + hq) * Sq + i] = (L > 0.f) ? M + logf(L) : -INFINITY;
}

template <int D, int MASK, int BIAS>
static hipError_t launch_f32_one(const FwdParams& p, hipStream_t s) {
    dim3 grid((p.Sq + kRowsF32 - 1) / kRowsF32, p.Hq, p.B);
    hipLaunchKernelGGL((sdpa_fwd_f32_kernel<D, MASK, BIAS>), grid, dim3(kRowsF32 * waves_f32<D>()), 0, s, p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_f32_d(const FwdParams& p, int mask, int bias, hipStream_t s) {
#define SDPA_CASE(M, Bk) \
    if (mask == M && bias == Bk) return launch_f32_one<D, M, Bk>(p, s);
    SDPA_CASE(MASK_NONE, BIAS_NONE) SDPA_CASE(MASK_NONE, BIAS_T5) SDPA_CASE(MASK_NONE, BIAS_FULL)
    SDPA_CASE(MASK_CAUSAL, BIAS_NONE) SDPA_CASE(MASK_CAUSAL, BIAS_T5) SDPA_CASE(MASK_CAUSAL, BIAS_FULL)
    SDPA_CASE(MASK_SLIDING, BIAS_NONE) SDPA_CASE(MASK_SLIDING, BIAS_T5) SDPA_CASE(MASK_SLIDING, BIAS_FULL)
    SDPA_CASE(MASK_NONE, BIAS_ALIBI) SDPA_CASE(MASK_CAUSAL, BIAS_ALIBI) SDPA_CASE(MASK_SLIDING, BIAS_ALIBI)
    SDPA_CASE(MASK_NONE, BIAS_T5U) SDPA_CASE(MASK_CAUSAL, BIAS_T5U) SDPA_CASE(MASK_SLIDING, BIAS_T5U)
#undef SDPA_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_f32(FwdParams p, int D, int mask, int bias, hipStream_t s) {
    if (D == 32) return launch_f32_d<32>(p, mask, bias, s);
    if (D == 64) return launch_f32_d<64>(p, mask, bias, s);
    if (D == 128) return launch_f32_d<128>(p, mask, bias, s);
    if (D == 256) return launch_f32_d<256>(p, mask, bias, s);
    return hipErrorInvalidValue;
}

}  // namespace sdpa
