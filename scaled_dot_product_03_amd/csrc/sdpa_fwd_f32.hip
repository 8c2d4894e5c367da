// gfx950 fused attention forward, fp32 inputs and fp32 arithmetic (the high-precision path).
//
// Same operation and conventions as the bf16 kernel -- the four attention steps of the
// "jax-gpu-05-attention-gpu" codelab, section 1, with index-generated causal / sliding-window
// masks, T5 or full additive bias and GQA head sharing -- but computed with fp32 FMAs and
// full-precision expf, for workloads stored in fp32 (the codelab's fp32 inputs, section 3).
// It favours exactness over speed: one wave per 64 query rows, one lane per row, keys visited
// in ascending tiles of 32 staged in LDS, online softmax with one rescale per tile.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sdpa_params.h"

namespace sdpa {

constexpr int kRowsF32 = 64;
constexpr int kKeysF32 = 32;

template <int D, int MASK, int BIAS>
__global__ __launch_bounds__(kRowsF32) void sdpa_fwd_f32_kernel(const FwdParams p) {
    __shared__ float qs[kRowsF32][D + 1];
    __shared__ float ks[kKeysF32][D];
    __shared__ float vs[kKeysF32][D];
    __shared__ float tbl[kT5Buckets];

    const int tid = threadIdx.x;
    const int b = blockIdx.z, hq = blockIdx.y, kvh = hq / p.G;
    const int Sq = p.Sq, Sk = p.Sk;
    const int q0 = blockIdx.x * kRowsF32;
    const int i = q0 + tid;
    const bool row_ok = i < Sq;
    const int pos = i + p.off;

    const size_t q_row = (size_t)p.Hq * D, kv_row = (size_t)p.Hkv * D;
    const float* qg = (const float*)p.q + ((size_t)b * Sq * p.Hq + hq) * D;
    const float* kg = (const float*)p.k + ((size_t)b * Sk * p.Hkv + kvh) * D;
    const float* vg = (const float*)p.v + ((size_t)b * Sk * p.Hkv + kvh) * D;

    for (int e = tid; e < kRowsF32 * D; e += kRowsF32) {
        const int r = e / D, d = e % D;
        qs[r][d] = (q0 + r < Sq) ? qg[(size_t)(q0 + r) * q_row + d] : 0.f;
    }
    if constexpr (BIAS == BIAS_T5 || BIAS == BIAS_T5U) {
        if (tid < kT5Buckets) tbl[tid] = ((const float*)p.bias)[(size_t)hq * kT5Buckets + tid];
    }
    const float slope = BIAS == BIAS_ALIBI ? ((const float*)p.bias)[hq] : 0.f;

    // key range of the 64-row block
    const int pa = q0 + p.off, pb = min(q0 + kRowsF32, Sq) - 1 + p.off;
    int khi = Sk - 1, klo = 0;
    if constexpr (MASK != MASK_NONE) khi = min(khi, pb);
    if constexpr (MASK == MASK_SLIDING) klo = max(0, pa - p.window + 1);

    float o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = 0.f;
    float m = -INFINITY, l = 0.f;
    const float* brow = nullptr;
    if constexpr (BIAS == BIAS_FULL)
        brow = (const float*)p.bias + (((size_t)b * p.Hq + hq) * Sq + (row_ok ? i : 0)) * (size_t)Sk;

    for (int j0 = (klo / kKeysF32) * kKeysF32; j0 <= khi; j0 += kKeysF32) {
        __syncthreads();
        for (int e = tid; e < kKeysF32 * D; e += kRowsF32) {
            const int r = e / D, d = e % D;
            const int j = j0 + r;
            ks[r][d] = (j < Sk) ? kg[(size_t)j * kv_row + d] : 0.f;
            vs[r][d] = (j < Sk) ? vg[(size_t)j * kv_row + d] : 0.f;
        }
        __syncthreads();

        float s[kKeysF32];
        float mt = -INFINITY;
#pragma unroll 4
        for (int jj = 0; jj < kKeysF32; ++jj) {
            const int j = j0 + jj;
            float acc = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d) acc = fmaf(qs[tid][d], ks[jj][d], acc);
            float x = acc * p.scale;
            if constexpr (BIAS == BIAS_T5) x += tbl[t5_bucket(j - pos)];
            if constexpr (BIAS == BIAS_T5U) x += tbl[t5u_bucket(j - pos)];
            if constexpr (BIAS == BIAS_ALIBI) x -= slope * fabsf((float)(j - pos));
            if constexpr (BIAS == BIAS_FULL) x += (row_ok && j < Sk) ? brow[j] : 0.f;
            bool vis = j < Sk;
            if constexpr (MASK != MASK_NONE) vis = vis && (j <= pos);
            if constexpr (MASK == MASK_SLIDING) vis = vis && (pos - j < p.window);
            s[jj] = vis ? x : -INFINITY;
            mt = fmaxf(mt, s[jj]);
        }
        const float m_new = fmaxf(m, mt);
        if (m_new != -INFINITY) {
            const float alpha = expf(m - m_new);
            l *= alpha;
#pragma unroll
            for (int d = 0; d < D; ++d) o[d] *= alpha;
            m = m_new;
#pragma unroll 4
            for (int jj = 0; jj < kKeysF32; ++jj) {
                const float pj = expf(s[jj] - m);
                l += pj;
#pragma unroll
                for (int d = 0; d < D; ++d) o[d] = fmaf(pj, vs[jj][d], o[d]);
            }
        }
    }

    if (row_ok) {
        float* og = (float*)p.out + ((size_t)b * Sq + i) * q_row + (size_t)hq * D;
        const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) og[d] = o[d] * inv;
        p.lse[((size_t)b * p.Hq + hq) * Sq + i] = (l > 0.f) ? m + logf(l) : -INFINITY;
    }
}

template <int D, int MASK, int BIAS>
static hipError_t launch_f32_one(const FwdParams& p, hipStream_t s) {
    dim3 grid((p.Sq + kRowsF32 - 1) / kRowsF32, p.Hq, p.B);
    hipLaunchKernelGGL((sdpa_fwd_f32_kernel<D, MASK, BIAS>), grid, dim3(kRowsF32), 0, s, p);
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
