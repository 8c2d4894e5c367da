// gfx950 fused attention forward, bf16 inputs, bf16 MFMA with fp32 accumulation.
//
// Computes O = softmax(Q.K^T * scale + bias + mask) . V and the row log-sum-exp (the four
// steps of the "jax-gpu-05-attention-gpu" codelab, section 1) in one launch without ever
// forming the [Sq, Sk] score matrix (the fused, blockwise evaluation of codelab section 8,
// sequence-length sweep). Masks and the T5 bias are generated from indices in registers
// (codelab section 7; transformers issue "Slowdown in Training Speed Due to SDPA Mask Fix in
// Version 4.40.0"; FAT5 README, T5-like relative position bias), and key tiles that a mask
// hides completely are never visited.
//
// Work decomposition (one workgroup = 4 wave64s = one 128-row query tile of one (batch, head)):
//   * each wave owns 32 query rows; its Q fragment stays in VGPRs for the whole kernel;
//   * keys are visited in tiles of 64, ascending; K (row-major) and V (transposed, [d][key])
//     tiles are staged in a 2-deep LDS ring, the next tile's global loads in flight while the
//     current one is computed;
//   * scores are computed transposed, S^T = K . Q^T, with v_mfma_f32_32x32x16_bf16: each lane
//     then holds one query row (lane % 32) and 32 of the tile's keys, so the row max/sum are
//     in-lane plus one permlane32 exchange with the lane holding the other 32 keys;
//   * O^T += V^T . P^T with the same MFMA; P comes straight from the score registers (bf16,
//     nearest even) as the B operand, so P never leaves the lane;
//   * online softmax in the log2 domain with a lazy rescale: the running reference max only
//     moves (and O is only rescaled) when a row's max grows by more than 2^8.
// Reduction order is fixed (ascending key tiles, fixed MFMA chains, no atomics): results are
// bitwise reproducible run to run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdpa_params.h"

namespace sdpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kBM = 128;        // query rows per workgroup
constexpr int kBN = 64;         // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;   // log2 units: p may reach 2^8 before O is rescaled

// Row permutation inside a 32-row MFMA operand: the A-operand row held by lane r = 8g+4h+t
// is taken from source row 16h+4g+t, so that output register v of a lane in half h holds
// row 16h+v (16 consecutive keys / head dims per lane instead of four runs of four).
__device__ __forceinline__ int perm32(int r) {
    return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3);
}

// LDS bank swizzles (XOR on the 16-byte chunk index within a row).
// K tile [64 keys][D], D=128: rows of 16 chunks; D=64: rows of 8 chunks.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
    if constexpr (D == 128) {
        return (row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3);
    } else {
        return ((row & 3) ^ ((row >> 2) & 1)) | (((row >> 4) & 1) << 2);
    }
}
// V^T tile [D][64 keys]: rows of 8 chunks; conflict-free for both the transposing writes
// (8 lanes on rows 8 apart) and the MFMA reads (8 lanes on rows {0..3, 16..19} + 4g).
__device__ __forceinline__ int v_swz(int d) {
    return (((d & 3) | (((d >> 4) & 1) << 2)) ^ ((d >> 3) & 7) ^ ((d >> 2) & 1)) & 7;
}

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ float partner_max(float x) {
    // value of lane l ^ 32 (the other half of the wave)
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float partner_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

template <int D, int MASK, int BIAS, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 2) void sdpa_fwd_bf16_kernel(const FwdParams p) {
    constexpr int KCH = D / 8;          // 16-byte chunks per K row
    constexpr int KS = D / 16;          // k-steps of Q.K^T
    constexpr int DB = D / 32;          // 32-wide d blocks of O^T
    constexpr int K_TILE = kBN * D;     // bf16 elements per K buffer
    constexpr int V_TILE = D * kBN;     // bf16 elements per V^T buffer
    // Global->LDS staging: K by threads [0, 128) (NK 16-byte chunks each); V by 8x8 blocks,
    // one per thread in [128, 128 + NVB).
    constexpr int K_THREADS = 128;
    constexpr int NK = (kBN * KCH) / K_THREADS;
    constexpr int NVB = (kBN / 8) * (D / 8);
    static_assert(NK * K_THREADS == kBN * KCH, "K staging");
    static_assert(K_THREADS + NVB <= kThreads, "V staging");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (K_TILE + V_TILE)];
    __shared__ float t5s[BIAS == BIAS_T5 ? 2 * kT5Sat + 1 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, r32 = lane & 31;

    const WorkItem w = decode_work(p, blockIdx.x);
    const int b = w.b, hq = w.hq, kvh = hq / p.G;
    const int Sq = p.Sq, Sk = p.Sk, off = p.off;
    const int q0 = w.qt * kBM;

    // ---- key range of the workgroup; tiles outside it are never visited -------------------
    const int pa = q0 + off;
    const int pb = min(q0 + kBM, Sq) - 1 + off;
    int khi = Sk - 1, klo = 0;
    if constexpr (MASK != MASK_NONE) khi = min(khi, pb);
    if constexpr (MASK == MASK_SLIDING) klo = max(0, pa - p.window + 1);
    const int t_begin = klo / kBN;
    const int t_end = (khi < klo) ? t_begin : khi / kBN + 1;

    const size_t q_row = (size_t)p.Hq * D;
    const size_t kv_row = (size_t)p.Hkv * D;
    const uint16_t* qg = (const uint16_t*)p.q + ((size_t)b * Sq * p.Hq + hq) * D;
    const uint16_t* kg = (const uint16_t*)p.k + ((size_t)b * Sk * p.Hkv + kvh) * D;
    const uint16_t* vg = (const uint16_t*)p.v + ((size_t)b * Sk * p.Hkv + kvh) * D;

    const int wq0 = q0 + wave * 32;          // first query row of this wave
    const int my_i = wq0 + r32;              // query row of this lane
    const bool row_ok = my_i < Sq;
    const int my_pos = my_i + off;
    const bool wave_ok = wq0 < Sq;
    const int pwa = wq0 + off;
    const int pwb = min(wq0 + 31, Sq - 1) + off;

    // ---- output helpers --------------------------------------------------------------------
    float* lse_row = p.lse + ((size_t)b * p.Hq + hq) * Sq;
    auto out_ptr = [&](int i) -> char* {
        const size_t e = ((size_t)b * Sq + i) * q_row + (size_t)hq * D;
        return (char*)p.out + e * (OUT_F32 ? 4 : 2);
    };

    if (t_end == t_begin) {   // every row of the tile sees no key: O = 0, LSE = -inf
        if (row_ok) {
            char* o = out_ptr(my_i);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d0 = db * 32 + hh * 16;
                if constexpr (OUT_F32) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) *(u32x4*)(o + (d0 + 4 * c) * 4) = u32x4{0, 0, 0, 0};
                } else {
#pragma unroll
                    for (int c = 0; c < 2; ++c) *(u32x4*)(o + (d0 + 8 * c) * 2) = u32x4{0, 0, 0, 0};
                }
            }
            if (hh == 0) lse_row[my_i] = -INFINITY;
        }
        return;
    }

    // ---- T5: expanded bias by relative position, already in log2 units --------------------
    if constexpr (BIAS == BIAS_T5) {
        const float* tbl = (const float*)p.bias + (size_t)hq * kT5Buckets;
        if (tid < 2 * kT5Sat + 1) t5s[tid] = tbl[t5_bucket(tid - kT5Sat)] * kLog2e;
    }

    // ---- Q fragment: lane holds row my_i, dims 16ks + 8hh .. +7 ----------------------------
    bf16x8 qf[KS];
    {
        const uint16_t* qr = qg + (size_t)my_i * q_row + hh * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = row_ok ? *(const u32x4*)(qr + ks * 16) : u32x4{0, 0, 0, 0};
            qf[ks] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // ---- global -> register staging of one K/V tile ----------------------------------------
    u32x4 stage[8];
    const bool is_k_thread = tid < K_THREADS;
    const bool is_v_thread = !is_k_thread && (tid - K_THREADS) < NVB;
    // V block of this thread: key rows 8*vjo .. +7, dims 8*vdc .. +7
    const int vu = tid - K_THREADS;
    const int vdc = vu % (D / 8), vjo = vu / (D / 8);

    auto load_tile = [&](int t) {
        const int j0 = t * kBN;
        if (is_k_thread) {
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                const int cid = tid + i * K_THREADS;
                const int row = cid / KCH, c = cid % KCH;
                const int j = j0 + row;
                stage[i] = (j < Sk) ? *(const u32x4*)(kg + (size_t)j * kv_row + c * 8)
                                    : u32x4{0, 0, 0, 0};
            }
        } else if (is_v_thread) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int j = j0 + vjo * 8 + i;
                stage[i] = (j < Sk) ? *(const u32x4*)(vg + (size_t)j * kv_row + vdc * 8)
                                    : u32x4{0, 0, 0, 0};
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* kb = smem + buf * (K_TILE + V_TILE);
        uint16_t* vb = kb + K_TILE;
        if (is_k_thread) {
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                const int cid = tid + i * K_THREADS;
                const int row = cid / KCH, c = cid % KCH;
                *(u32x4*)(kb + row * D + ((c ^ k_swz<D>(row)) * 8)) = stage[i];
            }
        } else if (is_v_thread) {
            // transpose the 8x8 block: output row d = 8*vdc + e holds keys 8*vjo .. +7
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                u32x4 o;
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    o[m] = perm_b32(stage[2 * m + 1][e >> 1], stage[2 * m][e >> 1], sel);
                const int d = vdc * 8 + e;
                *(u32x4*)(vb + d * kBN + ((vjo ^ v_swz(d)) * 8)) = o;
            }
        }
    };

    // ---- per-lane LDS read offsets (in bf16 elements) --------------------------------------
    // K: A operand row (lane % 32) -> key perm32(r32) (+32 for the second key block).
    const int krow = perm32(r32);
    const int k_sw = k_swz<D>(krow);          // identical for krow + 32
    // V^T: A operand row -> head dim 32*db + perm32(r32).
    const int vrow = perm32(r32);

    f32x16 o_acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o_acc[db][v] = 0.f;
    float m_ref = -INFINITY;     // reference max (log2 units) of this lane's row
    float l_part = 0.f;          // sum of p over this lane's keys, relative to m_ref

    const float c_scale = p.scale_log2;

    load_tile(t_begin);
    store_tile(0);
    __syncthreads();

    for (int t = t_begin; t < t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        const bool has_next = t + 1 < t_end;
        if (has_next) load_tile(t + 1);

        const int j0 = t * kBN;
        // wave-level classification of this tile
        bool skip = !wave_ok;
        if constexpr (MASK != MASK_NONE) skip = skip || (j0 > pwb);
        if constexpr (MASK == MASK_SLIDING) skip = skip || (j0 + kBN - 1 <= pwa - p.window);

        if (!skip) {
            const uint16_t* kb = smem + buf * (K_TILE + V_TILE);
            const uint16_t* vb = kb + K_TILE;

            // ---- S^T = K . Q^T (two 32-key blocks) ----
            f32x16 s0, s1;
#pragma unroll
            for (int v = 0; v < 16; ++v) { s0[v] = 0.f; s1[v] = 0.f; }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int ch = ((2 * ks + hh) ^ k_sw) * 8;
                const bf16x8 a0 = *(const bf16x8*)(kb + krow * D + ch);
                const bf16x8 a1 = *(const bf16x8*)(kb + (krow + 32) * D + ch);
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], s1, 0, 0, 0);
            }

            // ---- scores in log2 units, bias, mask.  x[16*jb + v] is key j0 + 32jb + 16hh + v
            float x[32];
#pragma unroll
            for (int v = 0; v < 16; ++v) { x[v] = s0[v]; x[16 + v] = s1[v]; }

            const int jl = j0 + 16 * hh;   // key of x[0] in this lane
            if constexpr (BIAS == BIAS_T5) {
                const int rmin = j0 - pwb, rmax = j0 + kBN - 1 - pwa;
                if (rmin >= kT5Sat || rmax <= -kT5Sat) {
                    const float bc = t5s[rmin >= kT5Sat ? 2 * kT5Sat : 0];
#pragma unroll
                    for (int e = 0; e < 32; ++e) x[e] = fmaf(x[e], c_scale, bc);
                } else {
                    const int rel0 = jl - my_pos;
#pragma unroll
                    for (int e = 0; e < 32; ++e) {
                        const int rel = rel0 + (e >> 4) * 32 + (e & 15);
                        const int idx = min(max(rel, -kT5Sat), kT5Sat) + kT5Sat;
                        x[e] = fmaf(x[e], c_scale, t5s[idx]);
                    }
                }
            } else if constexpr (BIAS == BIAS_FULL) {
                const uint16_t* br = (const uint16_t*)p.bias +
                                     (((size_t)b * p.Hq + hq) * Sq + (row_ok ? my_i : 0)) * (size_t)Sk;
                const bool vec_ok = row_ok && (j0 + kBN <= Sk) && ((Sk & 7) == 0);
                if (vec_ok) {
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) {
                        const u32x4 lo = *(const u32x4*)(br + jl + 32 * jb);
                        const u32x4 hi = *(const u32x4*)(br + jl + 32 * jb + 8);
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            x[16 * jb + 2 * c] = fmaf(x[16 * jb + 2 * c], c_scale, bf16_to_f32(lo[c] & 0xffffu) * kLog2e);
                            x[16 * jb + 2 * c + 1] = fmaf(x[16 * jb + 2 * c + 1], c_scale, bf16_to_f32(lo[c] >> 16) * kLog2e);
                            x[16 * jb + 8 + 2 * c] = fmaf(x[16 * jb + 8 + 2 * c], c_scale, bf16_to_f32(hi[c] & 0xffffu) * kLog2e);
                            x[16 * jb + 9 + 2 * c] = fmaf(x[16 * jb + 9 + 2 * c], c_scale, bf16_to_f32(hi[c] >> 16) * kLog2e);
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 32; ++e) {
                        const int j = jl + (e >> 4) * 32 + (e & 15);
                        const float bv = (row_ok && j < Sk) ? bf16_to_f32(br[j]) : 0.f;
                        x[e] = fmaf(x[e], c_scale, bv * kLog2e);
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 32; ++e) x[e] = x[e] * c_scale;
            }

            bool need_mask = (j0 + kBN > Sk);
            if constexpr (MASK != MASK_NONE) need_mask = need_mask || (j0 + kBN - 1 > pwa);
            if constexpr (MASK == MASK_SLIDING) need_mask = need_mask || (j0 <= pwb - p.window);
            if (need_mask) {
#pragma unroll
                for (int e = 0; e < 32; ++e) {
                    const int j = jl + (e >> 4) * 32 + (e & 15);
                    bool vis = j < Sk;
                    if constexpr (MASK != MASK_NONE) vis = vis && (j <= my_pos);
                    if constexpr (MASK == MASK_SLIDING) vis = vis && (my_pos - j < p.window);
                    x[e] = vis ? x[e] : -INFINITY;
                }
            }

            // ---- online softmax (log2 domain, lazy rescale) ----
            float mt = x[0];
#pragma unroll
            for (int e = 1; e < 32; ++e) mt = fmaxf(mt, x[e]);
            mt = partner_max(mt);
            if (__builtin_amdgcn_ballot_w64(mt > m_ref + kRescaleSlack) != 0) {
                const float m_new = fmaxf(m_ref, mt);
                const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
                m_ref = m_new;
                l_part *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v) o_acc[db][v] *= alpha;
            }
            const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                x[e] = __builtin_amdgcn_exp2f(x[e] - m_use);
                psum += x[e];
            }
            l_part += psum;

            // ---- O^T += V^T . P^T ----
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    u32x4 pk;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        pk[c] = pack_bf16x2(x[16 * jb + 8 * s + 2 * c], x[16 * jb + 8 * s + 2 * c + 1]);
                    const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
                    const int vch = 4 * jb + 2 * hh + s;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const int d = 32 * db + vrow;
                        const bf16x8 a = *(const bf16x8*)(vb + d * kBN + ((vch ^ v_swz(d)) * 8));
                        o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o_acc[db], 0, 0, 0);
                    }
                }
            }
        }

        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l) ---------------------------------
    const float l_tot = partner_sum(l_part);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (row_ok) {
        char* o = out_ptr(my_i);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d0 = db * 32 + hh * 16;
            if constexpr (OUT_F32) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    u32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = __float_as_uint(o_acc[db][4 * c + e] * inv);
                    *(u32x4*)(o + (d0 + 4 * c) * 4) = x;
                }
            } else {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    u32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        x[e] = pack_bf16x2(o_acc[db][8 * c + 2 * e] * inv, o_acc[db][8 * c + 2 * e + 1] * inv);
                    *(u32x4*)(o + (d0 + 8 * c) * 2) = x;
                }
            }
        }
        if (hh == 0)
            lse_row[my_i] = (l_tot > 0.f) ? (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    }
}

// ------------------------------------------------------------------------------------------
// host-side launch (called by the C ABI after validation)
// ------------------------------------------------------------------------------------------
template <int D, int MASK, int BIAS, bool OUT_F32>
static hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
    const unsigned grid = (unsigned)((size_t)p.B * p.Hq * p.n_qt);
    hipLaunchKernelGGL((sdpa_fwd_bf16_kernel<D, MASK, BIAS, OUT_F32>), dim3(grid), dim3(kThreads),
                       0, stream, p);
    return hipGetLastError();
}

template <int D, bool OUT_F32>
static hipError_t launch_d(const FwdParams& p, int mask, int bias, hipStream_t s) {
#define SDPA_CASE(M, Bk) \
    if (mask == M && bias == Bk) return launch_one<D, M, Bk, OUT_F32>(p, s);
    SDPA_CASE(MASK_NONE, BIAS_NONE) SDPA_CASE(MASK_NONE, BIAS_T5) SDPA_CASE(MASK_NONE, BIAS_FULL)
    SDPA_CASE(MASK_CAUSAL, BIAS_NONE) SDPA_CASE(MASK_CAUSAL, BIAS_T5) SDPA_CASE(MASK_CAUSAL, BIAS_FULL)
    SDPA_CASE(MASK_SLIDING, BIAS_NONE) SDPA_CASE(MASK_SLIDING, BIAS_T5) SDPA_CASE(MASK_SLIDING, BIAS_FULL)
#undef SDPA_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16(FwdParams p, int D, int mask, int bias, bool out_f32, hipStream_t s) {
    p.n_qt = (p.Sq + kBM - 1) / kBM;
    p.xcd_remap = ((p.B * p.Hkv) % 8 == 0) ? 1 : 0;
    if (D == 128) return out_f32 ? launch_d<128, true>(p, mask, bias, s) : launch_d<128, false>(p, mask, bias, s);
    if (D == 64) return out_f32 ? launch_d<64, true>(p, mask, bias, s) : launch_d<64, false>(p, mask, bias, s);
    return hipErrorInvalidValue;
}

}  // namespace sdpa
