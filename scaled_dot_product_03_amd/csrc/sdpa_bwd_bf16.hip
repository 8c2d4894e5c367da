// gfx950 attention backward: gradients dQ, dK, dV of L = sum(dO * O) for the fused forward
// O = softmax(Q.K^T * scale + bias + mask) . V (the four steps of the "jax-gpu-05-attention-gpu"
// codelab, section 1; masks of its section 7 and of the transformers issue "Slowdown in
// Training Speed Due to SDPA Mask Fix in Version 4.40.0"; biases of the FAT5 README; head
// sharing of codelab section 9). With P the softmax weights (recomputed from the forward's
// row log-sum-exp) and D_i = rowsum(dO_i * O_i):
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
// Two launches, each output element written once, fixed summation order, no atomics, so the
// gradients are bitwise reproducible run to run (the determinism asked of a training step in
// the transformers issue "Transformer models are not deterministic when using Flash Attention 2").
//
//   dq_kernel    : one workgroup = 8 waves = 256 query rows of one (batch, query head), like the
//                  forward. It first forms D_i = rowsum(dO_i * O_i) for its rows and stores it
//                  in the caller's workspace for the second launch. Q and dO fragments stay in
//                  VGPRs, K and V tiles of 64 keys stream
//                  through 2-slot LDS rings (LDS DMA). Per 32-key half: S^T = K.Q^T and
//                  dP^T = V.dO^T (lane = query row, 16 keys per lane half), P and dS^T in
//                  registers, then dQ^T += K^T.dS^T with K^T from transposing LDS reads.
//   dkdv_lag_kernel : one workgroup = 8 waves = 128 keys of one (batch, KV head) (D = 256: 4
//                  waves, 64 keys). The waves come in two roles over the same 32-key blocks: a
//                  dV wave keeps its keys' K fragments in VGPRs and accumulates dV^T; a dK
//                  wave keeps V fragments and accumulates dK^T. Q and dO tiles stream through
//                  a 3-slot LDS ring over the rows of the G query heads sharing the KV head
//                  (heads ascending, rows ascending). Per 32-row block (lane = key, 16 rows per
//                  lane half): the dV wave forms S = Q.K^T and P, then dV^T += dO^T.P with
//                  dO^T from transposing reads, and leaves P in LDS; the dK wave, one step
//                  behind, forms dP = dO.V^T and dS = P (dP - D) with that P, then
//                  dK^T += Q^T.dS with Q^T from transposing reads.
//   dkdv_kernel  : a full bias at D = 32, 128 and 256, where a bias tile per slot does not
//                  fit beside the 3-slot ring and the P buffers: the same roles over a 2-slot
//                  ring with the bias tile in LDS, the dK wave forming S itself.
// MFMA: v_mfma_f32_32x32x16_bf16 throughout; P and dS are rounded to bf16 (nearest even) as
// MFMA operands, all sums are fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sdpa_device.h"
#include "sdpa_params.h"

namespace sdpa {
namespace bwd {

using namespace dev;

// ------------------------------------------------------------------------------------------
// dQ: 256 query rows per workgroup, 64-key tiles
// ------------------------------------------------------------------------------------------
// waves per workgroup: 8 (two per SIMD); at D = 256 a wave needs the whole register file, so 4
template <int D> constexpr int bwd_waves() { return D == 256 ? 4 : 8; }

template <int D, int MASK, int BIAS, bool OUT_F32>
__global__ __launch_bounds__(64 * bwd_waves<D>(), 1) void dq_kernel(const BwdParams p) {
    constexpr int kWaves = bwd_waves<D>(), kThreads = 64 * kWaves, kBM = 32 * kWaves, kBN = 64;
    constexpr int CH = D / 8, KS = D / 16, DB = D / 32, TILE = kBN * D;
    constexpr bool FB = BIAS == BIAS_FULL;
    constexpr bool IS_T5 = BIAS == BIAS_T5 || BIAS == BIAS_T5U;
    constexpr bool ALIBI = BIAS == BIAS_ALIBI;
    constexpr int kSat = BIAS == BIAS_T5U ? kT5USat : kT5Sat;
    constexpr int kT5Pad = kSat + kBN + 31;
    // full-bias tile: kBM rows x 64 keys through LDS (at D = 256 the K/V slots fill the LDS: the
    // bias is read from HBM by each lane)
    constexpr bool FB_LDS = FB && D != 256;
    constexpr int BTILE = FB_LDS ? kBM * kBN : 0;
    // K slots 0-1, V slots 2-3, then (full bias) two bias slots
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * TILE + 2 * BTILE];
    __shared__ float t5s[IS_T5 ? 2 * kT5Pad + 1 : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, r32 = lane & 31;
    const WorkItem w = decode_work(p, blockIdx.x);
    const int b = w.b, hq = w.hq, kvh = hq / p.G;
    const int Sq = p.Sq, Sk = p.Sk, off = p.off;
    const int q0 = w.qt * kBM;

    const int pa = q0 + off, pb = min(q0 + kBM, Sq) - 1 + off;
    int khi = Sk - 1, klo = 0;
    if constexpr (MASK != MASK_NONE) khi = min(khi, pb);
    if constexpr (MASK == MASK_SLIDING) klo = max(0, pa - p.window + 1);
    const int t_begin = klo / kBN;
    const int t_end = (khi < klo) ? t_begin : khi / kBN + 1;

    const size_t q_row = (size_t)p.Hq * D, kv_row = (size_t)p.Hkv * D;
    const uint16_t* qg = (const uint16_t*)p.q + ((size_t)b * Sq * p.Hq + hq) * D;
    const uint16_t* dog = (const uint16_t*)p.dout + ((size_t)b * Sq * p.Hq + hq) * D;
    const uint16_t* kg = (const uint16_t*)p.k + ((size_t)b * Sk * p.Hkv + kvh) * D;
    const uint16_t* vg = (const uint16_t*)p.v + ((size_t)b * Sk * p.Hkv + kvh) * D;

    const int wq0 = q0 + wave * 32, my_i = wq0 + r32;
    const bool row_ok = my_i < Sq, wave_ok = wq0 < Sq;
    const int my_pos = my_i + off;
    const int pwa = wq0 + off, pwb = min(wq0 + 31, Sq - 1) + off;
    char* dq_row = (char*)p.dq + (((size_t)b * Sq + (row_ok ? my_i : 0)) * q_row + (size_t)hq * D) * (OUT_F32 ? 4 : 2);

    // dO fragment of this lane's row (dims 16 ks + 8 hh .. + 7, the B operand of dP^T) and the
    // row constant D_i = rowsum(dO_i * O_i): each lane half sums its 64 (or 32) dims in
    // ascending order, then the halves are added. Written to the workspace for the dK/dV
    // kernel, which runs after this one on the same stream.
    const size_t ro = (size_t)(row_ok ? my_i : 0) * q_row + hh * 8;
    bf16x8 dof[KS];
    float drow;
    {
        const uint16_t* og = (const uint16_t*)p.o + ((size_t)b * Sq * p.Hq + hq) * D;
        float part = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 y = *(const u32x4*)(dog + ro + ks * 16);
            u32x4 o = *(const u32x4*)(og + ro + ks * 16);
            if (!row_ok) { y = u32x4{0, 0, 0, 0}; o = u32x4{0, 0, 0, 0}; }
            dof[ks] = __builtin_bit_cast(bf16x8, y);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                part = fmaf(bf16_to_f32(y[e] & 0xffffu), bf16_to_f32(o[e] & 0xffffu), part);
                part = fmaf(bf16_to_f32(y[e] >> 16), bf16_to_f32(o[e] >> 16), part);
            }
        }
        drow = partner_sum(part);
        if (row_ok && hh == 0) p.delta[((size_t)b * p.Hq + hq) * Sq + my_i] = drow;
    }

    if (t_end == t_begin) {   // no row of the tile sees a key: dQ = 0
        if (row_ok) store_zero_row<D, OUT_F32>(dq_row, hh);
        return;
    }
    if constexpr (IS_T5) {
        const float* tbl = (const float*)p.bias + (size_t)hq * kT5Buckets;
        for (int i = tid; i < 2 * kT5Pad + 1; i += kThreads)
            t5s[i] = tbl[BIAS == BIAS_T5U ? t5u_bucket(i - kT5Pad) : t5_bucket(i - kT5Pad)] * kLog2e;
    }
    const float aslope = ALIBI ? ((const float*)p.bias)[hq] * kLog2e : 0.f;   // ALiBi, log2 units

    // A negative scale flips the sign of the Q fragment (S is unchanged); dQ = scale * dS K
    // uses the signed scale. A zero scale computes P with the smallest normal float.
    const bool neg = p.scale_log2 < 0.f;
    const float c_scale = neg ? -p.scale_log2 : (p.scale_log2 == 0.f ? kTinyScale : p.scale_log2);
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = *(const u32x4*)(qg + ro + ks * 16);
        if (!row_ok) x = u32x4{0, 0, 0, 0};
        if (neg) x ^= 0x80008000u;
        qf[ks] = __builtin_bit_cast(bf16x8, x);
    }
    // log-sum-exp of the row in log2 units (+inf for a row with no visible key, so that its
    // P is 0)
    float lse2 = INFINITY;
    if (row_ok) {
        const float l = p.lse[((size_t)b * p.Hq + hq) * Sq + my_i];
        lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
    }

    // K and V tiles: 64 keys x D, row-major, swizzled chunks; 2 slots each. The 1 KB transfers
    // of a tile are spread over the waves (at D = 32 a tile is 4 transfers: waves 0-3 issue).
    constexpr int ROWS_PER_XFER = 1024 / (D * 2), XFERS = (kBN * D * 2) / 1024;
    constexpr int XPW = XFERS >= kWaves ? XFERS / kWaves : 1, NXW = XFERS / XPW;
    static_assert(XPW * NXW == XFERS && NXW <= kWaves, "dma split");
    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)smem);
    // A full bias goes through LDS when its rows split into whole 16-byte chunks: tile
    // [256 rows][64 keys], 128-byte rows, chunk swizzle (row >> 1) & 7; keys past the end of a
    // partial last tile re-read the last whole chunk (they are masked).
    const bool fb_dma = FB_LDS && ((Sk & 7) == 0);
    constexpr int XPB = FB_LDS ? (BTILE * 2 / 1024) / kWaves : 0;
    const uint16_t* fbg = FB ? (const uint16_t*)p.bias + ((size_t)b * p.Hq + hq) * (size_t)Sq * Sk
                             : nullptr;
    auto dma_tile = [&](int t) {
        const int sl = (t - t_begin) & 1, j0 = t * kBN;
        if (NXW == kWaves || wave < NXW) {
#pragma unroll
            for (int n = 0; n < XPW; ++n) {
                const int xi = wave * XPW + n;
                const int row = xi * ROWS_PER_XFER + lane / CH;
                const int j = min(j0 + row, Sk - 1);
                const int ch = ((lane % CH) ^ swz<D>(row)) * 8;
                dma16(kg + (size_t)j * kv_row + ch, lds_base + (uint32_t)((sl * TILE) * 2 + xi * 1024));
                dma16(vg + (size_t)j * kv_row + ch, lds_base + (uint32_t)(((2 + sl) * TILE) * 2 + xi * 1024));
            }
        }
        if constexpr (FB_LDS) {
            if (fb_dma) {
                const int nchunk = min(kBN, Sk - j0) / 8;
#pragma unroll
                for (int n = 0; n < XPB; ++n) {
                    const int xi = wave * XPB + n;
                    const int row = xi * 8 + (lane >> 3);
                    const int c = min((lane & 7) ^ ((row >> 1) & 7), nchunk - 1);
                    dma16(fbg + (size_t)min(q0 + row, Sq - 1) * Sk + j0 + 8 * c,
                          lds_base + (uint32_t)((4 * TILE + sl * BTILE) * 2 + xi * 1024));
                }
            }
        }
    };

    f32x16 dq_acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) dq_acc[db][v] = 0.f;

    auto active = [&](int t) {
        const int j0 = t * kBN;
        bool skip = !wave_ok;
        if constexpr (MASK != MASK_NONE) skip = skip || (j0 > pwb);
        if constexpr (MASK == MASK_SLIDING) skip = skip || (j0 + kBN - 1 <= pwa - p.window);
        return !skip;
    };
    auto needs_mask = [&](int t) {
        const int j0 = t * kBN;
        bool m = (j0 + kBN > Sk);
        if constexpr (MASK != MASK_NONE) m = m || (j0 + kBN - 1 > pwa);
        if constexpr (MASK == MASK_SLIDING) m = m || (j0 <= pwb - p.window);
        return m;
    };

    auto compute_tile = [&](int t) {
        const int sl = (t - t_begin) & 1, j0 = t * kBN;
        const uint16_t* kb = smem + sl * TILE;
        const uint16_t* vb = smem + (2 + sl) * TILE;
        const bool msk = uniform(needs_mask(t));
        // bias of the tile: constant for T5 far from the diagonal
        bool per_elem = FB;
        float bconst = 0.f;
        if constexpr (IS_T5) {
            const int rmin = j0 - pwb, rmax = j0 + kBN - 1 - pwa;
            const int side = uniform(rmin >= kSat ? 1 : (rmax <= -kSat ? -1 : 0));
            if (side > 0) bconst = t5s[2 * kT5Pad];
            else if (side < 0) bconst = t5s[0];
            else per_elem = true;
        }
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int jl = j0 + 32 * jb + 16 * hh;     // key of register 0 of this lane
            f32x16 s, dp;
#pragma unroll
            for (int v = 0; v < 16; ++v) { s[v] = 0.f; dp[v] = 0.f; }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 ak = read_rows<D>(kb, jb, ks, lane);
                const bf16x8 av = read_rows<D>(vb, jb, ks, lane);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[ks], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, dof[ks], dp, 0, 0, 0);
            }
            // x = scores in log2 units including the bias
            float x[16];
            if constexpr (ALIBI) {
                const float base = (float)(jl - my_pos);
#pragma unroll
                for (int v = 0; v < 16; ++v) x[v] = fmaf(s[v], c_scale, -aslope * fabsf(base + (float)v));
            } else if constexpr (IS_T5) {
                if (per_elem) {
                    const float* trow = t5s + kT5Pad + (jl - min(my_pos, pwb));
#pragma unroll
                    for (int v = 0; v < 16; ++v) x[v] = fmaf(s[v], c_scale, trow[v]);
                } else {
#pragma unroll
                    for (int v = 0; v < 16; ++v) x[v] = fmaf(s[v], c_scale, bconst);
                }
            } else if constexpr (FB) {
                if (FB_LDS && fb_dma) {
                    // 16 keys from two chunks of this lane's bias row in LDS
                    const int lr = wave * 32 + r32, c0 = 4 * jb + 2 * hh, sw = (lr >> 1) & 7;
                    const uint16_t* brow = smem + 4 * TILE + sl * BTILE + lr * kBN;
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const u32x4 w = *(const u32x4*)(brow + (((c0 + h2) ^ sw) << 3));
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int v = 8 * h2 + 2 * e;
                            x[v] = fmaf(__uint_as_float(w[e] << 16), kLog2e, s[v] * c_scale);
                            x[v + 1] = fmaf(__uint_as_float(w[e] & 0xffff0000u), kLog2e, s[v + 1] * c_scale);
                        }
                    }
                } else {
                    const uint16_t* br = fbg + (size_t)(row_ok ? my_i : 0) * Sk;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int j = jl + v;
                        const float bv = (row_ok && j < Sk) ? bf16_to_f32(br[j]) : 0.f;
                        x[v] = fmaf(bv, kLog2e, s[v] * c_scale);
                    }
                }
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) x[v] = s[v] * c_scale;
            }
            if (msk) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int j = jl + v;
                    bool vis = j < Sk;
                    if constexpr (MASK != MASK_NONE) vis = vis & (j <= my_pos);
                    if constexpr (MASK == MASK_SLIDING) vis = vis & (my_pos - j < p.window);
                    x[v] = vis ? x[v] : -INFINITY;
                }
            }
            // P from the row's log-sum-exp, then dS^T
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float pv = __builtin_amdgcn_exp2f(x[v] - lse2);
                s[v] = pv * (dp[v] - drow);
            }
            // dQ^T += K^T dS^T over the two 16-key groups of this half
#pragma unroll
            for (int sg = 0; sg < 2; ++sg) {
                u32x4 pk;
#pragma unroll
                for (int c = 0; c < 4; ++c) pk[c] = pack_bf16x2(s[8 * sg + 2 * c], s[8 * sg + 2 * c + 1]);
                bf16x8 kt[DB];
                read_tr<D>(kb, 2 * jb + sg, lane, kt);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    dq_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[db], __builtin_bit_cast(bf16x8, pk), dq_acc[db], 0, 0, 0);
            }
        }
    };

    dma_tile(t_begin);
    dma_wait();
    __syncthreads();
#pragma unroll 1
    for (int t = t_begin; t < t_end; ++t) {
        const bool has_next = t + 1 < t_end;
        if (has_next) dma_tile(t + 1);
        if (uniform(active(t))) compute_tile(t);
        if (has_next) dma_wait();
        __syncthreads();
    }
    if (row_ok) store_row<D, OUT_F32>(dq_row, dq_acc, p.scale, hh);
}

// ------------------------------------------------------------------------------------------
// dK, dV with a full bias at D = 32, 128 and 256: 128 keys of one (batch, KV head) per
// workgroup (64 at D = 256), query rows in steps of 128 (64 at D = 128 and 256). The first half
// of the waves accumulate dV and the second half dK for the same 32-key groups, so each wave
// holds one 32 x D accumulator. Both roles form S = Q.K^T with the same instructions (so their
// P agree bit for bit); the dK waves also form dP = dO.V^T. The bias tile shares the 2-slot
// ring's LDS; dkdv_lag_kernel below has no room for it at these head dims (reading the bias
// per lane from HBM there instead made the call 2.7x to 4.5x slower).
// ------------------------------------------------------------------------------------------
template <int D, int MASK, int BIAS, bool OUT_F32>
__global__ __launch_bounds__(64 * bwd_waves<D>(), 1) void dkdv_kernel(const BwdParams p) {
    static_assert(BIAS == BIAS_FULL && D != 64, "full bias at D = 32, 128, 256 only");
    // keys per workgroup: 32 per dV / dK wave pair; query rows per step: 128 (64 at D = 128 and
    // 256, whose tiles share the LDS with the bias tiles)
    constexpr int kWaves = bwd_waves<D>(), kBK = 32 * (kWaves / 2);
    constexpr int kBQ = (D == 128 || D == 256) ? 64 : 128;
    constexpr bool FB_LDS = D != 256;      // D = 256: each lane reads its bias from HBM
    constexpr int NB = kBQ / 32;
    constexpr int CH = D / 8, KS = D / 16, DB = D / 32, QT = kBQ * D, BTILE = FB_LDS ? kBQ * kBK : 0;
    // LDS: slot sl holds the Q tile at [2 sl] and the dO tile at [2 sl + 1] (kBQ rows each),
    // then two bias slots of kBQ rows x 128 keys
    __shared__ __attribute__((aligned(16))) uint16_t smem[4 * QT + 2 * BTILE];
    __shared__ __attribute__((aligned(16))) float rowc[2][2][kBQ];    // [slot][lse2, D][row]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, r32 = lane & 31;
    const bool role_dk = uniform(wave >= kWaves / 2);
    // workgroup -> (batch, KV head, key tile); with xcd_remap all key tiles of one (batch,
    // KV head) run on one XCD (workgroup x is dispatched to XCD x % 8), where they share the
    // Q / dO rows in that XCD's L2
    int group, kt_idx;
    {
        const int x = blockIdx.x;
        if (p.xcd_remap) {
            const int slot = x >> 3, gl = slot / p.n_kt;
            kt_idx = slot - gl * p.n_kt;
            group = gl * 8 + (x & 7);
        } else {
            group = x / p.n_kt;
            kt_idx = x - group * p.n_kt;
        }
    }
    const int b = group / p.Hkv, kvh = group - b * p.Hkv;
    const int Sq = p.Sq, Sk = p.Sk, off = p.off, G = p.G;
    const int k0 = kt_idx * kBK;
    const int kw0 = k0 + 32 * (wave % (kWaves / 2));   // first key of this wave
    const int my_j = kw0 + r32;                // key of this lane
    const bool key_ok = my_j < Sk;
    const bool wave_ok = kw0 < Sk;
    const int kwe = min(kw0 + 31, Sk - 1);     // last valid key of the wave

    const size_t q_row = (size_t)p.Hq * D, kv_row = (size_t)p.Hkv * D;
    const size_t kv_off = ((size_t)b * Sk + (key_ok ? my_j : 0)) * kv_row + (size_t)kvh * D;
    char* out_row = (char*)(role_dk ? p.dk : p.dv) + kv_off * (OUT_F32 ? 4 : 2);

    // query rows the workgroup's keys can see (positions of the rows: i + off)
    const int kend = min(k0 + kBK, Sk) - 1;
    int qlo = 0, qhi = Sq;
    if constexpr (MASK != MASK_NONE) qlo = max(0, k0 - off);
    if constexpr (MASK == MASK_SLIDING) qhi = min(Sq, kend + p.window - off);
    const int s_begin = qlo / kBQ;
    const int s_end = (qhi <= qlo) ? s_begin : (qhi + kBQ - 1) / kBQ;
    const int nqs = s_end - s_begin;
    const int n_steps = G * nqs;

    if (n_steps == 0) {        // no query row sees these keys: dK = dV = 0
        if (key_ok) store_zero_row<D, OUT_F32>(out_row, hh);
        return;
    }
    const bool neg = p.scale_log2 < 0.f;
    const float c_scale = neg ? -p.scale_log2 : (p.scale_log2 == 0.f ? kTinyScale : p.scale_log2);

    // Q / dO tiles of step n: head h = kvh * G + n / nqs, rows kBQ s .. + kBQ - 1 (clamped)
    constexpr int ROWS_PER_XFER = 1024 / (D * 2), XFERS = (kBQ * D * 2) / 1024, XPW = XFERS / kWaves;
    static_assert(XPW * kWaves == XFERS, "dma split");
    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)smem);
    // A full bias goes through LDS when its rows split into whole 16-byte chunks: tile
    // [kBQ rows][128 keys], 256-byte rows, chunk swizzle 4 * ((row >> 4) & 1); keys past the end
    // of a partial last tile re-read the last whole chunk (they are masked).
    const bool fb_dma = FB_LDS && ((Sk & 7) == 0);
    constexpr int XPB = FB_LDS ? (BTILE * 2 / 1024) / kWaves : 0;
    auto issue_step = [&](int n) {
        const int sl = n & 1;
        const int h = kvh * G + n / nqs;
        const int i0 = (s_begin + n % nqs) * kBQ;
        const uint16_t* qg = (const uint16_t*)p.q + ((size_t)b * Sq * p.Hq + h) * D;
        const uint16_t* dg = (const uint16_t*)p.dout + ((size_t)b * Sq * p.Hq + h) * D;
#pragma unroll
        for (int x = 0; x < XPW; ++x) {
            const int xi = wave * XPW + x;
            const int row = xi * ROWS_PER_XFER + lane / CH;
            const int i = min(i0 + row, Sq - 1);
            const int ch = ((lane % CH) ^ swz<D>(row)) * 8;
            dma16(qg + (size_t)i * q_row + ch, lds_base + (uint32_t)((2 * sl) * QT * 2 + xi * 1024));
            dma16(dg + (size_t)i * q_row + ch, lds_base + (uint32_t)((2 * sl + 1) * QT * 2 + xi * 1024));
        }
        if constexpr (FB_LDS) {
            if (fb_dma) {
                const uint16_t* bg = (const uint16_t*)p.bias + ((size_t)b * p.Hq + h) * (size_t)Sq * Sk;
                const int nchunk = min(kBK, Sk - k0) / 8;
#pragma unroll
                for (int x = 0; x < XPB; ++x) {
                    const int xi = wave * XPB + x;
                    const int row = xi * 4 + (lane >> 4);
                    const int c = min((lane & 15) ^ (4 * ((row >> 4) & 1)), nchunk - 1);
                    dma16(bg + (size_t)min(i0 + row, Sq - 1) * Sk + k0 + 8 * c,
                          lds_base + (uint32_t)((4 * QT + sl * BTILE) * 2 + xi * 1024));
                }
            }
        }
        if (tid < kBQ) {
            const int i = i0 + tid;
            float l2 = INFINITY, dd = 0.f;
            if (i < Sq) {
                const size_t ri = ((size_t)b * p.Hq + h) * Sq + i;
                const float l = p.lse[ri];
                l2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
                dd = p.delta[ri];
            }
            rowc[sl][0][tid] = l2;
            rowc[sl][1][tid] = dd;
        }
    };

    // Lane-dependent LDS byte offsets inside a tile; block, group and slot offsets are
    // compile-time constants added on top. Row-wise reads (A operand of S and dP): row
    // perm32(r32) + 32 qb, chunk (2 ks + hh) ^ swz. Transposing reads (A operand of the
    // dV / dK products): rows 16 hh + (li >> 2) (+4) + 8 sg + 32 qb, see read_tr.
    uint32_t rr_off[KS], tr_off[2 * DB];
    {
        const int row = perm32(r32);
        const int sw = swz<D>(row);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) rr_off[ks] = (uint32_t)(row * D + (((2 * ks + hh) ^ sw) << 3)) * 2;
        const int li = lane & 15, la = li & 3, gg = lane >> 4;
        const int trow = 16 * hh + (li >> 2);
        const int dlo = 16 * DB * (gg & 1) + 8 * (la & 1) + 4 * (la >> 1);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int r = trow + 4 * half;
            const int sw2 = swz<D>(r);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = 16 * db + dlo;
                tr_off[2 * db + half] = (uint32_t)(r * D + ((((d >> 3) ^ sw2) << 3) | (d & 7))) * 2;
            }
        }
    }
    const char* lds = (const char*)smem;

    // The whole row loop of one role. Both roles run the same number of steps and barriers.
    auto run = [&](auto role) {
        constexpr bool DK = decltype(role)::value;
        // K fragments (sign-flipped for a negative scale) and, for dK, V fragments of this
        // lane's key: dims 16 ks + 8 hh .. + 7 (B operands of S = Q.K^T and dP = dO.V^T)
        bf16x8 kf[KS], vf[DK ? KS : 1];
        {
            const uint16_t* kr = (const uint16_t*)p.k + kv_off + hh * 8;
            const uint16_t* vr = (const uint16_t*)p.v + kv_off + hh * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 x = *(const u32x4*)(kr + ks * 16);
                if (!key_ok) x = u32x4{0, 0, 0, 0};
                if (neg) x ^= 0x80008000u;
                kf[ks] = __builtin_bit_cast(bf16x8, x);
                if constexpr (DK) {
                    u32x4 y = *(const u32x4*)(vr + ks * 16);
                    if (!key_ok) y = u32x4{0, 0, 0, 0};
                    vf[ks] = __builtin_bit_cast(bf16x8, y);
                }
            }
        }
        f32x16 acc[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;

        // one 32-row block (rows r0 = kBQ s + 32 QB ..) of step n in slot SL
        auto compute_block = [&](int n, auto sl_tag, auto qb_tag) {
            constexpr int SL = decltype(sl_tag)::value, QB = decltype(qb_tag)::value;
            const int h = kvh * G + n / nqs;
            const int r0 = (s_begin + n % nqs) * kBQ + 32 * QB;
            const int pa = r0 + off, pb = min(r0 + 31, Sq - 1) + off;
            bool skip = !wave_ok || r0 >= Sq;
            if constexpr (MASK != MASK_NONE) skip = skip || (pb < kw0);
            if constexpr (MASK == MASK_SLIDING) skip = skip || (pa - kwe >= p.window);
            if (uniform(skip)) return;
            bool m = (r0 + 31 >= Sq) || (kw0 + 31 >= Sk);
            if constexpr (MASK != MASK_NONE) m = m || (pa < kwe);
            if constexpr (MASK == MASK_SLIDING) m = m || (pb - kw0 >= p.window);
            const bool msk = uniform(m);
            constexpr uint32_t QTB = (2 * SL) * QT * 2, DTB = (2 * SL + 1) * QT * 2;   // tile bytes
            constexpr uint32_t BLK = 32 * QB * D * 2;
            f32x16 s, dp;
#pragma unroll
            for (int v = 0; v < 16; ++v) { s[v] = 0.f; dp[v] = 0.f; }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 aq = *(const bf16x8*)(lds + rr_off[ks] + (QTB + BLK));
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[ks], s, 0, 0, 0);
                if constexpr (DK) {
                    const bf16x8 ad = *(const bf16x8*)(lds + rr_off[ks] + (DTB + BLK));
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, vf[ks], dp, 0, 0, 0);
                }
            }
            // register v of lane half hh: query row r0 + 16 hh + v, key my_j
            const int rl = 32 * QB + 16 * hh;                      // row of register 0 in the tile
            const int pos0 = r0 + 16 * hh + off;                   // its position
            float x[16];
            {
                if (FB_LDS && fb_dma) {
                    // column my_j of rows rl .. rl + 15 of the bias tile (row bit 4 = hh)
                    const int kk = my_j - k0;
                    const uint16_t* bcol = smem + 4 * QT + SL * BTILE + rl * kBK +
                                           ((((kk >> 3) ^ (4 * hh)) << 3) | (kk & 7));
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        x[v] = fmaf(bf16_to_f32(bcol[v * kBK]), kLog2e, s[v] * c_scale);
                } else {
                    const uint16_t* br = (const uint16_t*)p.bias + ((size_t)b * p.Hq + h) * Sq * (size_t)Sk;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int i = r0 + 16 * hh + v;
                        const float bv = (i < Sq && key_ok) ? bf16_to_f32(br[(size_t)i * Sk + my_j]) : 0.f;
                        x[v] = fmaf(bv, kLog2e, s[v] * c_scale);
                    }
                }
            }
            if (msk) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int pos = pos0 + v;
                    bool vis = key_ok & (pos - off < Sq);
                    if constexpr (MASK != MASK_NONE) vis = vis & (my_j <= pos);
                    if constexpr (MASK == MASK_SLIDING) vis = vis & (pos - my_j < p.window);
                    x[v] = vis ? x[v] : -INFINITY;
                }
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 lr = *(const u32x4*)(&rowc[SL][0][rl + 4 * c]);
                u32x4 dr;
                if constexpr (DK) dr = *(const u32x4*)(&rowc[SL][1][rl + 4 * c]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = 4 * c + e;
                    const float pv = __builtin_amdgcn_exp2f(x[v] - __uint_as_float(lr[e]));
                    if constexpr (DK) s[v] = pv * (dp[v] - __uint_as_float(dr[e]));   // dS
                    else s[v] = pv;                                                     // P
                }
            }
            // dV^T += dO^T P  or  dK^T += Q^T dS, over the two 16-row groups of the block
            constexpr uint32_t TTB = DK ? QTB : DTB;
#pragma unroll
            for (int sg = 0; sg < 2; ++sg) {
                u32x4 pk;
#pragma unroll
                for (int c = 0; c < 4; ++c) pk[c] = pack_bf16x2(s[8 * sg + 2 * c], s[8 * sg + 2 * c + 1]);
                const bf16x8 bp = __builtin_bit_cast(bf16x8, pk);
                const uint32_t gofs = TTB + (uint32_t)((32 * QB + 8 * sg) * D * 2);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const s16x4 lo = lds_read_tr((const uint16_t*)(lds + tr_off[2 * db] + gofs));
                    const s16x4 hi = lds_read_tr((const uint16_t*)(lds + tr_off[2 * db + 1] + gofs));
                    u32x4 av;
                    av[0] = __builtin_bit_cast(u32x2, lo)[0];
                    av[1] = __builtin_bit_cast(u32x2, lo)[1];
                    av[2] = __builtin_bit_cast(u32x2, hi)[0];
                    av[3] = __builtin_bit_cast(u32x2, hi)[1];
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), bp, acc[db], 0, 0, 0);
                }
            }
        };

        auto step = [&](int n, auto sl_tag) {
            const bool has_next = n + 1 < n_steps;
            if (has_next) issue_step(n + 1);
            compute_block(n, sl_tag, std::integral_constant<int, 0>{});
            compute_block(n, sl_tag, std::integral_constant<int, 1>{});
            if constexpr (NB == 4) {
                compute_block(n, sl_tag, std::integral_constant<int, 2>{});
                compute_block(n, sl_tag, std::integral_constant<int, 3>{});
            }
            static_assert(NB == 2 || NB == 4, "two or four 32-row blocks per step");
            if (has_next) dma_wait();
            __syncthreads();
        };
#pragma unroll 1
        for (int n = 0; n < n_steps; n += 2) {
            step(n, std::integral_constant<int, 0>{});
            if (n + 1 < n_steps) step(n + 1, std::integral_constant<int, 1>{});
        }
        if (key_ok) store_row<D, OUT_F32>(out_row, acc, DK ? p.scale : 1.f, hh);
    };

    issue_step(0);
    dma_wait();
    __syncthreads();
    if (role_dk) run(std::true_type{});
    else run(std::false_type{});
}

// ------------------------------------------------------------------------------------------
// dK, dV: 128 keys of one (batch, KV head) per workgroup (64 at D = 256), query rows in steps
// of 64 (128 at D = 32, 32 at D = 256) through a 3-slot LDS ring, scores formed once per
// (row, key). The first half of the waves (dV) form S = Q.K^T and P for their
// 32 keys each, accumulate dV^T += dO^T.P and leave P, rounded to bf16 as their MFMA operand,
// in LDS. The second half (dK) run one step behind on the same keys: dP = dO.V^T,
// dS = P (dP - D) with that P, dK^T += Q^T.dS; they need neither the bias nor the mask (P is
// 0 wherever the mask hides a pair). Each step ends
// with one barrier; after it the dK waves read what the dV waves wrote, and the ring slot of
// the step two back is refilled (its last reader, a dK wave, finished before the barrier).
// ------------------------------------------------------------------------------------------
template <int D, int MASK, int BIAS, bool OUT_F32>
__global__ __launch_bounds__(64 * bwd_waves<D>(), 1) void dkdv_lag_kernel(const BwdParams p) {
    constexpr int kWaves = bwd_waves<D>(), kThreads = 64 * kWaves, KG = kWaves / 2;
    constexpr int kBK = 32 * KG, NS = 3;       // keys per workgroup, ring slots
    constexpr int kBQ = D == 256 ? 32 : (D == 32 ? 128 : 64), NB = kBQ / 32;
    constexpr int CH = D / 8, KS = D / 16, DB = D / 32, QT = kBQ * D;
    constexpr bool IS_T5 = BIAS == BIAS_T5 || BIAS == BIAS_T5U;
    constexpr bool ALIBI = BIAS == BIAS_ALIBI;
    constexpr int kSat = BIAS == BIAS_T5U ? kT5USat : kT5Sat;
    constexpr int kT5Pad = kSat + 64 + 31;
    constexpr bool FB = BIAS == BIAS_FULL;
    // A full bias (D = 64 only; dkdv_kernel takes it at the other head dims, where the slots
    // and the P buffers leave no room for it) goes through the ring: a [kBQ rows][128 keys]
    // tile per slot.
    static_assert(!FB || D == 64, "full bias: D = 64 only");
    constexpr bool FB_LDS = FB;
    constexpr int BTILE = FB_LDS ? kBQ * kBK : 0;
    // LDS: slot sl holds the Q tile at [2 sl] and the dO tile at [2 sl + 1] (kBQ rows each), the
    // bias tiles follow at [2 NS QT + sl BTILE]; P of slot sl, key group kg (the dV wave), row
    // block qb, 8-row group sg: pbuf[sl][kg][qb][sg] (lane-major, so every write and read is one
    // conflict-free 16-byte access per lane)
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * NS * QT + NS * BTILE];
    __shared__ __attribute__((aligned(16))) u32x4 pbuf[NS][KG][NB][2][64];
    __shared__ __attribute__((aligned(16))) float rowc[NS][2][kBQ];    // [slot][lse2, D][row]
    __shared__ float t5s[IS_T5 ? 2 * kT5Pad + 1 : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, r32 = lane & 31;
    const bool role_dk = uniform(wave >= KG);
    const int kg = wave % KG;                  // key group: one dV and one dK wave share it
    int group, kt_idx;
    {
        const int x = blockIdx.x;
        if (p.xcd_remap) {
            const int slot = x >> 3, gl = slot / p.n_kt;
            kt_idx = slot - gl * p.n_kt;
            group = gl * 8 + (x & 7);
        } else {
            group = x / p.n_kt;
            kt_idx = x - group * p.n_kt;
        }
    }
    const int b = group / p.Hkv, kvh = group - b * p.Hkv;
    const int Sq = p.Sq, Sk = p.Sk, off = p.off, G = p.G;
    const int k0 = kt_idx * kBK;
    const int kw0 = k0 + 32 * kg;              // first key of this wave
    const int my_j = kw0 + r32;                // key of this lane
    const bool key_ok = my_j < Sk;
    const bool wave_ok = kw0 < Sk;
    const int kwe = min(kw0 + 31, Sk - 1);     // last valid key of the wave

    const size_t q_row = (size_t)p.Hq * D, kv_row = (size_t)p.Hkv * D;
    const size_t kv_off = ((size_t)b * Sk + (key_ok ? my_j : 0)) * kv_row + (size_t)kvh * D;
    char* out_row = (char*)(role_dk ? p.dk : p.dv) + kv_off * (OUT_F32 ? 4 : 2);

    // query rows the workgroup's keys can see (positions of the rows: i + off)
    const int kend = min(k0 + kBK, Sk) - 1;
    int qlo = 0, qhi = Sq;
    if constexpr (MASK != MASK_NONE) qlo = max(0, k0 - off);
    if constexpr (MASK == MASK_SLIDING) qhi = min(Sq, kend + p.window - off);
    const int s_begin = qlo / kBQ;
    const int s_end = (qhi <= qlo) ? s_begin : (qhi + kBQ - 1) / kBQ;
    const int nqs = s_end - s_begin;
    const int n_steps = G * nqs;

    if (n_steps == 0) {        // no query row sees these keys: dK = dV = 0
        if (key_ok) store_zero_row<D, OUT_F32>(out_row, hh);
        return;
    }
    const bool neg = p.scale_log2 < 0.f;
    const float c_scale = neg ? -p.scale_log2 : (p.scale_log2 == 0.f ? kTinyScale : p.scale_log2);

    // Q / dO tiles of step n into slot sl: head h = kvh * G + n / nqs, rows kBQ s .. + kBQ - 1
    // (clamped), and the rows' lse (log2 units) and D
    constexpr int ROWS_PER_XFER = 1024 / (D * 2), XFERS = (kBQ * D * 2) / 1024, XPW = XFERS / kWaves;
    static_assert(XPW * kWaves == XFERS, "dma split");
    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)smem);
    // The bias tile goes through LDS when its rows split into whole 16-byte chunks: 256-byte
    // rows, chunk swizzle 4 * ((row >> 4) & 1); keys past the end of a partial last tile re-read
    // the last whole chunk (they are masked).
    const bool fb_dma = FB_LDS && ((Sk & 7) == 0);
    constexpr int XPB = FB_LDS ? (BTILE * 2 / 1024) / kWaves : 0;
    static_assert(!FB_LDS || XPB * kWaves * 1024 == BTILE * 2, "bias dma split");
    auto issue_step = [&](int n, int sl) {
        const int h = kvh * G + n / nqs;
        const int i0 = (s_begin + n % nqs) * kBQ;
        const uint16_t* qg = (const uint16_t*)p.q + ((size_t)b * Sq * p.Hq + h) * D;
        const uint16_t* dg = (const uint16_t*)p.dout + ((size_t)b * Sq * p.Hq + h) * D;
#pragma unroll
        for (int x = 0; x < XPW; ++x) {
            const int xi = wave * XPW + x;
            const int row = xi * ROWS_PER_XFER + lane / CH;
            const int i = min(i0 + row, Sq - 1);
            const int ch = ((lane % CH) ^ swz<D>(row)) * 8;
            dma16(qg + (size_t)i * q_row + ch, lds_base + (uint32_t)((2 * sl) * QT * 2 + xi * 1024));
            dma16(dg + (size_t)i * q_row + ch, lds_base + (uint32_t)((2 * sl + 1) * QT * 2 + xi * 1024));
        }
        if constexpr (FB_LDS) {
            if (fb_dma) {
                // k0 < Sk and both multiples of 8: at least one whole chunk
                const uint16_t* bg = (const uint16_t*)p.bias + ((size_t)b * p.Hq + h) * (size_t)Sq * Sk;
                const int nchunk = min(kBK, Sk - k0) / 8;
#pragma unroll
                for (int x = 0; x < XPB; ++x) {
                    const int xi = wave * XPB + x;
                    const int row = xi * 4 + (lane >> 4);
                    const int c = min((lane & 15) ^ (4 * ((row >> 4) & 1)), nchunk - 1);
                    dma16(bg + (size_t)min(i0 + row, Sq - 1) * Sk + k0 + 8 * c,
                          lds_base + (uint32_t)((2 * NS * QT + sl * BTILE) * 2 + xi * 1024));
                }
            }
        }
        if (tid < kBQ) {
            const int i = i0 + tid;
            float l2 = INFINITY, dd = 0.f;
            if (i < Sq) {
                const size_t ri = ((size_t)b * p.Hq + h) * Sq + i;
                const float l = p.lse[ri];
                l2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
                dd = p.delta[ri];
            }
            rowc[sl][0][tid] = l2;
            rowc[sl][1][tid] = dd;
        }
    };

    // Lane-dependent LDS byte offsets inside a tile: row-wise reads for the
    // A operands of S and dP, transposing reads for the A operands of the dV / dK products.
    uint32_t rr_off[KS], tr_off[2 * DB];
    {
        const int row = perm32(r32);
        const int sw = swz<D>(row);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) rr_off[ks] = (uint32_t)(row * D + (((2 * ks + hh) ^ sw) << 3)) * 2;
        const int li = lane & 15, la = li & 3, gg = lane >> 4;
        const int trow = 16 * hh + (li >> 2);
        const int dlo = 16 * DB * (gg & 1) + 8 * (la & 1) + 4 * (la >> 1);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int r = trow + 4 * half;
            const int sw2 = swz<D>(r);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int d = 16 * db + dlo;
                tr_off[2 * db + half] = (uint32_t)(r * D + ((((d >> 3) ^ sw2) << 3) | (d & 7))) * 2;
            }
        }
    }
    const char* lds = (const char*)smem;

    auto run = [&](auto role) {
        constexpr bool DK = decltype(role)::value;
        // B operand fragments of this lane's key, dims 16 ks + 8 hh .. + 7: K (sign-flipped for a
        // negative scale) for S = Q.K^T in the dV role, V for dP = dO.V^T in the dK role
        bf16x8 bfr[KS];
        {
            const uint16_t* r = (const uint16_t*)(DK ? p.v : p.k) + kv_off + hh * 8;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 x = *(const u32x4*)(r + ks * 16);
                if (!key_ok) x = u32x4{0, 0, 0, 0};
                if (!DK && neg) x ^= 0x80008000u;
                bfr[ks] = __builtin_bit_cast(bf16x8, x);
            }
        }
        f32x16 acc[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;

        // one 32-row block (rows r0 = kBQ s + 32 QB ..) of step n in slot SL
        auto compute_block = [&](int n, auto sl_tag, auto qb_tag) {
            constexpr int SL = decltype(sl_tag)::value, QB = decltype(qb_tag)::value;
            const int r0 = (s_begin + n % nqs) * kBQ + 32 * QB;
            const int pa = r0 + off, pb = min(r0 + 31, Sq - 1) + off;
            // the same test in both roles: a block the dV wave skips leaves no P, and the dK
            // wave skips it too
            bool skip = !wave_ok || r0 >= Sq;
            if constexpr (MASK != MASK_NONE) skip = skip || (pb < kw0);
            if constexpr (MASK == MASK_SLIDING) skip = skip || (pa - kwe >= p.window);
            if (uniform(skip)) return;
            constexpr uint32_t QTB = (2 * SL) * QT * 2, DTB = (2 * SL + 1) * QT * 2;   // tile bytes
            constexpr uint32_t BLK = 32 * QB * D * 2;
            const int rl = 32 * QB + 16 * hh;      // tile row of register 0 of this lane half
            f32x16 s;
#pragma unroll
            for (int v = 0; v < 16; ++v) s[v] = 0.f;
            // S = Q.K^T (dV role) or dP = dO.V^T (dK role); register v of lane half hh: query
            // row r0 + 16 hh + v, key my_j
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = *(const bf16x8*)(lds + rr_off[ks] + ((DK ? DTB : QTB) + BLK));
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bfr[ks], s, 0, 0, 0);
            }
            u32x4 pk[2];
            if constexpr (!DK) {
                const int h = kvh * G + n / nqs;
                bool m = (r0 + 31 >= Sq) || (kw0 + 31 >= Sk);
                if constexpr (MASK != MASK_NONE) m = m || (pa < kwe);
                if constexpr (MASK == MASK_SLIDING) m = m || (pb - kw0 >= p.window);
                const bool msk = uniform(m);
                const int pos0 = r0 + 16 * hh + off;   // position of register 0's row
                float x[16];
                if constexpr (ALIBI) {
                    // rel = my_j - position of row v
                    const float aslope = ((const float*)p.bias)[h] * kLog2e;
                    const float base = (float)(my_j - pos0);
#pragma unroll
                    for (int v = 0; v < 16; ++v) x[v] = fmaf(s[v], c_scale, -aslope * fabsf(base - (float)v));
                } else if constexpr (IS_T5) {
                    const int rmin = kw0 - pb, rmax = kwe - pa;
                    const int side = uniform(rmin >= kSat ? 1 : (rmax <= -kSat ? -1 : 0));
                    if (side == 0) {
                        // rel = my_j - position of row v; stays inside the padded table
                        const float* trow = t5s + kT5Pad + (my_j - pos0);
#pragma unroll
                        for (int v = 0; v < 16; ++v) x[v] = fmaf(s[v], c_scale, trow[-v]);
                    } else {
                        const float bconst = side > 0 ? t5s[2 * kT5Pad] : t5s[0];
#pragma unroll
                        for (int v = 0; v < 16; ++v) x[v] = fmaf(s[v], c_scale, bconst);
                    }
                } else if constexpr (FB) {
                    if (FB_LDS && fb_dma) {
                        // column my_j of rows rl .. rl + 15 of the bias tile (row bit 4 = hh)
                        const int kk = my_j - k0;
                        const uint16_t* bcol = smem + 2 * NS * QT + SL * BTILE + rl * kBK +
                                               ((((kk >> 3) ^ (4 * hh)) << 3) | (kk & 7));
#pragma unroll
                        for (int v = 0; v < 16; ++v)
                            x[v] = fmaf(bf16_to_f32(bcol[v * kBK]), kLog2e, s[v] * c_scale);
                    } else {
                        const uint16_t* br = (const uint16_t*)p.bias + ((size_t)b * p.Hq + h) * Sq * (size_t)Sk;
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int i = r0 + 16 * hh + v;
                            const float bv = (i < Sq && key_ok) ? bf16_to_f32(br[(size_t)i * Sk + my_j]) : 0.f;
                            x[v] = fmaf(bv, kLog2e, s[v] * c_scale);
                        }
                    }
                } else {
#pragma unroll
                    for (int v = 0; v < 16; ++v) x[v] = s[v] * c_scale;
                }
                if (msk) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int pos = pos0 + v;
                        bool vis = key_ok & (pos - off < Sq);
                        if constexpr (MASK != MASK_NONE) vis = vis & (my_j <= pos);
                        if constexpr (MASK == MASK_SLIDING) vis = vis & (pos - my_j < p.window);
                        x[v] = vis ? x[v] : -INFINITY;
                    }
                }
                float pv[16];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4 lr = *(const u32x4*)(&rowc[SL][0][rl + 4 * c]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) pv[4 * c + e] = __builtin_amdgcn_exp2f(x[4 * c + e] - __uint_as_float(lr[e]));
                }
#pragma unroll
                for (int sg = 0; sg < 2; ++sg) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) pk[sg][c] = pack_bf16x2(pv[8 * sg + 2 * c], pv[8 * sg + 2 * c + 1]);
                    pbuf[SL][kg][QB][sg][lane] = pk[sg];
                }
            } else {
                // dS = P (dP - D) with the dV wave's P of the same (row, key)
#pragma unroll
                for (int sg = 0; sg < 2; ++sg) {
                    const u32x4 pin = pbuf[SL][kg][QB][sg][lane];
                    const u32x4 dr0 = *(const u32x4*)(&rowc[SL][1][rl + 8 * sg]);
                    const u32x4 dr1 = *(const u32x4*)(&rowc[SL][1][rl + 8 * sg + 4]);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int v = 8 * sg + 2 * c;
                        const float d0 = __uint_as_float(c < 2 ? dr0[2 * c] : dr1[2 * c - 4]);
                        const float d1 = __uint_as_float(c < 2 ? dr0[2 * c + 1] : dr1[2 * c - 3]);
                        const float p0 = bf16_to_f32(pin[c] & 0xffffu), p1 = bf16_to_f32(pin[c] >> 16);
                        pk[sg][c] = pack_bf16x2(p0 * (s[v] - d0), p1 * (s[v + 1] - d1));
                    }
                }
            }
            // dV^T += dO^T P  or  dK^T += Q^T dS, over the two 8-row groups of each lane half
            constexpr uint32_t TTB = DK ? QTB : DTB;
#pragma unroll
            for (int sg = 0; sg < 2; ++sg) {
                const bf16x8 bp = __builtin_bit_cast(bf16x8, pk[sg]);
                const uint32_t gofs = TTB + (uint32_t)((32 * QB + 8 * sg) * D * 2);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const s16x4 lo = lds_read_tr((const uint16_t*)(lds + tr_off[2 * db] + gofs));
                    const s16x4 hi = lds_read_tr((const uint16_t*)(lds + tr_off[2 * db + 1] + gofs));
                    u32x4 av;
                    av[0] = __builtin_bit_cast(u32x2, lo)[0];
                    av[1] = __builtin_bit_cast(u32x2, lo)[1];
                    av[2] = __builtin_bit_cast(u32x2, hi)[0];
                    av[3] = __builtin_bit_cast(u32x2, hi)[1];
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), bp, acc[db], 0, 0, 0);
                }
            }
        };

        // iteration it: the dV waves take step it (slot SL), the dK waves step it - 1 (slot
        // (SL + 2) % 3), and step it + 1 streams into slot (SL + 1) % 3. Both roles run the same
        // iterations and barriers.
        auto iter = [&](int it, auto sl_tag) {
            constexpr int SL = decltype(sl_tag)::value, SP = (SL + 2) % NS, SN = (SL + 1) % NS;
            if constexpr (IS_T5) {
                // table of the dV waves' head when it changes (its readers of the previous table
                // finished before the last barrier; one more barrier after the writes)
                if (it < n_steps) {
                    const int h = kvh * G + it / nqs;
                    if (it == 0 || h != kvh * G + (it - 1) / nqs) {
                        const float* tbl = (const float*)p.bias + (size_t)h * kT5Buckets;
                        for (int i = tid; i < 2 * kT5Pad + 1; i += kThreads)
                            t5s[i] = tbl[BIAS == BIAS_T5U ? t5u_bucket(i - kT5Pad) : t5_bucket(i - kT5Pad)] * kLog2e;
                        __syncthreads();
                    }
                }
            }
            const bool has_next = it + 1 < n_steps;
            if (has_next) issue_step(it + 1, SN);
            if constexpr (DK) {
                if (it >= 1) {
                    compute_block(it - 1, std::integral_constant<int, SP>{}, std::integral_constant<int, 0>{});
                    if constexpr (NB >= 2)
                        compute_block(it - 1, std::integral_constant<int, SP>{}, std::integral_constant<int, 1>{});
                    if constexpr (NB == 4) {
                        compute_block(it - 1, std::integral_constant<int, SP>{}, std::integral_constant<int, 2>{});
                        compute_block(it - 1, std::integral_constant<int, SP>{}, std::integral_constant<int, 3>{});
                    }
                }
            } else {
                if (it < n_steps) {
                    compute_block(it, std::integral_constant<int, SL>{}, std::integral_constant<int, 0>{});
                    if constexpr (NB >= 2)
                        compute_block(it, std::integral_constant<int, SL>{}, std::integral_constant<int, 1>{});
                    if constexpr (NB == 4) {
                        compute_block(it, std::integral_constant<int, SL>{}, std::integral_constant<int, 2>{});
                        compute_block(it, std::integral_constant<int, SL>{}, std::integral_constant<int, 3>{});
                    }
                }
            }
            static_assert(NB == 1 || NB == 2 || NB == 4, "one, two or four 32-row blocks per step");
            if (has_next) dma_wait();
            __syncthreads();
        };
#pragma unroll 1
        for (int it = 0; it <= n_steps; it += NS) {
            iter(it, std::integral_constant<int, 0>{});
            if (it + 1 <= n_steps) iter(it + 1, std::integral_constant<int, 1>{});
            if (it + 2 <= n_steps) iter(it + 2, std::integral_constant<int, 2>{});
        }
        if (key_ok) store_row<D, OUT_F32>(out_row, acc, DK ? p.scale : 1.f, hh);
    };

    issue_step(0, 0);
    dma_wait();
    __syncthreads();
    if (role_dk) run(std::true_type{});
    else run(std::false_type{});
}

// ------------------------------------------------------------------------------------------
// host-side launch
// ------------------------------------------------------------------------------------------
template <int D, int MASK, int BIAS, bool OUT_F32>
static hipError_t launch_grads(const BwdParams& p, hipStream_t s) {
    const unsigned gq = (unsigned)((size_t)p.B * p.Hq * p.n_qt);
    hipLaunchKernelGGL((dq_kernel<D, MASK, BIAS, OUT_F32>), dim3(gq), dim3(64 * bwd_waves<D>()), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned gk = (unsigned)((size_t)p.B * p.Hkv * p.n_kt);
    if constexpr (BIAS != BIAS_FULL || D == 64)
        hipLaunchKernelGGL((dkdv_lag_kernel<D, MASK, BIAS, OUT_F32>), dim3(gk), dim3(64 * bwd_waves<D>()), 0, s, p);
    else
        hipLaunchKernelGGL((dkdv_kernel<D, MASK, BIAS, OUT_F32>), dim3(gk), dim3(64 * bwd_waves<D>()), 0, s, p);
    return hipGetLastError();
}

template <int D, bool OUT_F32>
static hipError_t launch_d(BwdParams p, int mask, int bias, hipStream_t s) {
    // dQ work items of 32 rows per wave, dK/dV work items of 32 keys per wave pair
    p.n_qt = (p.Sq + 32 * bwd_waves<D>() - 1) / (32 * bwd_waves<D>());
    p.n_kt = (p.Sk + 16 * bwd_waves<D>() - 1) / (16 * bwd_waves<D>());
#define SDPA_CASE(M, Bk) \
    if (mask == M && bias == Bk) return launch_grads<D, M, Bk, OUT_F32>(p, s);
    SDPA_CASE(MASK_NONE, BIAS_NONE) SDPA_CASE(MASK_NONE, BIAS_T5) SDPA_CASE(MASK_NONE, BIAS_FULL)
    SDPA_CASE(MASK_CAUSAL, BIAS_NONE) SDPA_CASE(MASK_CAUSAL, BIAS_T5) SDPA_CASE(MASK_CAUSAL, BIAS_FULL)
    SDPA_CASE(MASK_SLIDING, BIAS_NONE) SDPA_CASE(MASK_SLIDING, BIAS_T5) SDPA_CASE(MASK_SLIDING, BIAS_FULL)
    SDPA_CASE(MASK_NONE, BIAS_ALIBI) SDPA_CASE(MASK_CAUSAL, BIAS_ALIBI) SDPA_CASE(MASK_SLIDING, BIAS_ALIBI)
    SDPA_CASE(MASK_NONE, BIAS_T5U) SDPA_CASE(MASK_CAUSAL, BIAS_T5U) SDPA_CASE(MASK_SLIDING, BIAS_T5U)
#undef SDPA_CASE
    return hipErrorInvalidValue;
}

}  // namespace bwd

hipError_t launch_bwd_bf16(BwdParams p, int D, int mask, int bias, bool out_f32, hipStream_t s) {
    p.xcd_remap = ((p.B * p.Hkv) % 8 == 0) ? 1 : 0;   // both kernels map (batch, KV head) groups to XCDs
    if (D == 128)
        return out_f32 ? bwd::launch_d<128, true>(p, mask, bias, s) : bwd::launch_d<128, false>(p, mask, bias, s);
    if (D == 64)
        return out_f32 ? bwd::launch_d<64, true>(p, mask, bias, s) : bwd::launch_d<64, false>(p, mask, bias, s);
    if (D == 32)
        return out_f32 ? bwd::launch_d<32, true>(p, mask, bias, s) : bwd::launch_d<32, false>(p, mask, bias, s);
    if (D == 256)
        return out_f32 ? bwd::launch_d<256, true>(p, mask, bias, s) : bwd::launch_d<256, false>(p, mask, bias, s);
    return hipErrorInvalidValue;
}

}  // namespace sdpa
