// gfx950 split-key decode: O = softmax(Q.K^T * scale + bias + mask) . V for few query rows
// against a long key/value cache (generation: each new token's queries attend to the cached
// keys and values, the KV-cache section of the Medium post "Simplified Explanation of
// Attention"), with the masks, biases and head sharing of the forward kernel (the
// "jax-gpu-05-attention-gpu" codelab, sections 1, 7 and 9; FAT5 README attention biases).
//
// With one query row per head there is too little work per (batch, head) to fill the chip by
// splitting query rows, so the key range is split instead:
//   split_kernel : one workgroup = 4 waves = one 32-row block of the G * Sq query rows sharing
//                  a KV head (row r = i * G + g: query row i of head kvh * G + g), and one
//                  contiguous range of 64-key tiles. K and V tiles stream through a 4-slot LDS
//                  ring with three tiles in flight (D = 256, and D = 128 when a split has at
//                  most 32 tiles: 2 slots, one tile in flight, two workgroups per CU at
//                  D = 128; the LDS holds only two K/V tile pairs at D = 256). Wave (kh, dh)
//                  takes key half kh of every tile and head-dim half dh of O: S^T = K.Q^T
//                  (lane = query row), an online softmax (running max m, sum l, both per row)
//                  and O^T += V^T.P^T with V^T from transposing LDS reads. The two key halves' (m, l, O) are then combined
//                  in a fixed order into one partial result per split, stored in the workspace
//                  (or, with a single split, normalised and stored as the output).
//   merge_kernel : combines the splits of each row in split order:
//                  m = max m_s, l = sum l_s 2^(m_s - m), O = sum O_s 2^(m_s - m) / l.
// Every value has one writer and a fixed summation order: bitwise reproducible run to run.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "sdpa_decode.h"
#include "sdpa_device.h"
#include "sdpa_params.h"

namespace sdpa {
namespace dec {

using namespace dev;

constexpr int kWaves = 4, kThreads = 256, kBN = 64;
template <int D> constexpr int ring_slots() { return D == 256 ? 2 : 4; }
constexpr float kLn2 = 0.6931471805599453f;

// D / 8 output columns starting at col0 of query row r (= i * G + g) of (batch b, KV head kvh),
// times mul, and (from the first column chunk) the row's log-sum-exp
template <int D, bool OUT_F32>
__device__ __forceinline__ void store_out(const DecParams& p, int b, int kvh, int r, int col0,
                                          const float* o, float mul, float lse) {
    const int i = r / p.G, hq = kvh * p.G + (r - i * p.G);
    const size_t row = ((size_t)b * p.Sq + i) * p.Hq + hq;
    if constexpr (OUT_F32) {
        float* dst = (float*)p.out + row * D + col0;
#pragma unroll
        for (int c = 0; c < D / 8; c += 4) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(o[c + e] * mul);
            *(u32x4*)(dst + c) = w;
        }
    } else if constexpr (D / 8 >= 8) {
        uint16_t* dst = (uint16_t*)p.out + row * D + col0;
#pragma unroll
        for (int c = 0; c < D / 8; c += 8) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(o[c + 2 * e] * mul, o[c + 2 * e + 1] * mul);
            *(u32x4*)(dst + c) = w;
        }
    } else {                                         // D = 32: 4 columns
        uint16_t* dst = (uint16_t*)p.out + row * D + col0;
        u32x2 w;
        w[0] = pack_bf16x2(o[0] * mul, o[1] * mul);
        w[1] = pack_bf16x2(o[2] * mul, o[3] * mul);
        *(u32x2*)dst = w;
    }
    if (col0 == 0) p.lse[((size_t)b * p.Hq + hq) * p.Sq + i] = lse;
}

// ------------------------------------------------------------------------------------------
// one (batch, KV head, 32-row block, key split)
// ------------------------------------------------------------------------------------------
// NS: ring slots (tiles in flight + 1). A 4-slot ring at D = 128 fills the LDS of a CU; with 2
// slots two workgroups fit one CU.
template <int D, int MASK, int BIAS, bool OUT_F32, int NS>
__global__ __launch_bounds__(256, (D == 256 || (D == 128 && NS == 4)) ? 1 : 2)
void split_kernel(const DecParams p) {
    constexpr int KS = D / 16, DB = D / 32, TILE = kBN * D, CH = D / 8;
    constexpr bool FB = BIAS == BIAS_FULL;
    // slot u of the ring: K tile at [2u], V tile at [2u + 1]; reused for the wave merge
    constexpr int kNS = NS;
    // the ring, and after the last tile the buffer that merges the two key halves
    constexpr int RING = kNS * 2 * TILE, MERGE = (kWaves * 32 * D + 4 * 32) * 2;
    __shared__ __attribute__((aligned(16))) uint16_t smem[RING > MERGE ? RING : MERGE];
    constexpr bool IS_T5 = BIAS == BIAS_T5 || BIAS == BIAS_T5U;
    __shared__ float t5s[IS_T5 ? 32 * kT5Buckets : 1];   // [row of block][bucket]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, r32 = lane & 31;
    const int split = blockIdx.x % p.n_split;
    const int rest = blockIdx.x / p.n_split;
    const int rb = rest % p.n_rb, group = rest / p.n_rb;
    const int b = group / p.Hkv, kvh = group - b * p.Hkv;
    const int G = p.G, Sq = p.Sq, Sk = p.Sk, off = p.off;

    // this lane's query row
    const int r = 32 * rb + r32;
    const bool row_ok = r < p.rows;
    const int rr = row_ok ? r : 0;
    const int my_i = rr / G, my_g = rr - my_i * G, my_hq = kvh * G + my_g;
    const int my_pos = my_i + off;

    // keys any row of the block may see, cut into this split's range of 64-key tiles
    const int r_last = min(32 * rb + 31, p.rows - 1);
    const int pmin = (32 * rb) / G + off, pmax = r_last / G + off;
    int klo = 0, khi = Sk - 1;
    if constexpr (MASK != MASK_NONE) khi = min(khi, pmax);
    if constexpr (MASK == MASK_SLIDING) klo = max(0, pmin - p.window + 1);
    const int t_lo = klo / kBN;
    const int n_t = (khi < klo) ? 0 : khi / kBN - t_lo + 1;
    const int tps = (n_t + p.n_split - 1) / p.n_split;
    const int ts = t_lo + split * tps;
    const int nt = max(0, min(t_lo + n_t, ts + tps) - ts);

    // workspace of this unit
    const size_t unit = ((size_t)group * p.n_rb + rb) * p.n_split + split;
    const size_t units = (size_t)p.B * p.Hkv * p.n_rb * p.n_split;
    float* ws_o = p.ws + unit * 32 * D;
    float* ws_ml = p.ws + units * 32 * D + unit * 64;

    if constexpr (IS_T5) {
        for (int idx = tid; idx < 32 * kT5Buckets; idx += kThreads) {
            const int row = idx / kT5Buckets, bk = idx - row * kT5Buckets;
            const int rw = min(32 * rb + row, p.rows - 1);
            const int hq = kvh * G + (rw - (rw / G) * G);
            t5s[idx] = ((const float*)p.bias)[(size_t)hq * kT5Buckets + bk] * kLog2e;
        }
    }

    // ALiBi slope of this lane's head, log2 units
    const float aslope = BIAS == BIAS_ALIBI ? ((const float*)p.bias)[my_hq] * kLog2e : 0.f;
    const bool neg = p.scale_log2 < 0.f;
    const float c_scale = neg ? -p.scale_log2 : (p.scale_log2 == 0.f ? kTinyScale : p.scale_log2);
    bf16x8 qf[KS];
    {
        const uint16_t* qr = (const uint16_t*)p.q + (((size_t)b * Sq + my_i) * p.Hq + my_hq) * D + hh * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = *(const u32x4*)(qr + ks * 16);
            if (!row_ok) x = u32x4{0, 0, 0, 0};
            if (neg) x ^= 0x80008000u;
            qf[ks] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // K / V tile u of the split (rows past the end of the cache clamped; they are masked)
    const size_t kv_row = (size_t)p.Hkv * D;
    const uint16_t* kg = (const uint16_t*)p.k + ((size_t)b * Sk * p.Hkv + kvh) * D;
    const uint16_t* vg = (const uint16_t*)p.v + ((size_t)b * Sk * p.Hkv + kvh) * D;
    constexpr int ROWS_PER_XFER = 1024 / (D * 2), XFERS = TILE * 2 / 1024, XPW = XFERS / kWaves;
    static_assert(XPW * kWaves == XFERS, "dma split");
    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)smem);
    auto dma_tile = [&](int u) {
        const int sl = u % kNS, j0 = (ts + u) * kBN;
#pragma unroll
        for (int n = 0; n < XPW; ++n) {
            const int xi = wave * XPW + n;
            const int row = xi * ROWS_PER_XFER + lane / CH;
            const int j = min(j0 + row, Sk - 1);
            const int ch = ((lane % CH) ^ swz<D>(row)) * 8;
            dma16(kg + (size_t)j * kv_row + ch, lds_base + (uint32_t)((2 * sl) * TILE * 2 + xi * 1024));
            dma16(vg + (size_t)j * kv_row + ch, lds_base + (uint32_t)((2 * sl + 1) * TILE * 2 + xi * 1024));
        }
    };

    // Each 64-key tile is computed by all four waves: wave (kh, dh) takes key half kh and
    // accumulates the head dims of fragment half dh, so both waves of a key half form the same
    // S and P (same instructions). Running state of this wave's rows: max m (log2 units), this
    // lane half's part of the sum l, and its half of O^T (head dims x rows). At D = 32 there is
    // one fragment: the dh = 0 waves accumulate it, the dh = 1 waves only follow the softmax.
    constexpr int DH = DB > 1 ? DB / 2 : 1;
    constexpr bool ONE = DB == 1;
    const int kh = wave & 1, dh = wave >> 1;
    float m = -INFINITY, l = 0.f;
    f32x16 acc[DH];
#pragma unroll
    for (int db = 0; db < DH; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[db][v] = 0.f;

    const uint16_t* fbrow = FB ? (const uint16_t*)p.bias + (((size_t)b * p.Hq + my_hq) * Sq + my_i) * (size_t)Sk
                               : nullptr;
    auto compute = [&](int u) {
        const int sl = u % kNS;
        const int j0 = (ts + u) * kBN + 32 * kh;     // key of register 0 of lane half 0
        const uint16_t* kb = smem + (2 * sl) * TILE;
        const uint16_t* vb = smem + (2 * sl + 1) * TILE;
        f32x16 s;
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_rows<D>(kb, kh, ks, lane), qf[ks], s, 0, 0, 0);
        const int jl = j0 + 16 * hh;                 // key of register 0 of this lane
        float x[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float t = s[v] * c_scale;
            if constexpr (BIAS == BIAS_T5) t += t5s[r32 * kT5Buckets + t5_bucket(jl + v - my_pos)];
            if constexpr (BIAS == BIAS_T5U) t += t5s[r32 * kT5Buckets + t5u_bucket(jl + v - my_pos)];
            if constexpr (BIAS == BIAS_ALIBI) t -= aslope * fabsf((float)(jl + v - my_pos));
            if constexpr (FB) {
                const int j = jl + v;
                t = fmaf((row_ok && j < Sk) ? bf16_to_f32(fbrow[j]) : 0.f, kLog2e, t);
            }
            x[v] = t;
        }
        bool mneed = !uniform(p.rows >= 32 * rb + 32) || (j0 + 32 > Sk);
        if constexpr (MASK != MASK_NONE) mneed = mneed || (j0 + 31 > pmin);
        if constexpr (MASK == MASK_SLIDING) mneed = mneed || (j0 <= pmax - p.window);
        if (uniform(mneed)) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int j = jl + v;
                bool vis = row_ok & (j < Sk);
                if constexpr (MASK != MASK_NONE) vis = vis & (j <= my_pos);
                if constexpr (MASK == MASK_SLIDING) vis = vis & (my_pos - j < p.window);
                x[v] = vis ? x[v] : -INFINITY;
            }
        }
        float mx = x[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, x[v]);
        const float m_new = fmaxf(m, partner_max(mx));
        const float mref = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - mref);
        float ps = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            x[v] = __builtin_amdgcn_exp2f(x[v] - mref);
            ps += x[v];
        }
        l = fmaf(l, alpha, ps);
        m = m_new;
#pragma unroll
        for (int db = 0; db < DH; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
        // O^T += V^T P^T over the two 16-key groups of this half, head-dim fragments of half dh
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
            u32x4 pk;
#pragma unroll
            for (int c = 0; c < 4; ++c) pk[c] = pack_bf16x2(x[8 * sg + 2 * c], x[8 * sg + 2 * c + 1]);
            bf16x8 vt[DB];
            read_tr<D>(vb, 2 * kh + sg, lane, vt);
            if (!ONE || dh == 0) {
#pragma unroll
                for (int db = 0; db < DH; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((!ONE && dh) ? vt[DH + db] : vt[db],
                                                                      __builtin_bit_cast(bf16x8, pk), acc[db], 0, 0, 0);
            }
        }
    };

    // Ring of kNS tiles, F = kNS - 1 in flight: tile u + F is requested while tile u is
    // computed, and each iteration waits only for tile u + 1 (the DMA requests of the younger
    // tiles, 2 * XPW per tile and wave, may stay outstanding).
    constexpr int F = kNS - 1;
    static_assert(F >= 1 && F <= 3, "tiles in flight");
    constexpr int PT = 2 * XPW;                      // DMA requests per tile and wave
    auto wait_tile = [&](int younger) {              // younger tiles still allowed in flight
        if (younger >= 2) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * PT) : "memory");
        else if (younger == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(PT) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };
    for (int u = 0; u < F; ++u)
        if (u < nt) dma_tile(u);
    wait_tile(min(nt, F) - 1);
    __syncthreads();
#pragma unroll 1
    for (int u = 0; u < nt; ++u) {
        if (u + F < nt) dma_tile(u + F);
        compute(u);
        wait_tile(min(nt - 1, u + F) - (u + 1));
        __syncthreads();
    }

    // combine the two key halves in order (LDS of the ring is free after the last barrier):
    // waves (0, dh) and (1, dh) hold the same head dims for key halves 0 and 1
    float* obuf = (float*)smem;                      // [wave][row][D], half of D used per wave
    float* mbuf = obuf + kWaves * 32 * D;            // [key half][row]
    float* lbuf = mbuf + 2 * 32;                     // [key half][row]
    static_assert((kWaves * 32 * D + 4 * 32) * 4 <= sizeof(smem), "merge buffer");
    {
        const float l_row = partner_sum(l);
        float* orow = obuf + (wave * 32 + r32) * D;
#pragma unroll
        for (int q = 0; q < ((!ONE || dh == 0) ? DH : 0); ++q) {
            const int db = dh * DH + q;
            const int d0[2] = {16 * db + 8 * hh, 16 * (db + DB) + 8 * hh};
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int hv = 0; hv < 2; ++hv) {
                    u32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(acc[q][8 * c + 4 * hv + e]);
                    *(u32x4*)(orow + d0[c] + 4 * hv) = w;
                }
        }
        if (hh == 0 && dh == 0) {
            mbuf[kh * 32 + r32] = m;
            lbuf[kh * 32 + r32] = l_row;
        }
    }
    __syncthreads();
    {
        const int row = tid >> 3, cc = tid & 7;      // 32 rows x 8 column chunks of D / 8
        const int c0 = cc * (D / 8);
        // fragment db holds the 16-dim blocks db and db + DB; waves with dh hold fragments
        // dh * DH .. dh * DH + DH - 1, so the chunk's 16-dim block picks the wave pair
        const int dhc = ((c0 / 16) % DB) / DH;
        const float m0 = mbuf[row], m1 = mbuf[32 + row];
        const float ms = fmaxf(m0, m1);
        const float w0 = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m0 - ms);
        const float w1 = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - ms);
        const float ls = fmaf(lbuf[32 + row], w1, lbuf[row] * w0);
        const float* o0 = obuf + ((2 * dhc + 0) * 32 + row) * D + c0;
        const float* o1 = obuf + ((2 * dhc + 1) * 32 + row) * D + c0;
        float o[D / 8];
#pragma unroll
        for (int c = 0; c < D / 8; ++c) o[c] = fmaf(o1[c], w1, o0[c] * w0);
        const int rg = 32 * rb + row;
        if (p.n_split == 1) {
            if (rg < p.rows)
                store_out<D, OUT_F32>(p, b, kvh, rg, c0, o, ls > 0.f ? 1.f / ls : 0.f,
                                      ls > 0.f ? (ms + __builtin_amdgcn_logf(ls)) * kLn2 : -INFINITY);
        } else if (rg < p.rows) {
            float* dst = ws_o + row * D + c0;
#pragma unroll
            for (int c = 0; c < D / 8; c += 4) {
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(o[c + e]);
                *(u32x4*)(dst + c) = w;
            }
            if (cc == 0) {
                ws_ml[2 * row] = ms;
                ws_ml[2 * row + 1] = ls;
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// combine the splits of each (batch, KV head, row block) in split order
// ------------------------------------------------------------------------------------------
// Each thread merges 4 consecutive columns of one row: a workgroup covers kMergeRows rows, and
// a 32-row block takes 32 / kMergeRows workgroups (enough of them to spread the reads).
template <int D>
constexpr int merge_rows() { return 256 / (D / 4); }

template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void merge_kernel(const DecParams p) {
    constexpr int TPR = D / 4;                      // threads per row
    constexpr int MR = merge_rows<D>();             // rows per workgroup
    constexpr int SUB = 32 / MR;                    // workgroups per 32-row block
    const int tid = threadIdx.x;
    const int row = (blockIdx.x % SUB) * MR + tid / TPR, c0 = 4 * (tid % TPR);
    const int blk = blockIdx.x / SUB;
    const int rb = blk % p.n_rb, group = blk / p.n_rb;
    const int b = group / p.Hkv, kvh = group - b * p.Hkv;
    const int rg = 32 * rb + row;
    if (rg >= p.rows) return;
    const size_t units = (size_t)p.B * p.Hkv * p.n_rb * p.n_split;
    const size_t unit0 = ((size_t)group * p.n_rb + rb) * p.n_split;
    const float* ml = p.ws + units * 32 * D + unit0 * 64 + 2 * row;
    const float* src0 = p.ws + unit0 * 32 * D + row * D + c0;
    // Both passes run in split order. The partial results were written by workgroups on other
    // XCDs (far away), so the loads of U splits are issued together before they are combined;
    // the arithmetic, and so every bit of the result, is that of the plain loop.
    const int ns = p.n_split;
    float ms = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < ns; ++s) ms = fmaxf(ms, ml[64 * s]);
    float ls = 0.f;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    auto combine = [&](float2 m_l, u32x4 v) {
        float w = __builtin_amdgcn_exp2f(m_l.x - ms);
        w = (ms == -INFINITY) ? 0.f : w;
        ls = fmaf(m_l.y, w, ls);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fmaf(__uint_as_float(v[e]), w, o[e]);
    };
    constexpr int U = 8;
    int s = 0;
    for (; s + U <= ns; s += U) {
        float2 m_l[U];
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            m_l[u] = *(const float2*)(ml + 64 * (s + u));
            v[u] = *(const u32x4*)(src0 + (size_t)(s + u) * 32 * D);
        }
        __builtin_amdgcn_sched_barrier(0);   // every load of the batch is issued before any use
#pragma unroll
        for (int u = 0; u < U; ++u) combine(m_l[u], v[u]);
    }
    if (s < ns) {                            // the last, partial batch, loaded the same way
        float2 m_l[U];
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int su = min(s + u, ns - 1);   // past the end: re-read the last split, unused
            m_l[u] = *(const float2*)(ml + 64 * su);
            v[u] = *(const u32x4*)(src0 + (size_t)su * 32 * D);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (s + u < ns) combine(m_l[u], v[u]);
    }
    // store the 4 columns (and, from column 0, the row's log-sum-exp)
    const float mul = ls > 0.f ? 1.f / ls : 0.f;
    const int i = rg / p.G, hq = kvh * p.G + (rg - i * p.G);
    const size_t orow = ((size_t)b * p.Sq + i) * p.Hq + hq;
    if constexpr (OUT_F32) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(o[e] * mul);
        *(u32x4*)((float*)p.out + orow * D + c0) = w;
    } else {
        u32x2 w;
        w[0] = pack_bf16x2(o[0] * mul, o[1] * mul);
        w[1] = pack_bf16x2(o[2] * mul, o[3] * mul);
        *(u32x2*)((uint16_t*)p.out + orow * D + c0) = w;
    }
    if (c0 == 0)
        p.lse[((size_t)b * p.Hq + hq) * p.Sq + i] = ls > 0.f ? (ms + __builtin_amdgcn_logf(ls)) * kLn2 : -INFINITY;
}

// 64-key tiles per split of the last row block (under a causal mask the widest key range), as
// split_kernel cuts them
template <int MASK>
static int tiles_per_split(const DecParams& p) {
    const int rb = p.n_rb - 1;
    const int pmin = (32 * rb) / p.G + p.off, pmax = (p.rows - 1) / p.G + p.off;
    int klo = 0, khi = p.Sk - 1;
    if (MASK != MASK_NONE) khi = khi < pmax ? khi : pmax;
    if (MASK == MASK_SLIDING) klo = pmin - p.window + 1 > 0 ? pmin - p.window + 1 : 0;
    const int n_t = (khi < klo) ? 0 : khi / kBN - klo / kBN + 1;
    return (n_t + p.n_split - 1) / p.n_split;
}

template <int D, int MASK, int BIAS, bool OUT_F32>
static hipError_t launch_one(const DecParams& p, hipStream_t s) {
    const unsigned grid = (unsigned)((size_t)p.B * p.Hkv * p.n_rb * p.n_split);
    // D = 128: splits of up to 32 tiles take the 2-slot ring (two workgroups per CU; measured
    // +7 % on MQA decode, +12 % with a 4096-key window, at 16 tiles per split), longer ones
    // the 4-slot ring (three tiles in flight; +5 % at 128 tiles per split). The ring depth does
    // not change the arithmetic: the results are the same bits either way.
    if (D == 128 && tiles_per_split<MASK>(p) <= 32)
        hipLaunchKernelGGL((split_kernel<D, MASK, BIAS, OUT_F32, 2>), dim3(grid), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((split_kernel<D, MASK, BIAS, OUT_F32, ring_slots<D>()>), dim3(grid), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_split == 1) return e;
    const unsigned gm = (unsigned)((size_t)p.B * p.Hkv * p.n_rb * (32 / merge_rows<D>()));
    hipLaunchKernelGGL((merge_kernel<D, OUT_F32>), dim3(gm), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <int D, bool OUT_F32>
static hipError_t launch_d(const DecParams& p, int mask, int bias, hipStream_t s) {
#define SDPA_CASE(M, Bk) \
    if (mask == M && bias == Bk) return launch_one<D, M, Bk, OUT_F32>(p, s);
    SDPA_CASE(MASK_NONE, BIAS_NONE) SDPA_CASE(MASK_NONE, BIAS_T5) SDPA_CASE(MASK_NONE, BIAS_FULL)
    SDPA_CASE(MASK_CAUSAL, BIAS_NONE) SDPA_CASE(MASK_CAUSAL, BIAS_T5) SDPA_CASE(MASK_CAUSAL, BIAS_FULL)
    SDPA_CASE(MASK_SLIDING, BIAS_NONE) SDPA_CASE(MASK_SLIDING, BIAS_T5) SDPA_CASE(MASK_SLIDING, BIAS_FULL)
    SDPA_CASE(MASK_NONE, BIAS_ALIBI) SDPA_CASE(MASK_CAUSAL, BIAS_ALIBI) SDPA_CASE(MASK_SLIDING, BIAS_ALIBI)
    SDPA_CASE(MASK_NONE, BIAS_T5U) SDPA_CASE(MASK_CAUSAL, BIAS_T5U) SDPA_CASE(MASK_SLIDING, BIAS_T5U)
#undef SDPA_CASE
    return hipErrorInvalidValue;
}

}  // namespace dec

// Partial results of the no-allocation decode entry point (callers that cannot allocate: HIP
// graph capture, serving loops). Each GPU the library runs on holds its own copy until the
// process ends. It lives in this file, with the kernels that use it, so that it belongs to a
// code object the runtime loads for those kernels. In host code the name is only a stand-in
// for the symbol: kernels get the device address that decode_scratch returns.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

// The device address of `scratch` on the current device, resolved with hipGetSymbolAddress on
// the first call there and kept per device.
hipError_t decode_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        fprintf(stderr, "sdpa: current device not found (device %d): %s\n", dev,
                hipGetErrorString(e));
        return e != hipSuccess ? e : hipErrorInvalidDevice;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !a) {
            fprintf(stderr, "sdpa: scratch of device %d not resolved: %s\n", dev,
                    hipGetErrorString(e));
            return e != hipSuccess ? e : hipErrorInvalidSymbol;
        }
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_decode_bf16(DecParams p, int D, int mask, int bias, bool out_f32, hipStream_t s) {
    p.rows = p.G * p.Sq;
    p.n_rb = dec_row_blocks(p.G, p.Sq);
    p.n_split = dec_splits(p.B, p.Hkv, p.G, p.Sq, p.Sk);
    if (D == 256)
        return out_f32 ? dec::launch_d<256, true>(p, mask, bias, s) : dec::launch_d<256, false>(p, mask, bias, s);
    if (D == 128)
        return out_f32 ? dec::launch_d<128, true>(p, mask, bias, s) : dec::launch_d<128, false>(p, mask, bias, s);
    if (D == 64)
        return out_f32 ? dec::launch_d<64, true>(p, mask, bias, s) : dec::launch_d<64, false>(p, mask, bias, s);
    if (D == 32)
        return out_f32 ? dec::launch_d<32, true>(p, mask, bias, s) : dec::launch_d<32, false>(p, mask, bias, s);
    return hipErrorInvalidValue;
}

}  // namespace sdpa
