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
//   * keys are visited in tiles of 64, ascending; K and V tiles are staged row-major
//     ([key][d], XOR-swizzled 16-byte chunks) in a 2-deep LDS ring, the next tile's global
//     loads in flight while the current one is computed;
//   * scores are computed transposed, S^T = K . Q^T, with v_mfma_f32_32x32x16_bf16: each lane
//     then holds one query row (lane % 32) and 32 of the tile's keys, so the row max/sum are
//     in-lane plus one permlane32 exchange with the lane holding the other 32 keys;
//   * O^T += V^T . P^T with the same MFMA; the V^T operand comes from the row-major V tile
//     through ds_read_b64_tr_b16 (transposing LDS read), P straight from the score registers
//     (bf16, nearest even) as the B operand, so P never leaves the lane;
//   * online softmax in the log2 domain with a lazy rescale: the running reference max only
//     moves (and O is only rescaled) when a row's max grows by more than 2^8;
//   * interior tiles (no key masked for any row of the wave) run a separate code path with no
//     per-element mask work; scale*log2(e) is folded into the exponent's FMA.
// Reduction order is fixed (ascending key tiles, fixed MFMA chains, no atomics): results are
// bitwise reproducible run to run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sdpa_params.h"

namespace sdpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

#ifndef SDPA_PRIO
#define SDPA_PRIO 1
#endif
#ifndef SDPA_VMAP
#define SDPA_VMAP 1
#endif
#ifndef SDPA_DMA
#define SDPA_DMA 1
#endif
#ifndef SDPA_WAVES
#define SDPA_WAVES 8
#endif
constexpr int kThreads = 64 * SDPA_WAVES;
constexpr int kBM = 32 * SDPA_WAVES;    // query rows per workgroup
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

// LDS bank swizzles: XOR on the 16-byte chunk index within a row of the K or V tile.
// K (read by ds_read_b128, 8 lanes on rows {0..3, 16..19} + 4g): D=128 rows are 16 chunks,
// D=64 rows are 8 chunks.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
    if constexpr (D == 128) {
        return (row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3);
    } else {
        return ((row & 3) ^ ((row >> 2) & 1)) | (((row >> 4) & 1) << 2);
    }
}
// V (read by ds_read_b64_tr_b16, a 16-lane group touching chunks {c, c+2} of 4 consecutive
// rows): rows 4k..4k+3 go to XOR patterns {0, 1, 4, 5}.
__device__ __forceinline__ int v_swz(int row) {
#if SDPA_VMAP
    return 2 * (row & 3);
#else
    return (row & 1) | ((row & 2) << 1);
#endif
}

__device__ __forceinline__ float partner_max(float x) {
    // max of this lane and lane l ^ 32 (the other half of the wave)
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float partner_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

template <int D, int MASK, int BIAS, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 8 / SDPA_WAVES) void sdpa_fwd_bf16_kernel(const FwdParams p) {
    constexpr int CH = D / 8;           // 16-byte chunks per K/V row
    constexpr int KS = D / 16;          // k-steps of Q.K^T
    constexpr int DB = D / 32;          // 32-wide d blocks of O^T
    constexpr int TILE = kBN * D;       // bf16 elements per K (or V) buffer
    constexpr int NST = kBN * CH / kThreads;   // staged 16-byte chunks per thread per tensor
    static_assert(NST * kThreads == kBN * CH, "staging");

    // Ring depth: 3 for the full-bias D = 64 kernel (the bias stream needs the latency
    // cover; 144 KB of LDS), 2 otherwise. Each stage holds K, V and, for a full bias, the
    // [256 rows][64 keys] bias tile.
    constexpr bool FB_LDS = SDPA_DMA && BIAS == BIAS_FULL;
    constexpr int NBUF = (FB_LDS && D == 64) ? 3 : 2;
    constexpr int BTILE = FB_LDS ? kBM * kBN : 0;      // bf16 elements of a bias buffer
    constexpr int STAGE = 2 * TILE + BTILE;
    __shared__ __attribute__((aligned(16))) uint16_t smem[NBUF * STAGE];
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
                constexpr int NV = OUT_F32 ? 4 : 2;
#pragma unroll
                for (int c = 0; c < NV; ++c)
                    *(u32x4*)(o + (d0 * (OUT_F32 ? 4 : 2)) + 16 * c) = u32x4{0, 0, 0, 0};
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
        const uint16_t* qr = qg + (size_t)(row_ok ? my_i : 0) * q_row + hh * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = *(const u32x4*)(qr + ks * 16);
            if (!row_ok) x = u32x4{0, 0, 0, 0};
            qf[ks] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // ---- global -> register -> LDS staging of one K/V tile ---------------------------------
    // Thread tid stages chunk c = tid % CH of rows tid / CH + i * (256 / CH), for K and V.
    // Rows past the end of the keys are clamped to the last key: those keys are masked.
    constexpr int ROW_STEP = kThreads / CH;
    const int st_c = tid % CH, st_r = tid / CH;
    uint32_t st_off[NST];      // element offset of this thread's chunks inside a key tile
#pragma unroll
    for (int i = 0; i < NST; ++i) st_off[i] = (uint32_t)((st_r + i * ROW_STEP) * p.Hkv * D + st_c * 8);
    u32x4 stk[NST], stv[NST];
    auto load_tile = [&](int t) {
        const int j0 = t * kBN;
        const uint16_t* kt = kg + (size_t)j0 * kv_row;
        const uint16_t* vt = vg + (size_t)j0 * kv_row;
        if (j0 + kBN <= Sk) {
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                stk[i] = *(const u32x4*)(kt + st_off[i]);
                stv[i] = *(const u32x4*)(vt + st_off[i]);
            }
        } else {
            // last, partial tile: rows past the end are clamped to the last key (masked)
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                const int j = min(j0 + st_r + i * ROW_STEP, Sk - 1);
                const size_t o = (size_t)j * kv_row + st_c * 8;
                stk[i] = *(const u32x4*)(kg + o);
                stv[i] = *(const u32x4*)(vg + o);
            }
        }
    };
    // LDS-DMA staging: each wave issues 1 KB global_load_lds_dwordx4 transfers (lane i lands at
    // M0 + 16 i). Lane i of a transfer fetches the global chunk whose swizzled LDS slot is
    // 16 i, so the XOR layout is produced on the global side. Issued through inline asm: the
    // compiler would otherwise wait for every outstanding DMA before any LDS read. The waits
    // are explicit: vmcnt(0) before the barrier that publishes the tile.
    constexpr int ROWS_PER_XFER = 1024 / (D * 2);              // rows of one 1 KB transfer
    constexpr int XFERS = (kBN * D * 2) / 1024;                // per tensor per tile
    constexpr int XPW = XFERS / (kThreads / 64);               // per wave per tensor
    static_assert(XPW * (kThreads / 64) == XFERS, "dma split");
    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)smem);
    // full bias through the LDS ring when rows split into whole 16-byte chunks
    constexpr int XPB = FB_LDS ? (kBM * kBN * 2 / 1024) / (kThreads / 64) : 0;
    const bool fb_dma = FB_LDS && ((Sk & 7) == 0);
    const uint16_t* fbg = (BIAS == BIAS_FULL)
        ? (const uint16_t*)p.bias + ((size_t)b * p.Hq + hq) * (size_t)Sq * Sk : nullptr;
    auto dma_tile = [&](int t, int buf) {
        const int j0 = t * kBN;
#pragma unroll
        for (int n = 0; n < XPW; ++n) {
            const int xi = wave * XPW + n;                      // transfer index in the tile
            const int row = xi * ROWS_PER_XFER + lane / CH;     // tile row this lane fills
            const int pc = lane % CH;                           // physical chunk in the row
            const int j = min(j0 + row, Sk - 1);
            const uint16_t* ksrc = kg + (size_t)j * kv_row + ((pc ^ k_swz<D>(row)) * 8);
            const uint16_t* vsrc = vg + (size_t)j * kv_row + ((pc ^ v_swz(row)) * 8);
            const uint32_t kdst = __builtin_amdgcn_readfirstlane(
                lds_base + (uint32_t)((buf * STAGE) * 2 + xi * 1024));
            const uint32_t vdst = kdst + (uint32_t)(TILE * 2);
            asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                         :: "v"(ksrc), "s"(kdst) : "memory");
            asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                         :: "v"(vsrc), "s"(vdst) : "memory");
        }
        if constexpr (FB_LDS) {
            if (fb_dma) {
                // bias tile [kBM rows][kBN keys], 128-byte rows, chunk swizzle (row >> 1) & 7;
                // keys past the end of a partial last tile re-read the last whole chunk
                const int nchunk = min(kBN, Sk - j0) / 8;
#pragma unroll
                for (int n = 0; n < XPB; ++n) {
                    const int xi = wave * XPB + n;
                    const int row = xi * 8 + (lane >> 3);
                    const int c = min((lane & 7) ^ ((row >> 1) & 7), nchunk - 1);
                    const uint16_t* bsrc = fbg + (size_t)min(q0 + row, Sq - 1) * Sk + j0 + 8 * c;
                    const uint32_t bdst = __builtin_amdgcn_readfirstlane(
                        lds_base + (uint32_t)((buf * STAGE + 2 * TILE) * 2 + xi * 1024));
                    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                                 :: "v"(bsrc), "s"(bdst) : "memory");
                }
            }
        }
    };
    auto dma_wait = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
    // wait until at most this wave's transfers of one tile are still in flight
    // wait until at most one tile's transfers of this wave are still in flight
    auto dma_wait_one_behind = [&]() {
        static_assert(2 * XPW + XPB <= 63, "vmcnt field");
        if (fb_dma)
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * XPW + XPB) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * XPW) : "memory");
    };

    auto store_tile = [&](int buf) {
        uint16_t* kb = smem + buf * STAGE;
        uint16_t* vb = kb + TILE;
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const int row = st_r + i * ROW_STEP;
            *(u32x4*)(kb + row * D + ((st_c ^ k_swz<D>(row)) * 8)) = stk[i];
            *(u32x4*)(vb + row * D + ((st_c ^ v_swz(row)) * 8)) = stv[i];
        }
    };

    // ---- per-lane LDS read offsets (bf16 elements) -----------------------------------------
    // K: A operand row (lane % 32) -> key perm32(r32) (+32 for the second key block).
    const int krow = perm32(r32);
    const int k_sw = k_swz<D>(krow);          // identical for krow + 32
    // V^T via transposing reads: within 16-lane group gg = lane / 16, source lane i = lane % 16
    // points at key 16*hh + (i >> 2) (+ 32 jb + 8 s + 4 half) and head dims
    // 32 db + 16 (a & 1) + 8 (gg & 1) + 4 (a >> 1) .. +3 with a = i & 3; the read hands lane
    // (gg, a, c) the 4 keys of head dim 32 db + perm32(16 (gg & 1) + 4 a + c).
    const int gg = lane >> 4, li = lane & 15, la = li & 3;
    const int v_key = 16 * hh + (li >> 2);
#if SDPA_VMAP
    // rows 0..15 of the O^T MFMA for block db hold head dims 16 db + sigma, rows 16..31 hold
    // 16 (db + DB) + sigma: the two 16-lane halves of a transposing read touch opposite
    // 128-byte halves of the LDS banks.
    const int v_dlo = 16 * DB * (gg & 1) + 8 * (la & 1) + 4 * (la >> 1);
#else
    const int v_dlo = 16 * (la & 1) + 8 * (gg & 1) + 4 * (la >> 1);   // within a 32-d block
#endif
    const int v_sw = v_swz(v_key);                                     // same for key + 4n

    f32x16 o_acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o_acc[db][v] = 0.f;
    float m_ref = -INFINITY;     // reference max (log2 units) of this lane's row
    float l_part = 0.f;          // sum of p over this lane's keys, relative to m_ref

    // The tile loop assumes a positive scale. A negative scale flips the sign of the Q
    // fragment and of the scale together (exact in bf16, same products); a zero scale uses the
    // smallest normal float instead (the exponents change by < 1e-35).
    float c_scale = p.scale_log2;
    if (c_scale < 0.f) {
        c_scale = -c_scale;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, qf[ks]) ^ 0x80008000u);
    } else if (c_scale == 0.f) {
        c_scale = 1.17549435e-38f;
    }

    // One key tile for this wave. MASKED: apply per-key masks (edge tiles only).
    auto compute_tile = [&](auto masked_tag, int buf, int j0) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const uint16_t* kb = smem + buf * STAGE;
        const uint16_t* vb = kb + TILE;

        // full bias: issue this tile's bias loads first (consumed after the MFMAs)
        u32x4 fb[4];
        const uint16_t* br = nullptr;
        const int jl = j0 + 16 * hh;   // key of register 0 of this lane
        bool fb_vec = false;
        if constexpr (BIAS == BIAS_FULL) {
            br = (const uint16_t*)p.bias +
                 (((size_t)b * p.Hq + hq) * Sq + (row_ok ? my_i : 0)) * (size_t)Sk;
            fb_vec = (j0 + kBN <= Sk) && ((Sk & 7) == 0);
            if (fb_dma) {
                // this tile's bias rows from the LDS ring: row (wave*32 + r32), chunks
                // 4 jb + 2 hh + {0, 1}
                fb_vec = true;
                const int ir = wave * 32 + r32;
                const uint16_t* bt = smem + buf * STAGE + 2 * TILE + ir * kBN;
                const int sw = (ir >> 1) & 7;
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    fb[2 * jb] = *(const u32x4*)(bt + (((4 * jb + 2 * hh) ^ sw) * 8));
                    fb[2 * jb + 1] = *(const u32x4*)(bt + (((4 * jb + 2 * hh + 1) ^ sw) * 8));
                }
            } else if (fb_vec) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    fb[2 * jb] = *(const u32x4*)(br + jl + 32 * jb);
                    fb[2 * jb + 1] = *(const u32x4*)(br + jl + 32 * jb + 8);
                }
            }
        }

        // ---- S^T = K . Q^T (two 32-key blocks) ----
        f32x16 s0, s1;
#pragma unroll
        for (int v = 0; v < 16; ++v) { s0[v] = 0.f; s1[v] = 0.f; }
        // K fragments are read two k-steps ahead of their MFMAs; the scheduling barriers
        // keep the compiler from hoisting all of them (64 VGPRs) to the top.
        bf16x8 ka[2][2];
        auto read_k = [&](int ks, bf16x8* dst) {
            const int ch = ((2 * ks + hh) ^ k_sw) * 8;
            dst[0] = *(const bf16x8*)(kb + krow * D + ch);
            dst[1] = *(const bf16x8*)(kb + (krow + 32) * D + ch);
        };
        read_k(0, ka[0]);
        read_k(1, ka[1]);
#if SDPA_PRIO
        __builtin_amdgcn_s_setprio(1);
#endif
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a0 = ka[ks & 1][0], a1 = ka[ks & 1][1];
            if (ks + 2 < KS) read_k(ks + 2, ka[ks & 1]);
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], s1, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#if SDPA_PRIO
        __builtin_amdgcn_s_setprio(0);
#endif
        // V^T fragments of key group g = (jb, s): 4 keys from each of two transposing reads
        bf16x8 vfr[2][DB];
        auto read_v = [&](int g, bf16x8* dst) {
            const int key = v_key + 32 * (g >> 1) + 8 * (g & 1);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#if SDPA_VMAP
                const int d = 16 * db + v_dlo;
#else
                const int d = 32 * db + v_dlo;
#endif
                const int coff = (((d >> 3) ^ v_sw) << 3) + (d & 7);
                const s16x4 lo = lds_read_tr(vb + key * D + coff);
                const s16x4 hi = lds_read_tr(vb + (key + 4) * D + coff);
                u32x4 av;
                av[0] = __builtin_bit_cast(u32x2, lo)[0];
                av[1] = __builtin_bit_cast(u32x2, lo)[1];
                av[2] = __builtin_bit_cast(u32x2, hi)[0];
                av[3] = __builtin_bit_cast(u32x2, hi)[1];
                dst[db] = __builtin_bit_cast(bf16x8, av);
            }
        };
        read_v(0, vfr[0]);
        float x[32];    // x[16*jb + v] belongs to key jl + 32*jb + v
#pragma unroll
        for (int v = 0; v < 16; ++v) { x[v] = s0[v]; x[16 + v] = s1[v]; }

        // Visible keys of this lane's row form one interval [lo, hi]; register e of key block
        // jb holds key jl + 32 jb + (e & 15), so visibility is a compare of the compile-time
        // index e & 15 against per-lane bounds.
        int vis_hi[2], vis_lo[2];
        if constexpr (MASKED) {
            int hi = Sk - 1;
            if constexpr (MASK != MASK_NONE) hi = min(hi, my_pos);
            int lo = 0;
            if constexpr (MASK == MASK_SLIDING) lo = max(0, my_pos - p.window + 1);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                vis_hi[jb] = hi - (jl + 32 * jb);
                vis_lo[jb] = lo - (jl + 32 * jb);
            }
        }
        auto visible = [&](int e) {
            const int v = e & 15, jb = e >> 4;
            bool vis = v <= vis_hi[jb];
            if constexpr (MASK == MASK_SLIDING) vis = vis && (v >= vis_lo[jb]);
            return vis;
        };

        // Per-element path: full bias, or T5 near the diagonal. Otherwise
        // the bias is constant over the tile (none, or T5 far from the diagonal) and the scale
        // is folded into the exponent's FMA after a max over the raw scores.
        bool per_elem = (BIAS == BIAS_FULL);
        bool t5_near = false;
        float bconst = 0.f;
        if constexpr (BIAS == BIAS_T5) {
            const int rmin = j0 - pwb, rmax = j0 + kBN - 1 - pwa;
            if (rmin >= kT5Sat) bconst = t5s[2 * kT5Sat];
            else if (rmax <= -kT5Sat) bconst = t5s[0];
            else t5_near = per_elem = true;
        }

        float mt;     // row max of the log2-domain scores of this tile
        if (per_elem) {
            if constexpr (BIAS == BIAS_T5) {
                if (t5_near) {
                    const int rel0 = jl - my_pos;
#pragma unroll
                    for (int e = 0; e < 32; ++e) {
                        const int rel = rel0 + (e >> 4) * 32 + (e & 15);
                        const int idx = min(max(rel, -kT5Sat), kT5Sat) + kT5Sat;
                        x[e] = fmaf(x[e], c_scale, t5s[idx]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 32; ++e) x[e] = fmaf(x[e], c_scale, bconst);
                }
            } else if constexpr (BIAS == BIAS_FULL) {
                if (fb_vec) {
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                        for (int c = 0; c < 4; ++c)
#pragma unroll
                            for (int hv = 0; hv < 2; ++hv) {
                                const uint32_t lo = fb[2 * jb][c], hi = fb[2 * jb + 1][c];
                                const int e0 = 16 * jb + 2 * c + hv;
                                x[e0] = fmaf(x[e0], c_scale,
                                             bf16_to_f32(hv ? (lo >> 16) : (lo & 0xffffu)) * kLog2e);
                                x[e0 + 8] = fmaf(x[e0 + 8], c_scale,
                                                 bf16_to_f32(hv ? (hi >> 16) : (hi & 0xffffu)) * kLog2e);
                            }
                } else {
#pragma unroll
                    for (int e = 0; e < 32; ++e) {
                        const int j = jl + (e >> 4) * 32 + (e & 15);
                        const float bv = (row_ok && j < Sk) ? bf16_to_f32(br[j]) : 0.f;
                        x[e] = fmaf(x[e], c_scale, bv * kLog2e);
                    }
                }
            }
            if constexpr (MASKED) {
#pragma unroll
                for (int e = 0; e < 32; ++e) x[e] = visible(e) ? x[e] : -INFINITY;
            }
            mt = x[0];
#pragma unroll
            for (int e = 1; e < 32; ++e) mt = fmaxf(mt, x[e]);
            mt = partner_max(mt);
        } else {
            // max over the raw scores (scale > 0); hidden keys stay -inf through the FMA below
            if constexpr (MASKED) {
#pragma unroll
                for (int e = 0; e < 32; ++e) x[e] = visible(e) ? x[e] : -INFINITY;
            }
            float ext = x[0];
#pragma unroll
            for (int e = 1; e < 32; ++e) ext = fmaxf(ext, x[e]);
            ext = partner_max(ext);
            mt = (ext == -INFINITY) ? -INFINITY : fmaf(ext, c_scale, bconst);
        }

        // ---- online softmax (log2 domain, lazy rescale) ----
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
        if (per_elem) {
#pragma unroll
            for (int e = 0; e < 32; ++e) x[e] = __builtin_amdgcn_exp2f(x[e] - m_use);
        } else {
            const float nb = bconst - m_use;
#pragma unroll
            for (int e = 0; e < 32; ++e) x[e] = __builtin_amdgcn_exp2f(fmaf(x[e], c_scale, nb));
        }

        // ---- O^T += V^T . P^T ----
        // Four key groups g = (jb, s) of 8 keys per lane half; the V^T fragments of group g+1
        // are read while the MFMAs of group g run (group 0 was read before the softmax).
#if SDPA_PRIO
        __builtin_amdgcn_s_setprio(1);
#endif
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int jb = g >> 1, s = g & 1;
            u32x4 pk;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                pk[c] = pack_bf16x2(x[16 * jb + 8 * s + 2 * c], x[16 * jb + 8 * s + 2 * c + 1]);
                l_part += x[16 * jb + 8 * s + 2 * c] + x[16 * jb + 8 * s + 2 * c + 1];
            }
            const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
            if (g + 1 < 4) read_v(g + 1, vfr[(g + 1) & 1]);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[g & 1][db], pb, o_acc[db], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
#if SDPA_PRIO
        __builtin_amdgcn_s_setprio(0);
#endif
    };

    // wave-level classification of tile t and its computation on ring buffer `buf`
    auto run_tile = [&](int t, int buf) {
        const int j0 = t * kBN;
        bool skip = !wave_ok;
        if constexpr (MASK != MASK_NONE) skip = skip || (j0 > pwb);
        if constexpr (MASK == MASK_SLIDING) skip = skip || (j0 + kBN - 1 <= pwa - p.window);
        bool need_mask = (j0 + kBN > Sk);
        if constexpr (MASK != MASK_NONE) need_mask = need_mask || (j0 + kBN - 1 > pwa);
        if constexpr (MASK == MASK_SLIDING) need_mask = need_mask || (j0 <= pwb - p.window);
        if (!skip) {
            if (need_mask)
                compute_tile(std::true_type{}, buf, j0);
            else
                compute_tile(std::false_type{}, buf, j0);
        }
    };

#if SDPA_DMA
    if constexpr (NBUF == 2) {
        // tile t+1 is fetched while tile t is computed
        dma_tile(t_begin, 0);
        dma_wait();
        __syncthreads();
#pragma unroll 1
        for (int t = t_begin; t < t_end; ++t) {
            const int buf = (t - t_begin) & 1;
            const bool has_next = t + 1 < t_end;
            if (has_next) dma_tile(t + 1, buf ^ 1);
            run_tile(t, buf);
            if (has_next) dma_wait();
            __syncthreads();
        }
    } else {
        // tiles t+1 .. t+NBUF-1 in flight; the wait before each barrier leaves only the
        // transfers of tiles beyond the next one outstanding
        int fetch_t = t_begin, fetch_buf = 0;
        for (int n = 0; n < NBUF - 1 && fetch_t < t_end; ++n) {
            dma_tile(fetch_t, fetch_buf);
            ++fetch_t;
            fetch_buf = (fetch_buf + 1 == NBUF) ? 0 : fetch_buf + 1;
        }
        if (fetch_t > t_begin + 1) dma_wait_one_behind();
        else dma_wait();
        __syncthreads();
        int buf = 0;
#pragma unroll 1
        for (int t = t_begin; t < t_end; ++t) {
            const bool has_next = t + 1 < t_end;
            if (fetch_t < t_end) {
                dma_tile(fetch_t, fetch_buf);
                ++fetch_t;
                fetch_buf = (fetch_buf + 1 == NBUF) ? 0 : fetch_buf + 1;
            }
            run_tile(t, buf);
            if (has_next) {
                if (fetch_t > t + 2) dma_wait_one_behind();   // tile t+2 is also in flight
                else dma_wait();
            }
            buf = (buf + 1 == NBUF) ? 0 : buf + 1;
            __syncthreads();
        }
    }
#else
    load_tile(t_begin);
    store_tile(0);
    __syncthreads();
#pragma unroll 1
    for (int t = t_begin; t < t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        const bool has_next = t + 1 < t_end;
        if (has_next) load_tile(t + 1);
        run_tile(t, buf);
        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
    }
#endif

    // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l) ---------------------------------
    const float l_tot = partner_sum(l_part);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (row_ok) {
        char* o = out_ptr(my_i);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            // registers 8c .. 8c+7 of block db hold 8 consecutive head dims starting at d0[c]
#if SDPA_VMAP
            const int d0[2] = {16 * db + 8 * hh, 16 * (db + DB) + 8 * hh};
#else
            const int d0[2] = {32 * db + 16 * hh, 32 * db + 16 * hh + 8};
#endif
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                if constexpr (OUT_F32) {
#pragma unroll
                    for (int hv = 0; hv < 2; ++hv) {
                        u32x4 xo;
#pragma unroll
                        for (int e = 0; e < 4; ++e) xo[e] = __float_as_uint(o_acc[db][8 * c + 4 * hv + e] * inv);
                        *(u32x4*)(o + (d0[c] + 4 * hv) * 4) = xo;
                    }
                } else {
                    u32x4 xo;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        xo[e] = pack_bf16x2(o_acc[db][8 * c + 2 * e] * inv, o_acc[db][8 * c + 2 * e + 1] * inv);
                    *(u32x4*)(o + d0[c] * 2) = xo;
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
