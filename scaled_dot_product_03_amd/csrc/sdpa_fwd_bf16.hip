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
// Work decomposition (one work item = one query tile of one (batch, head), one workgroup per
// item or, for large launches, a persistent grid of one workgroup per CU walking the items;
// 32 query rows per wave; D = 64 and 128: 8 waves, two per SIMD (D = 64 with a full bias: 4
// waves, two workgroups per CU); D = 32: 4 waves, up to four workgroups per CU; D = 256: 4
// waves, one per SIMD, whose O accumulators need the whole register file):
//   * each wave owns 32 query rows; its Q fragment stays in VGPRs for the whole item;
//   * keys are visited in tiles of 64, ascending. K and V tiles are copied global -> LDS by
//     the DMA path of the load unit (global_load_lds_dwordx4) into a 2-slot K ring (a full
//     bias tile rides in the K slot) and a 2-slot V ring, stored row-major ([key][d]) with
//     XOR-swizzled 16-byte chunks; K runs one tile ahead of V;
//   * scores are computed transposed, S^T = K . Q^T, with v_mfma_f32_32x32x16_bf16: each lane
//     then holds one query row (lane % 32) and 32 of the tile's keys, so the row max/sum are
//     in-lane plus one permlane32 exchange with the lane holding the other 32 keys;
//   * O^T += V^T . P^T with the same MFMA; the V^T operand comes from the row-major V tile
//     through ds_read_b64_tr_b16 (transposing LDS read), P straight from the score registers
//     (bf16, nearest even) as the B operand, so P never leaves the lane;
//   * software pipeline inside each wave: iteration t runs the exponentials of tile t under
//     the S^T MFMAs of tile t+1 (phase A; a first batch of exponentials before the first MFMA,
//     while the first K fragments are read), then the P.V MFMAs of tile t under the bias, mask
//     and row max of tile t+1 (phase B), so the matrix cores are fed while the VALU works;
//   * online softmax in the log2 domain with a lazy rescale: the running reference max only
//     moves (and O is only rescaled) when a row's max grows by more than 2^8; scale*log2(e)
//     is folded into the exponent's FMA when the bias is constant over a tile. The row sum
//     adds the bf16-rounded weights that enter P.V (v_dot2_f32_bf16 against (1, 1)), so the
//     normaliser matches the numerator exactly (V = 1 gives O = 1).
// Reduction order is fixed (ascending key tiles, fixed MFMA chains, no atomics): results are
// bitwise reproducible run to run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
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


// waves per workgroup, and the waves per SIMD the register budget is sized for
template <int D, int BIAS> constexpr int waves_of() {
    return ((D == 64 && BIAS != BIAS_FULL) || D == 128) ? 8 : 4;
}
template <int D, int BIAS> constexpr int waves_per_eu_of() {
    return D == 256 ? 1 : ((D == 32 && BIAS != BIAS_FULL) ? 3 : 2);
}
template <int D, int BIAS> constexpr int rows_of() { return 32 * waves_of<D, BIAS>(); }   // query rows per workgroup
// Instances that take a persistent grid: dense, no full bias, D = 64 and 128 (not T5 at 128).
// The work loop costs ~15 VGPRs; the excluded instances would spill with it.
constexpr bool persist_ok(int D, int bias, bool varlen) {
    return !varlen && bias != BIAS_FULL &&
           (D == 64 || (D == 128 && bias != BIAS_T5 && bias != BIAS_T5U));
}
template <int D, int BIAS, bool VARLEN> constexpr bool persist_of() {
    return persist_ok(D, BIAS, VARLEN);
}
constexpr int kBN = 64;             // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;   // log2 units: p may reach 2^8 before O is rescaled

using True = std::true_type;
using False = std::false_type;

// Row permutation inside a 32-row MFMA operand: the A-operand row held by lane r = 8g+4h+t
// is taken from source row 16h+4g+t, so that output register v of a lane in half h holds
// row 16h+v (16 consecutive keys / head dims per lane instead of four runs of four).
__device__ __forceinline__ int perm32(int r) {
    return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3);
}

// LDS bank swizzles: XOR on the 16-byte chunk index within a row of the K or V tile.
// K (read by ds_read_b128, 8 lanes on rows {0..3, 16..19} + 4g): D=128 rows are 16 chunks
// (one full sweep of the 64 banks), D=256 rows two sweeps (the D=128 pattern on the low four
// bits of the chunk index), D=64 rows 8 chunks, D=32 rows 4 chunks (four rows per sweep).
template <int D>
__device__ __forceinline__ int k_swz(int row) {
    if constexpr (D >= 128) {
        return (row & 3) | (((row >> 4) & 1) << 2) | (((row >> 2) & 1) << 3);
    } else if constexpr (D == 64) {
        return ((row & 3) ^ ((row >> 2) & 1)) | (((row >> 4) & 1) << 2);
    } else {
        return ((row >> 2) & 1) | (((row >> 4) & 1) << 1);
    }
}
// V (read by ds_read_b64_tr_b16, a 16-lane group touching two adjacent chunks of 4
// consecutive rows): rows 4k..4k+3 go to XOR patterns {0, 2, 4, 6} ({0, 2} for the 4-chunk
// rows of D = 32). Depends on row & 3 only.
template <int D>
__device__ __forceinline__ int v_swz(int row) { return D == 32 ? 2 * (row & 1) : 2 * (row & 3); }

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

// Keeps a value's computation at this point of the program: the compiler would otherwise
// sink it to its first use and undo the interleaving of VALU work with MFMAs.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }


template <int D, int MASK, int BIAS, bool OUT_F32, bool VARLEN>
__global__ __launch_bounds__((64 * waves_of<D, BIAS>()), (waves_per_eu_of<D, BIAS>()))
void sdpa_fwd_bf16_kernel(const FwdParams p) {
    constexpr int kWaves = waves_of<D, BIAS>();
    constexpr int kThreads = 64 * kWaves;
    constexpr int kBM = rows_of<D, BIAS>();
    constexpr int CH = D / 8;           // 16-byte chunks per K/V row
    constexpr int KS = D / 16;          // k-steps of Q.K^T
    constexpr int DB = D / 32;          // 32-wide d blocks of O^T
    constexpr int TILE = kBN * D;       // bf16 elements per K (or V) tile

    // LDS: K ring (NKS slots, each a K tile followed, for a full bias, by the [256 rows][64 keys]
    // bias tile of the same keys), then the V ring (NVS slots).
    constexpr bool FB = BIAS == BIAS_FULL;
    // A full bias streams from HBM with the K tiles through the 2-slot K ring. At D = 64 the
    // workgroup has 4 waves (128 rows, 64 KB of LDS) so that two workgroups share a CU and
    // one computes while the other waits for its next bias tile. At D = 256 the K and V rings
    // fill the LDS: the bias is read from HBM by each lane instead.
    constexpr bool FB_LDS = FB && D != 256;
    constexpr int NKS = 2;
    constexpr int NVS = 2;
    constexpr int BTILE = FB_LDS ? kBM * kBN : 0;
    constexpr int KSTAGE = TILE + BTILE;
    constexpr int VRING = NKS * KSTAGE;
    static_assert((NKS * KSTAGE + NVS * TILE) * 2 <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(16))) uint16_t smem[NKS * KSTAGE + NVS * TILE];
    // T5 bias (bidirectional or decoder buckets) by relative position rel = key - query, log2
    // units, at t5s[kT5Pad + rel]. Padded so that every rel of a tile near the diagonal indexes
    // it without clamping: such a tile has j0 - pwb < kSat and j0 + 63 - pwa > -kSat, and
    // pwb - pwa <= 31, so |rel| < kT5Pad. Beyond +-kSat the bucket is constant.
    constexpr bool IS_T5 = BIAS == BIAS_T5 || BIAS == BIAS_T5U;
    constexpr bool ALIBI = BIAS == BIAS_ALIBI;
    constexpr bool ALIBI_LIN = ALIBI && MASK != MASK_NONE && D != 256;   // (D = 256: no registers to spare)
    constexpr int kSat = BIAS == BIAS_T5U ? kT5USat : kT5Sat;
    constexpr int kT5Pad = kSat + kBN + 31;
    __shared__ float t5s[IS_T5 ? 2 * kT5Pad + 1 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, r32 = lane & 31;

  // one work item = one query tile of one (batch, query head)
  auto run_item = [&](const int item) {
    const WorkItem w = decode_work(p, item);
    const int b = w.b, hq = w.hq, kvh = hq / p.G;
    int Sq = p.Sq, Sk = p.Sk, off = p.off;
    size_t q_base = (size_t)b * Sq, k_base = (size_t)b * Sk;   // first token of the sequence
    if constexpr (VARLEN) {
        // packed sequence b: its own lengths and alignment; offsets that leave the packed
        // buffers or exceed the launch's longest sequence make it empty
        const int qs = p.cu_q[b], qe = p.cu_q[b + 1], ks = p.cu_k[b], ke = p.cu_k[b + 1];
        const bool ok = 0 <= qs && qs <= qe && qe <= p.total_q && qe - qs <= p.Sq &&
                        0 <= ks && ks <= ke && ke <= p.total_k && ke - ks <= p.Sk;
        Sq = ok ? qe - qs : 0;
        Sk = ok ? ke - ks : 0;
        off = Sk - Sq;
        q_base = (size_t)(ok ? qs : 0);
        k_base = (size_t)(ok ? ks : 0);
    }
    const int q0 = w.qt * kBM;
    if constexpr (VARLEN) {
        if (q0 >= Sq) return;     // query tile past the end of a shorter sequence
    }

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
    const uint16_t* qg = (const uint16_t*)p.q + (q_base * p.Hq + hq) * D;
    const uint16_t* kg = (const uint16_t*)p.k + (k_base * p.Hkv + kvh) * D;
    const uint16_t* vg = (const uint16_t*)p.v + (k_base * p.Hkv + kvh) * D;

    const int wq0 = q0 + wave * 32;          // first query row of this wave
    const int my_i = wq0 + r32;              // query row of this lane
    const bool row_ok = my_i < Sq;
    const int my_pos = my_i + off;
    const bool wave_ok = wq0 < Sq;
    const int pwa = wq0 + off;
    const int pwb = min(wq0 + 31, Sq - 1) + off;

    float* lse_row = VARLEN ? p.lse + (size_t)hq * p.total_q + q_base
                            : p.lse + ((size_t)b * p.Hq + hq) * Sq;
    auto out_ptr = [&](int i) -> char* {
        const size_t e = (q_base + i) * q_row + (size_t)hq * D;
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
    if constexpr (IS_T5) {
        const float* tbl = (const float*)p.bias + (size_t)hq * kT5Buckets;
        for (int i = tid; i < 2 * kT5Pad + 1; i += kThreads)
            t5s[i] = tbl[BIAS == BIAS_T5U ? t5u_bucket(i - kT5Pad) : t5_bucket(i - kT5Pad)] * kLog2e;
    }
    // ALiBi: -slope * |p - j| in log2 units, slope of this head from the [Hq] table
    float aslope = 0.f;
    if constexpr (ALIBI) aslope = ((const float*)p.bias)[hq] * kLog2e;

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
    // the same positive scale in natural-log units (a full bias is added in those units)
    const float n_scale = (p.scale == 0.f) ? 1.17549435e-38f : fabsf(p.scale);
    // Under a causal or sliding mask no visible key follows its query, so the bias is
    // slope * (j - p): slope * (jl - p) per row and key block, folded into the row max and the
    // exponent's offset, plus slope * k for the key's offset k = 0..15 in the lane's run of 16
    // keys, added to the raw score as (slope / c) * k with the score scale c applied in the
    // exponent. c is floored at |slope| 2^-96 so that slope / c stays finite (only a zero or
    // vanishing softmax scale meets the floor; the scores then contribute below 2^-76 |slope|).
    const float al_c = ALIBI_LIN ? fmaxf(c_scale, fabsf(aslope) * 0x1p-96f) : 0.f;
    const float al_a = ALIBI_LIN ? aslope / al_c : 0.f;

    // ---- LDS-DMA staging -------------------------------------------------------------------
    // Each wave issues 1 KB global_load_lds_dwordx4 transfers (lane i lands at M0 + 16 i).
    // Lane i of a transfer fetches the global chunk whose swizzled LDS slot is 16 i, so the XOR
    // layout is produced on the global side. Rows past the end of the keys are clamped to the
    // last key (those keys are masked). Issued through inline asm: the compiler would otherwise
    // wait for every outstanding DMA before any LDS read. The waits are explicit: vmcnt(0)
    // before the barrier that publishes a tile.
    constexpr int ROWS_PER_XFER = 1024 / (D * 2);              // rows of one 1 KB transfer
    constexpr int XFERS = (kBN * D * 2) / 1024;                // per tensor per tile
    constexpr int XPW = XFERS / kWaves;                        // per wave per tensor
    static_assert(XPW * kWaves == XFERS, "dma split");
    constexpr int XPB = FB_LDS ? (kBM * kBN * 2 / 1024) / kWaves : 0;   // bias transfers per wave
    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint16_t*)smem);
    // a full bias goes through the LDS ring when its rows split into whole 16-byte chunks
    const bool fb_dma = FB_LDS && ((Sk & 7) == 0);
    const uint16_t* fbg = FB ? (const uint16_t*)p.bias + ((size_t)b * p.Hq + hq) * (size_t)Sq * Sk
                             : nullptr;
    auto kslot = [&](int t) { return (t - t_begin) % NKS; };
    auto vslot = [&](int t) { return (t - t_begin) % NVS; };
    auto kptr = [&](int t) { return smem + kslot(t) * KSTAGE; };
    auto vptr = [&](int t) { return smem + VRING + vslot(t) * TILE; };
    // M0 carries the LDS destination of each transfer; no other instruction of this kernel
    // reads M0.
    // K and V transfers use the scalar-base form: address = SGPR base of the tile + a 32-bit
    // per-lane byte offset that is the same for every full tile (row * Hkv * D * 2 < 2^32,
    // since Sk * Hkv * D < 2^31), so issuing one costs no vector instruction. In a partial last
    // tile, rows past the end of the keys are clamped to the last key (those keys are masked).
    const uint32_t kv_row_bytes = (uint32_t)(kv_row * 2);
    uint32_t k_off[XPW], v_off[XPW];
#pragma unroll
    for (int n = 0; n < XPW; ++n) {
        const int row = (wave * XPW + n) * ROWS_PER_XFER + lane / CH;   // tile row this lane fills
        k_off[n] = (uint32_t)row * kv_row_bytes + (uint32_t)((((lane % CH) ^ k_swz<D>(row))) * 16);
        v_off[n] = (uint32_t)row * kv_row_bytes + (uint32_t)((((lane % CH) ^ v_swz<D>(row))) * 16);
    }
    const uint32_t dma_wave_off = __builtin_amdgcn_readfirstlane((uint32_t)(wave * XPW * 1024));
    auto dma_kv_x = [&](const uint16_t* g, uint32_t off_full, bool vtile, uint32_t dst, int t, int n) {
        const int j0 = t * kBN;
        const uint16_t* base = g + (size_t)j0 * kv_row;
        uint32_t off = off_full;
        if (j0 + kBN > Sk) {
            const int row = (wave * XPW + n) * ROWS_PER_XFER + lane / CH;
            const int sw = vtile ? v_swz<D>(row) : k_swz<D>(row);
            base = g;
            off = (uint32_t)min(j0 + row, Sk - 1) * kv_row_bytes + (uint32_t)(((lane % CH) ^ sw) * 16);
        }
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                     :: "v"(off), "s"(base), "s"(dst) : "memory");
    };
    auto dma_k_x = [&](int t, int n) {     // K transfer n of tile t
        dma_kv_x(kg, k_off[n], false,
                 lds_base + (uint32_t)(kslot(t) * KSTAGE * 2 + n * 1024) + dma_wave_off, t, n);
    };
    auto dma_v_x = [&](int t, int n) {     // V transfer n of tile t
        dma_kv_x(vg, v_off[n], true,
                 lds_base + (uint32_t)((VRING + vslot(t) * TILE) * 2 + n * 1024) + dma_wave_off, t, n);
    };
    auto dma_b_x = [&](int t, int n) {     // full-bias transfer n of tile t
        if constexpr (FB_LDS) {
            if (fb_dma) {
                // bias tile [kBM rows][kBN keys], 128-byte rows, chunk swizzle (row >> 1) & 7;
                // keys past the end of a partial last tile re-read the last whole chunk
                const int j0 = t * kBN;
                const int nchunk = min(kBN, Sk - j0) / 8;
                const int xi = wave * XPB + n;
                const int row = xi * 8 + (lane >> 3);
                const int c = min((lane & 7) ^ ((row >> 1) & 7), nchunk - 1);
                const uint16_t* src = fbg + (size_t)min(q0 + row, Sq - 1) * Sk + j0 + 8 * c;
                const uint32_t dst = __builtin_amdgcn_readfirstlane(
                    lds_base + (uint32_t)(kslot(t) * KSTAGE * 2 + TILE * 2 + xi * 1024));
                asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                             :: "v"(src), "s"(dst) : "memory");
            }
        }
    };
    auto dma_k = [&](int t) {
#pragma unroll
        for (int n = 0; n < XPW; ++n) dma_k_x(t, n);
#pragma unroll
        for (int n = 0; n < XPB; ++n) dma_b_x(t, n);
    };
    auto dma_v = [&](int t) {
#pragma unroll
        for (int n = 0; n < XPW; ++n) dma_v_x(t, n);
    };
    // Transfers of one iteration (K and bias of tile t+2, V of tile t+1), numbered
    // 0 .. NXF-1; in a fused iteration they are issued one or two per k-step of phase A
    // instead of back to back.
    constexpr int NXF = 2 * XPW + XPB;
    // transfer i of iteration t: V(t+1) first, then K and bias of tile t + NKS
    auto dma_xfer = [&](int t, int i) {
        if (i < XPW) {
            dma_v_x(t + 1, i);
        } else if (i < 2 * XPW) {
            if (t + NKS < t_end) dma_k_x(t + NKS, i - XPW);
        } else {
            if (t + NKS < t_end) dma_b_x(t + NKS, i - 2 * XPW);
        }
    };
    auto dma_wait = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
    // with a 3-deep K ring: wait for everything but the K (and bias) transfers of tile u,
    // issued last, when tile u exists
    auto dma_wait_but_k = [&](int u) {
        if constexpr (NKS == 3) {
            if (u < t_end) {
                if (fb_dma) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(XPW + XPB) : "memory");
                else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(XPW) : "memory");
                return;
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    };

    // ---- per-lane LDS read offsets (bf16 elements) -----------------------------------------
    // K: A operand row (lane % 32) -> key perm32(r32) (+32 for the second key block).
    const int krow = perm32(r32);
    const int k_sw = k_swz<D>(krow);          // identical for krow + 32
    // V^T via transposing reads: within 16-lane group gg = lane / 16, source lane i = lane % 16
    // points at key 16*hh + (i >> 2) (+ 32 jb + 8 s + 4 half). Rows 0..15 of the O^T MFMA for
    // block db hold head dims 16 db + sigma, rows 16..31 hold 16 (db + DB) + sigma, so the two
    // 16-lane halves of a transposing read touch opposite 128-byte halves of the LDS banks.
    const int gg = lane >> 4, li = lane & 15, la = li & 3;
    const int v_key = 16 * hh + (li >> 2);
    const int v_dlo = 16 * DB * (gg & 1) + 8 * (la & 1) + 4 * (la >> 1);
    const int v_sw = v_swz<D>(v_key);         // same for key + 4n

    auto read_k = [&](const uint16_t* kb, int ks, bf16x8* dst) {
        const int ch = ((2 * ks + hh) ^ k_sw) * 8;
        dst[0] = *(const bf16x8*)(kb + krow * D + ch);
        dst[1] = *(const bf16x8*)(kb + (krow + 32) * D + ch);
    };
    // V^T fragments of key group g = (jb, s): 4 keys from each of two transposing reads
    auto read_v = [&](const uint16_t* vb, int g, bf16x8* dst) {
        const int key = v_key + 32 * (g >> 1) + 8 * (g & 1);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int d = 16 * db + v_dlo;
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

    // ---- wave-level tile classification ------------------------------------------------------
    auto active = [&](int t) {      // some key of tile t is visible to some row of the wave
        const int j0 = t * kBN;
        bool skip = !wave_ok;
        if constexpr (MASK != MASK_NONE) skip = skip || (j0 > pwb);
        if constexpr (MASK == MASK_SLIDING) skip = skip || (j0 + kBN - 1 <= pwa - p.window);
        return !skip;
    };
    auto needs_mask = [&](int t) {  // some key of tile t is hidden from some row of the wave
        const int j0 = t * kBN;
        bool m = (j0 + kBN > Sk);
        if constexpr (MASK != MASK_NONE) m = m || (j0 + kBN - 1 > pwa);
        if constexpr (MASK == MASK_SLIDING) m = m || (j0 <= pwb - p.window);
        return m;
    };

    // ---- softmax state ---------------------------------------------------------------------
    f32x16 o_acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o_acc[db][v] = 0.f;
    float m_ref = -INFINITY;     // reference max (log2 units) of this lane's row
    float l_part = 0.f;          // sum of p over this lane's keys, relative to m_ref
    // Prepared tile (the next one to exponentiate): row max in log2 units, and the exponent
    // p = exp2(x * cc + bc - m): cc = scale*log2(e), bc = constant bias for raw scores x, or
    // cc = 1, bc = 0 for scores already in the log2 domain (per-element bias).
    float mt_c = -INFINITY, cc_c = 0.f, bc_c = 0.f;
    // linear ALiBi: key block 1 of a lane starts 32 keys after block 0
    const float a32 = 32.f * aslope;
    constexpr int KPRE = 2;               // k-steps of K fragments read ahead of their MFMAs
    constexpr int VPRE = 1;               // key groups of V^T fragments read ahead
    bf16x8 vfr[VPRE + 1][DB];

    // Score registers: element e of a tile is ss[e >> 4][e & 15] and belongs to key
    // j0 + 16 hh + 32 (e >> 4) + (e & 15) of this lane's row.

    // Phase A: exponentials of the prepared tile in `cs` (DO_E) interleaved with the S^T MFMAs
    // of the next tile into `ns` (DO_S, K tile at kb). Ends with the first V^T fragments of
    // the tile in `cs` (V tile at vb) in flight.
    auto phase_a = [&](auto do_s_tag, auto do_e_tag, f32x16(&cs)[2], f32x16(&ns)[2],
                       const uint16_t* kb, const uint16_t* vb, auto&& hook) {
        constexpr bool DO_S = decltype(do_s_tag)::value;
        constexpr bool DO_E = decltype(do_e_tag)::value;
        float nn = 0.f, nn1 = 0.f;
        if constexpr (DO_E) {
            // online softmax (log2 domain, lazy rescale)
            if (__builtin_amdgcn_ballot_w64(mt_c > m_ref + kRescaleSlack) != 0) {
                const float m_new = fmaxf(m_ref, mt_c);
                const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
                m_ref = m_new;
                l_part *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int v = 0; v < 16; ++v) o_acc[db][v] *= alpha;
            }
            const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
            nn = bc_c - m_use;
            if constexpr (ALIBI_LIN) nn1 = nn + a32;
        }
        bf16x8 ka[KPRE][2];
        if constexpr (DO_S) {
#pragma unroll
            for (int v = 0; v < 16; ++v) { ns[0][v] = 0.f; ns[1][v] = 0.f; }
#pragma unroll
            for (int i = 0; i < KPRE; ++i) read_k(kb, i, ka[i]);
        }
        // The first E0 exponentials come before the first MFMAs: right after the barrier every
        // wave reads its first K fragments at once, and this work needs no LDS data, so it
        // covers that wait. The other exponentials are spread over the remaining k-steps.
        constexpr int E0 = 8;
        auto expo = [&](int e) {
            float pe = __builtin_amdgcn_exp2f(fmaf(cs[e >> 4][e & 15], cc_c, (ALIBI_LIN && (e >> 4)) ? nn1 : nn));
            pin(pe);
            cs[e >> 4][e & 15] = pe;
        };
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (DO_E) {
                if (ks == 0) {
#pragma unroll
                    for (int e = 0; e < E0; ++e) expo(e);
                }
            }
            if constexpr (DO_S) {
                const bf16x8 a0 = ka[ks % KPRE][0], a1 = ka[ks % KPRE][1];
                if (ks + KPRE < KS) read_k(kb, ks + KPRE, ka[ks % KPRE]);
                ns[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], ns[0], 0, 0, 0);
                ns[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], ns[1], 0, 0, 0);
            }
            if constexpr (DO_E) {
                if (ks > 0) {
#pragma unroll
                    for (int e = E0 + ((ks - 1) * (32 - E0)) / (KS - 1);
                         e < E0 + (ks * (32 - E0)) / (KS - 1); ++e)
                        expo(e);
                }
                if (ks >= KS - VPRE) read_v(vb, ks - (KS - VPRE), vfr[ks - (KS - VPRE)]);
            }
            hook(ks);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Phase B: P.V MFMAs of the tile in `cs` (DO_PV, V tile at vb) interleaved with the
    // preparation of the next tile tn in `ns` (DO_PREP): bias, mask, row max (K slot kb also
    // holds its full-bias tile).
    auto phase_b = [&](auto do_pv_tag, auto do_prep_tag, f32x16(&cs)[2], f32x16(&ns)[2],
                       const uint16_t* vb, const uint16_t* kb, int tn) {
        constexpr bool DO_PV = decltype(do_pv_tag)::value;
        constexpr bool DO_PREP = decltype(do_prep_tag)::value;
        const int j0 = tn * kBN;
        const int jl = j0 + 16 * hh;   // key of register 0 of this lane
        // Per-element path: full bias, or T5 near the diagonal. Otherwise the bias is constant
        // over the tile (none, or T5 far from the diagonal) and the scale is folded into the
        // exponent's FMA after a max over the raw scores.
        bool per_elem = FB || ALIBI;
        float bconst = 0.f;
        bool msk = false;
        if constexpr (DO_PREP) {
            msk = needs_mask(tn);
            if constexpr (IS_T5) {
                const int rmin = j0 - pwb, rmax = j0 + kBN - 1 - pwa;
                if (rmin >= kSat) bconst = t5s[2 * kT5Pad];
                else if (rmax <= -kSat) bconst = t5s[0];
                else per_elem = true;
            }
        }
        u32x4 fb[4];
        float ext = -INFINITY;
        // linear ALiBi: bias of key block 0 of this lane, slope * (jl - p)
        const float bl0 = ALIBI_LIN ? aslope * (float)(jl - my_pos) : 0.f;
        bf16x2 ones2;
        ones2[0] = (__bf16)1.0f;
        ones2[1] = (__bf16)1.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            if constexpr (DO_PV) {
                // Four key groups g = (jb, s) of 8 keys per lane half; the V^T fragments of
                // group g+1 are read while the MFMAs of group g run.
                const int jb = g >> 1, s = g & 1;
                u32x4 pk;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float p0 = cs[jb][8 * s + 2 * c], p1 = cs[jb][8 * s + 2 * c + 1];
                    pk[c] = pack_bf16x2(p0, p1);
                    // row sum of the bf16 weights the P.V product uses (one v_dot2 per pair).
                    // The pair is rounded again here rather than taken from pk[c]: reading the
                    // element of the packed vector made this compiler feed pk[0] to all four
                    // dot products; the two roundings are one instruction after CSE.
                    bf16x2 pr;
                    pr[0] = (__bf16)p0;
                    pr[1] = (__bf16)p1;
                    l_part = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, l_part, false);
                }
                const bf16x8 pbf = __builtin_bit_cast(bf16x8, pk);
                if (g + VPRE < 4) read_v(vb, g + VPRE, vfr[(g + VPRE) % (VPRE + 1)]);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[g % (VPRE + 1)][db], pbf, o_acc[db], 0, 0, 0);
            }
            if constexpr (DO_PREP) {
                if (g == 0) {
                    if constexpr (FB_LDS) {
                        if (fb_dma) {
                            // this tile's bias rows from the LDS ring: row (wave*32 + r32),
                            // chunks 4 jb + 2 hh + {0, 1}
                            const int ir = wave * 32 + r32;
                            const uint16_t* bt = kb + TILE + ir * kBN;
                            const int sw = (ir >> 1) & 7;
#pragma unroll
                            for (int jb = 0; jb < 2; ++jb) {
                                fb[2 * jb] = *(const u32x4*)(bt + (((4 * jb + 2 * hh) ^ sw) * 8));
                                fb[2 * jb + 1] = *(const u32x4*)(bt + (((4 * jb + 2 * hh + 1) ^ sw) * 8));
                            }
                        }
                    }
                } else if (g == 1) {
                    if (per_elem) {
                        if constexpr (ALIBI_LIN) {
#pragma unroll
                            for (int e = 0; e < 32; ++e)
                                ns[e >> 4][e & 15] = fmaf(al_a, (float)(e & 15), ns[e >> 4][e & 15]);
                        } else if constexpr (ALIBI) {
                            // register e holds key jl + 32 (e >> 4) + (e & 15)
                            const float base = (float)(jl - my_pos);
#pragma unroll
                            for (int e = 0; e < 32; ++e)
                                ns[e >> 4][e & 15] = fmaf(ns[e >> 4][e & 15], c_scale,
                                    -aslope * fabsf(base + (float)((e >> 4) * 32 + (e & 15))));
                        } else if constexpr (IS_T5) {
                            // register e holds key jl + 32 (e >> 4) + (e & 15): one base per
                            // lane, compile-time offsets (rows past the end of the queries use
                            // the wave's last row, so the index stays in the table)
                            const float* trow = t5s + kT5Pad + (jl - min(my_pos, pwb));
#pragma unroll
                            for (int e = 0; e < 32; ++e)
                                ns[e >> 4][e & 15] = fmaf(ns[e >> 4][e & 15], c_scale, trow[(e >> 4) * 32 + (e & 15)]);
                        } else if constexpr (FB) {
                            if (fb_dma) {
#pragma unroll
                                for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                                    for (int c = 0; c < 4; ++c)
#pragma unroll
                                        for (int hv = 0; hv < 2; ++hv) {
                                            const uint32_t lo = fb[2 * jb][c], hi = fb[2 * jb + 1][c];
                                            const int v0 = 2 * c + hv;
                                            ns[jb][v0] = fmaf(ns[jb][v0], n_scale,
                                                bf16_to_f32(hv ? (lo >> 16) : (lo & 0xffffu)));
                                            ns[jb][v0 + 8] = fmaf(ns[jb][v0 + 8], n_scale,
                                                bf16_to_f32(hv ? (hi >> 16) : (hi & 0xffffu)));
                                        }
                            } else {
                                const uint16_t* br = fbg + (size_t)(row_ok ? my_i : 0) * Sk;
#pragma unroll
                                for (int e = 0; e < 32; ++e) {
                                    const int j = jl + (e >> 4) * 32 + (e & 15);
                                    const float bv = (row_ok && j < Sk) ? bf16_to_f32(br[j]) : 0.f;
                                    ns[e >> 4][e & 15] = fmaf(ns[e >> 4][e & 15], n_scale, bv);
                                }
                            }
                        }
                    }
                    if (msk) {
                        // Visible keys of this lane's row form one interval [lo, hi]; register
                        // e of key block jb holds key jl + 32 jb + (e & 15), so visibility is a
                        // compare of the compile-time index e & 15 against per-lane bounds.
                        int hi = Sk - 1;
                        if constexpr (MASK != MASK_NONE) hi = min(hi, my_pos);
                        int lo = 0;
                        if constexpr (MASK == MASK_SLIDING) lo = max(0, my_pos - p.window + 1);
#pragma unroll
                        for (int jb = 0; jb < 2; ++jb) {
                            const int vh = hi - (jl + 32 * jb), vl = lo - (jl + 32 * jb);
#pragma unroll
                            for (int v = 0; v < 16; ++v) {
                                bool vis = v <= vh;
                                if constexpr (MASK == MASK_SLIDING) vis = vis && (v >= vl);
                                ns[jb][v] = vis ? ns[jb][v] : -INFINITY;
                            }
                        }
                    }
                } else {
                    // row max over key block g - 2 (hidden keys are -inf)
                    if constexpr (ALIBI_LIN) {
                        // each block's maximum, scaled, plus its per-row bias slope * (jl + 32 jb - p)
                        float eb = -INFINITY;
#pragma unroll
                        for (int v = 0; v < 16; ++v) eb = fmaxf(eb, ns[g - 2][v]);
                        ext = fmaxf(ext, fmaf(eb, al_c, g == 2 ? bl0 : bl0 + a32));
                    } else {
#pragma unroll
                        for (int v = 0; v < 16; ++v) ext = fmaxf(ext, ns[g - 2][v]);
                    }
                    pin(ext);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (DO_PREP) {
            ext = partner_max(ext);
            if constexpr (FB) {
                // scores plus bias in natural-log units: the exponent's FMA applies log2(e)
                mt_c = ext * kLog2e;
                cc_c = kLog2e;
                bc_c = 0.f;
            } else if (per_elem) {
                // T5 near the diagonal, ALiBi: scores already in the log2 domain (linear
                // ALiBi: raw scores plus the per-key part; scale and per-row part in the
                // exponent)
                mt_c = ext;
                cc_c = ALIBI_LIN ? al_c : 1.f;
                bc_c = ALIBI_LIN ? bl0 : 0.f;
            } else {
                // max over the raw scores (scale > 0); hidden keys stay -inf through the FMA
                mt_c = (ext == -INFINITY) ? -INFINITY : fmaf(ext, c_scale, bconst);
                cc_c = c_scale;
                bc_c = bconst;
            }
        }
    };

    // ---- main loop ---------------------------------------------------------------------------
    // Rings: K(t) (with its bias tile) in K slot (t - t_begin) % NKS, V(t) in V slot
    // (t - t_begin) & 1. Iteration t reads K(t+1) and V(t) while V(t+1) and K(t+NKS) are in
    // flight; the wait and barrier at its end publish V(t+1) and K(t+2) and free the slots of
    // V(t) and K(t+1).
    auto none = [](int) {};
    f32x16 sa[2], sb[2];
    dma_k(t_begin);
    dma_wait();
    __syncthreads();
    dma_v(t_begin);
    for (int u = t_begin + 1; u < t_begin + NKS && u < t_end; ++u) dma_k(u);
    if (active(t_begin)) {
        phase_a(True{}, False{}, sb, sa, kptr(t_begin), nullptr, none);
        phase_b(False{}, True{}, sb, sa, nullptr, kptr(t_begin), t_begin);
    }
    dma_wait_but_k(t_begin + 2);
    __syncthreads();

    // cs: prepared score registers of tile t; ns: receives S^T of tile t+1
    auto iteration = [&](int t, f32x16(&cs)[2], f32x16(&ns)[2]) {
        const bool has_next = t + 1 < t_end;
        const bool cur = active(t);
        const bool nxt = has_next && active(t + 1);
        if (!(cur && nxt)) {
            if (has_next) dma_v(t + 1);
            if (t + NKS < t_end) dma_k(t + NKS);
        }
        const uint16_t* kbn = kptr(t + 1);
        const uint16_t* vb = vptr(t);
        if (cur && nxt) {
            phase_a(True{}, True{}, cs, ns, kbn, vb, [&](int ks) {
#pragma unroll
                for (int i = 0; i < NXF; ++i)
                    if ((i * KS) / NXF == ks) dma_xfer(t, i);
            });
            phase_b(True{}, True{}, cs, ns, vb, kbn, t + 1);
        } else if (cur) {
            phase_a(False{}, True{}, cs, ns, kbn, vb, none);
            phase_b(True{}, False{}, cs, ns, vb, kbn, t + 1);
        } else if (nxt) {
            phase_a(True{}, False{}, cs, ns, kbn, vb, none);
            phase_b(False{}, True{}, cs, ns, vb, kbn, t + 1);
        }
        if (has_next) dma_wait_but_k(t + NKS);
        __syncthreads();
    };
    // unrolled by two so that the two score register sets swap roles without copies
#pragma unroll 1
    for (int t = t_begin; t < t_end; t += 2) {
        iteration(t, sa, sb);
        if (t + 1 >= t_end) break;
        iteration(t + 1, sb, sa);
    }

    // ---- epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l) ---------------------------------
    const float l_tot = partner_sum(l_part);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (row_ok) {
        char* o = out_ptr(my_i);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            // registers 8c .. 8c+7 of block db hold 8 consecutive head dims starting at d0[c]
            const int d0[2] = {16 * db + 8 * hh, 16 * (db + DB) + 8 * hh};
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
  };

    // ---- work items --------------------------------------------------------------------------
    // One item per workgroup, or (p.n_items > 0) a persistent grid of one workgroup per CU:
    // workgroup g runs on XCD g % 8 (round-robin dispatch) and takes that XCD's items (those
    // with index % 8 == g % 8, in decode_work's order) in rounds of nw = grid / 8, alternating
    // direction each round, so the heaviest and lightest causal tiles of a round pair up. The
    // hardware dispatcher places workgroup i on XCD i % 8 in index order and holds every later
    // workgroup while that XCD has no free CU; a persistent grid has no such gaps. Each item
    // is computed by the same code either way: the results do not depend on the grid.
    if constexpr (persist_of<D, BIAS, VARLEN>()) {
        const bool persist = p.n_items > 0;
        const int xcd = blockIdx.x & 7, l = blockIdx.x >> 3, nw = gridDim.x >> 3;
        auto item_of = [&](int r) {
            return persist ? (r * nw + ((r & 1) ? nw - 1 - l : l)) * 8 + xcd
                           : (r == 0 ? (int)blockIdx.x : 0x7fffffff);
        };
        const int lim = persist ? p.n_items : 0x7fffffff;
#pragma unroll 1
        for (int r = 0;; ++r) {
            const int x = item_of(r);
            if (x >= lim) break;
            run_item(x);
        }
    } else {
        run_item(blockIdx.x);
    }
}

// ------------------------------------------------------------------------------------------
// host-side launch (called by the C ABI after validation)
// ------------------------------------------------------------------------------------------
// compute units of the current device (cached per device)
static int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Workgroups of a launch (p.n_qt and p.xcd_remap set): one per work item, or a persistent grid
// when the kind allows it, every XCD receives whole (batch, KV head) groups and there are at
// least two items per workgroup; one workgroup fits a CU (registers), so that grid is the CU
// count rounded down to whole XCDs. Sets p.n_items (0: one workgroup per item).
static int fwd_grid(FwdParams& p, bool persist) {
    const int total = p.B * p.Hq * p.n_qt;
    p.n_items = 0;
    if (persist && p.xcd_remap) {
        const int pg = (cu_count() / 8) * 8;
        if (pg >= 8 && total >= 2 * pg) {
            p.n_items = total;
            return pg;
        }
    }
    return total;
}

template <int D, int MASK, int BIAS, bool OUT_F32, bool VARLEN>
static hipError_t launch_one(FwdParams p, hipStream_t stream) {
    const int grid = fwd_grid(p, persist_of<D, BIAS, VARLEN>());
    hipLaunchKernelGGL((sdpa_fwd_bf16_kernel<D, MASK, BIAS, OUT_F32, VARLEN>), dim3(grid),
                       dim3(64 * waves_of<D, BIAS>()), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool OUT_F32>
static hipError_t launch_d(const FwdParams& p, int mask, int bias, hipStream_t s) {
#define SDPA_CASE(M, Bk) \
    if (mask == M && bias == Bk) return launch_one<D, M, Bk, OUT_F32, false>(p, s);
    SDPA_CASE(MASK_NONE, BIAS_NONE) SDPA_CASE(MASK_NONE, BIAS_T5) SDPA_CASE(MASK_NONE, BIAS_FULL)
    SDPA_CASE(MASK_CAUSAL, BIAS_NONE) SDPA_CASE(MASK_CAUSAL, BIAS_T5) SDPA_CASE(MASK_CAUSAL, BIAS_FULL)
    SDPA_CASE(MASK_SLIDING, BIAS_NONE) SDPA_CASE(MASK_SLIDING, BIAS_T5) SDPA_CASE(MASK_SLIDING, BIAS_FULL)
    SDPA_CASE(MASK_NONE, BIAS_ALIBI) SDPA_CASE(MASK_CAUSAL, BIAS_ALIBI) SDPA_CASE(MASK_SLIDING, BIAS_ALIBI)
    SDPA_CASE(MASK_NONE, BIAS_T5U) SDPA_CASE(MASK_CAUSAL, BIAS_T5U) SDPA_CASE(MASK_SLIDING, BIAS_T5U)
#undef SDPA_CASE
    return hipErrorInvalidValue;
}

// packed variable-length sequences: no full bias (no [B][Hq][Sq][Sk] frame)
template <int D, bool OUT_F32>
static hipError_t launch_varlen_d(const FwdParams& p, int mask, int bias, hipStream_t s) {
#define SDPA_CASE(M, Bk) \
    if (mask == M && bias == Bk) return launch_one<D, M, Bk, OUT_F32, true>(p, s);
    SDPA_CASE(MASK_NONE, BIAS_NONE) SDPA_CASE(MASK_NONE, BIAS_T5)
    SDPA_CASE(MASK_CAUSAL, BIAS_NONE) SDPA_CASE(MASK_CAUSAL, BIAS_T5)
    SDPA_CASE(MASK_SLIDING, BIAS_NONE) SDPA_CASE(MASK_SLIDING, BIAS_T5)
    SDPA_CASE(MASK_NONE, BIAS_ALIBI) SDPA_CASE(MASK_CAUSAL, BIAS_ALIBI) SDPA_CASE(MASK_SLIDING, BIAS_ALIBI)
    SDPA_CASE(MASK_NONE, BIAS_T5U) SDPA_CASE(MASK_CAUSAL, BIAS_T5U) SDPA_CASE(MASK_SLIDING, BIAS_T5U)
#undef SDPA_CASE
    return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_dim(FwdParams p, int mask, int bias, bool out_f32, hipStream_t s) {
    if (p.cu_q)
        return out_f32 ? launch_varlen_d<D, true>(p, mask, bias, s) : launch_varlen_d<D, false>(p, mask, bias, s);
    return out_f32 ? launch_d<D, true>(p, mask, bias, s) : launch_d<D, false>(p, mask, bias, s);
}

// query tiles per (batch, head) and the XCD grouping of a launch
static bool fwd_geometry(FwdParams& p, int D, int bias) {
    int bm = 0;
    switch (D) {
        case 32: bm = rows_of<32, BIAS_NONE>(); break;
        case 64: bm = bias == BIAS_FULL ? rows_of<64, BIAS_FULL>() : rows_of<64, BIAS_NONE>(); break;
        case 128: bm = rows_of<128, BIAS_NONE>(); break;
        case 256: bm = rows_of<256, BIAS_NONE>(); break;
        default: return false;
    }
    p.n_qt = (p.Sq + bm - 1) / bm;
    p.xcd_remap = ((p.B * p.Hkv) % 8 == 0) ? 1 : 0;
    return true;
}

hipError_t fwd_bf16_workgroups(FwdParams p, int D, int bias, long long* workgroups) {
    if (!fwd_geometry(p, D, bias)) return hipErrorInvalidValue;
    *workgroups = fwd_grid(p, persist_ok(D, bias, p.cu_q != nullptr));
    return hipSuccess;
}

hipError_t launch_fwd_bf16(FwdParams p, int D, int mask, int bias, bool out_f32, hipStream_t s) {
    if (!fwd_geometry(p, D, bias)) return hipErrorInvalidValue;
    switch (D) {
        case 32: return launch_dim<32>(p, mask, bias, out_f32, s);
        case 64: return launch_dim<64>(p, mask, bias, out_f32, s);
        case 128: return launch_dim<128>(p, mask, bias, out_f32, s);
        case 256: return launch_dim<256>(p, mask, bias, out_f32, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sdpa
