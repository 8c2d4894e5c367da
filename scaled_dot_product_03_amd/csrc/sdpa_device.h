// Device helpers shared by the gfx950 gradient and decode kernels: vector types, the MFMA row
// permutation, the LDS swizzle of streamed K/V/Q/dO tiles, LDS-DMA transfers, transposing
// LDS reads and the O^T-layout row store. Index arithmetic and data movement only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTinyScale = 1.17549435e-38f;   // stands in for a zero scale (see the forward)

// Row permutation inside a 32-row MFMA operand (output register v of lane half h holds row
// 16h + v), as in the forward kernel.
__device__ __forceinline__ int perm32(int r) {
    return ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3);
}
// XOR swizzle of the 16-byte chunk index of a tile row. Streamed tiles are read both
// row-wise (ds_read_b128: 16 lanes per LDS cycle on rows {0..3, 16..19, 4..7, 20..23} + 8m,
// one chunk each) and through transposing reads (ds_read_b64_tr_b16: 32 lanes per cycle on 4
// consecutive rows, chunks c + {0, 1, 2DB, 2DB + 1}). Row bits 0-1 (D = 128) or bit 1 (D = 64,
// two rows per 256-byte bank line) pick distinct chunk pairs for the transposing reads; row
// bits 2 and 4 fill the remaining swizzle bits so the 16 rows of a row-wise read land on 16
// distinct chunks of the bank line. D = 32 rows are 4 chunks (four rows per bank line): the
// pattern takes row bits 2 and 4 and stays inside the row. D = 256 uses the D = 64 pattern.
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128)
        return (2 * (row & 3)) | ((row >> 4) & 1) | (((row >> 2) & 1) << 3);
    else if constexpr (D == 32)
        return ((row >> 2) & 1) | (((row >> 4) & 1) << 1);
    else
        return (row & 2) | ((row >> 4) & 1) | (((row >> 2) & 1) << 2);
}

// A value the caller knows to be equal in every lane of the wave, made visibly uniform to the
// compiler so that branches on it stay scalar.
__device__ __forceinline__ bool uniform(bool b) { return __builtin_amdgcn_readfirstlane((int)b) != 0; }
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float partner_max(float x) {
    // max of this lane's value and that of lane l ^ 32 (same result in both lanes)
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float partner_sum(float x) {
    // this lane's value plus that of lane l ^ 32 (same result in both lanes)
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

__device__ __forceinline__ void dma16(const uint16_t* src, uint32_t lds_dst) {
    // one 1 KB transfer: lane i's 16 bytes land at M0 + 16 i (no other instruction here reads
    // M0); waited for explicitly with s_waitcnt vmcnt before the publishing barrier
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds_dst)) : "memory");
}
__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposing read of 8 consecutive tile rows for the A operand of an MFMA whose k index runs
// over rows: key group g holds rows 16 h + 8 (g & 1) + 32 (g >> 1) + e of lane half h, the
// layout of the P / dS registers. Returns the DB fragments (32 head dims each) of group g;
// rows 0..15 of fragment db are head dims 16 db + sigma, rows 16..31 are 16 (db + DB) + sigma.
template <int D>
__device__ __forceinline__ void read_tr(const uint16_t* tile, int g, int lane, bf16x8* dst) {
    constexpr int DB = D / 32;
    const int hh = lane >> 5, gg = lane >> 4, li = lane & 15, la = li & 3;
    const int row = 16 * hh + (li >> 2) + 32 * (g >> 1) + 8 * (g & 1);
    const int dlo = 16 * DB * (gg & 1) + 8 * (la & 1) + 4 * (la >> 1);
    const int sw0 = swz<D>(row), sw1 = swz<D>(row + 4);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int d = 16 * db + dlo;
        const s16x4 lo = lds_read_tr(tile + row * D + ((((d >> 3) ^ sw0) << 3) | (d & 7)));
        const s16x4 hi = lds_read_tr(tile + (row + 4) * D + ((((d >> 3) ^ sw1) << 3) | (d & 7)));
        u32x4 av;
        av[0] = __builtin_bit_cast(u32x2, lo)[0];
        av[1] = __builtin_bit_cast(u32x2, lo)[1];
        av[2] = __builtin_bit_cast(u32x2, hi)[0];
        av[3] = __builtin_bit_cast(u32x2, hi)[1];
        dst[db] = __builtin_bit_cast(bf16x8, av);
    }
}

// Row-wise read for the A operand of S (rows perm32(lane % 32) + 32 blk of the tile, head dims
// 16 ks + 8 (lane / 32) .. + 7).
template <int D>
__device__ __forceinline__ bf16x8 read_rows(const uint16_t* tile, int blk, int ks, int lane) {
    const int row = perm32(lane & 31) + 32 * blk;
    const int ch = ((2 * ks + (lane >> 5)) ^ swz<D>(row)) * 8;
    return *(const bf16x8*)(tile + row * D + ch);
}

// Writes the O^T-layout accumulators of one lane (rows of head dims per block db, see read_tr)
// times `mul` to the D-element row at `dst`.
template <int D, bool OUT_F32>
__device__ __forceinline__ void store_row(char* dst, const f32x16 (&acc)[D / 32], float mul, int hh) {
    constexpr int DB = D / 32;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int d0[2] = {16 * db + 8 * hh, 16 * (db + DB) + 8 * hh};
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            if constexpr (OUT_F32) {
#pragma unroll
                for (int hv = 0; hv < 2; ++hv) {
                    u32x4 xo;
#pragma unroll
                    for (int e = 0; e < 4; ++e) xo[e] = __float_as_uint(acc[db][8 * c + 4 * hv + e] * mul);
                    *(u32x4*)(dst + (d0[c] + 4 * hv) * 4) = xo;
                }
            } else {
                u32x4 xo;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    xo[e] = pack_bf16x2(acc[db][8 * c + 2 * e] * mul, acc[db][8 * c + 2 * e + 1] * mul);
                *(u32x4*)(dst + d0[c] * 2) = xo;
            }
        }
    }
}

template <int D, bool OUT_F32>
__device__ __forceinline__ void store_zero_row(char* dst, int hh) {
    f32x16 z[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) z[db][v] = 0.f;
    store_row<D, OUT_F32>(dst, z, 0.f, hh);
}

}  // namespace dev
}  // namespace sdpa
