// Launch parameters of the split-key decode kernels (few query rows against a long KV cache)
// and the work split, shared by the C ABI and the kernels. Index arithmetic only.
#pragma once

#include <stddef.h>

namespace sdpa {

// Size of the static per-device scratch behind the no-allocation decode entry point (the
// partial results of every split); the public header states the same value.
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;

struct DecParams {
    const void* q;       // [B][Sq][Hq][D] bf16
    const void* k;       // [B][Sk][Hkv][D] bf16
    const void* v;       // [B][Sk][Hkv][D] bf16
    void* out;           // [B][Sq][Hq][D] bf16 or fp32
    float* lse;          // [B][Hq][Sq]
    float* ws;           // partial results: [group][row block][split][32][D] O, then [..][32][2] m, l
    const void* bias;    // T5 table [Hq][32] fp32, or full bias [B][Hq][Sq][Sk] bf16
    int B, Hq, Hkv, Sq, Sk;
    int G;               // Hq / Hkv
    int off;             // Sk - Sq
    int window;
    int rows;            // G * Sq query rows per (batch, KV head), ordered r = i * G + g
    int n_rb;            // 32-row blocks of those rows
    int n_split;         // key splits per row block
    float scale;
    float scale_log2;
};

// Work split: key splits per (batch, KV head, row block), chosen from the shape alone so the
// summation order (and so every bit of the result) depends on nothing else.
inline int dec_row_blocks(int G, int Sq) { return (G * Sq + 31) / 32; }
inline int dec_splits(int B, int Hkv, int G, int Sq, int Sk) {
    const long long groups = (long long)B * Hkv * dec_row_blocks(G, Sq);
    const int tiles = (Sk + 63) / 64;
    // about one workgroup per CU of the 256 (measured: 256 splits in total beat 128, 384 and
    // 768 on every decode shape; each workgroup keeps three tiles in flight)
    long long n = (256 + groups - 1) / groups;
    const int cap = tiles / 4 > 1 ? tiles / 4 : 1;   // at least four 64-key tiles per split
    if (n > cap) n = cap;
    if (n < 1) n = 1;
    return (int)n;
}
inline size_t dec_ws_floats(int B, int Hkv, int G, int Sq, int Sk, int D) {
    const size_t units = (size_t)B * Hkv * dec_row_blocks(G, Sq) * dec_splits(B, Hkv, G, Sq, Sk);
    return units * 32 * (size_t)(D + 2);
}

}  // namespace sdpa
