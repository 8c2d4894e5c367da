// Launch parameters and index helpers shared by the gfx950 attention-forward kernels and the
// host launcher. Only index arithmetic lives here; the kernels hold the attention math.
#pragma once

#include <stdint.h>

namespace sdpa {

enum { MASK_NONE = 0, MASK_CAUSAL = 1, MASK_SLIDING = 2 };
enum { BIAS_NONE = 0, BIAS_T5 = 1, BIAS_FULL = 2, BIAS_ALIBI = 3, BIAS_T5U = 4 };

// T5 relative-position table: [Hq][32] fp32. Within one sign of (key - query) the bucket
// saturates for distances >= 91, so a relative position only matters inside [-91, 91].
constexpr int kT5Buckets = 32;
constexpr int kT5Sat = 91;

struct FwdParams {
    const void* q;       // [B][Sq][Hq][D]
    const void* k;       // [B][Sk][Hkv][D]
    const void* v;       // [B][Sk][Hkv][D]
    void* out;           // [B][Sq][Hq][D]
    float* lse;          // [B][Hq][Sq]
    const void* bias;    // T5 table [Hq][32] fp32, or full bias [B][Hq][Sq][Sk]
    int B, Hq, Hkv, Sq, Sk;
    int G;               // Hq / Hkv: query heads per KV head
    int off;             // Sk - Sq: absolute position of query row i is i + off
    int window;          // sliding window (keys with 0 <= pos - j < window are visible)
    int n_qt;            // query tiles per (batch, head)
    int xcd_remap;       // 1: place all work of one (batch, KV head) on one XCD
    float scale;         // softmax scale
    float scale_log2;    // scale * log2(e)
    // Packed variable-length sequences (B = number of sequences, Sq / Sk = the longest query /
    // key sequence): sequence b owns query tokens cu_q[b] .. cu_q[b+1]-1 of q/out ([total_q]
    // [Hq][D]) and key tokens cu_k[b] .. cu_k[b+1]-1 of k/v; lse is [Hq][total_q].
    const int* cu_q;
    const int* cu_k;
    int total_q, total_k;
    // > 0: persistent grid (one workgroup per CU) walking this many work items
    int n_items;
};

// Backward: gradients of L = sum(dO * O) for the forward above.
struct BwdParams {
    const void* q;       // [B][Sq][Hq][D] bf16
    const void* k;       // [B][Sk][Hkv][D] bf16
    const void* v;       // [B][Sk][Hkv][D] bf16
    const void* o;       // [B][Sq][Hq][D] bf16: the forward's output
    const float* lse;    // [B][Hq][Sq]: the forward's row log-sum-exp
    const void* dout;    // [B][Sq][Hq][D] bf16: dL/dO
    void* dq;            // [B][Sq][Hq][D]  bf16 or fp32
    void* dk;            // [B][Sk][Hkv][D] bf16 or fp32
    void* dv;            // [B][Sk][Hkv][D] bf16 or fp32
    float* delta;        // [B][Hq][Sq] workspace: rowsum(dO * O)
    const void* bias;    // T5 table [Hq][32] fp32, or full bias [B][Hq][Sq][Sk] bf16
    int B, Hq, Hkv, Sq, Sk;
    int G;               // Hq / Hkv
    int off;             // Sk - Sq
    int window;
    int n_qt;            // 256-row query tiles per (batch, query head)   (dQ kernel)
    int n_kt;            // 128-key tiles per (batch, KV head)            (dK/dV kernel)
    int xcd_remap;
    float scale;
    float scale_log2;
};

// T5 bidirectional bucket of rel = key position - query position (integer form of the T5 log
// spacing: for 8 <= n < 91 the bucket 8 + floor(8 log(n/8) / log 16) equals 1 + bitlen(n^2)).
__host__ __device__ inline int t5_bucket(int rel) {
    int n = rel < 0 ? -rel : rel;
    int b;
    if (n < 8) {
        b = n;
    } else if (n >= kT5Sat) {
        b = 15;
    } else {
        unsigned nn = (unsigned)(n * n);
        int bitlen = 32 - __builtin_clz(nn);
        b = 1 + bitlen;
    }
    return b + (rel > 0 ? 16 : 0);
}

// T5 unidirectional (decoder) bucket of rel = key position - query position: keys at or after
// the query share bucket 0; a key n positions back gets n below 16, else
// 16 + floor(16 log(n/16) / log 8) capped at 31, i.e. 16 plus the number of thresholds below
// that n reaches (threshold b: the smallest n with n^16 >= 2^(64 + 3b), b = 1..15). Saturates
// from distance 113.
constexpr int kT5USat = 113;
__host__ __device__ inline int t5u_bucket(int rel) {
    const int n = rel < 0 ? -rel : 0;
    if (n < 16) return n;
    const int thr[15] = {19, 21, 24, 27, 31, 35, 40, 46, 52, 59, 67, 77, 87, 99, 113};
    int b = 16;
#pragma unroll
    for (int i = 0; i < 15; ++i) b += (n >= thr[i]) ? 1 : 0;
    return b;
}

// Decode a work item index into (batch, query head, query tile). Query tiles of one
// (batch, KV head) are consecutive, heaviest (latest, for causal masks) first; with
// xcd_remap, item x runs on XCD x % 8 (workgroup x under round-robin dispatch, or the
// persistent workgroup of that XCD), and every XCD receives whole (batch, KV head) groups so
// the G query heads sharing K/V hit the same L2.
struct WorkItem { int b, hq, qt; };

template <class Params>
__host__ __device__ inline WorkItem decode_work(const Params& p, int x) {
    const int per_group = p.G * p.n_qt;
    int group, r;
    if (p.xcd_remap) {
        const int xcd = x & 7, slot = x >> 3;
        const int gl = slot / per_group;
        r = slot - gl * per_group;
        group = gl * 8 + xcd;
    } else {
        group = x / per_group;
        r = x - group * per_group;
    }
    WorkItem w;
    w.b = group / p.Hkv;
    const int kvh = group - w.b * p.Hkv;
    const int qi = r / p.G;
    w.hq = kvh * p.G + (r - qi * p.G);
    w.qt = p.n_qt - 1 - qi;
    return w;
}

}  // namespace sdpa
