/*
 * sdpa.h -- C ABI of the MI355X (gfx950) fused scaled-dot-product attention forward and its
 * gradients (sdpa_bwd, below).
 *
 * Forward operation (one call = one fused kernel launch):
 *     O   = softmax(Q.K^T * scale + bias + mask) . V
 *     LSE = log(sum_j exp(Q.K^T * scale + bias + mask))        (natural log, per query row)
 *   Definition: the four steps (score, scale + softmax, attend, output with Q's shape) of the
 *   "jax-gpu-05-attention-gpu" codelab, section 1, and of the Medium post "Simplified
 *   Explanation of Attention", steps 1-4. Masks are generated inside the kernel from indices
 *   (codelab section 7, is_causal; transformers issue "Slowdown in Training Speed Due to SDPA
 *   Mask Fix in Version 4.40.0" for the sliding window). Biases: T5 bucketed relative-position
 *   bias or a full additive bias (FAT5 / flashT5 README, attention-bias list). Head sharing:
 *   MHA / GQA / MQA (codelab section 9).
 *
 * Layout (codelab section 3: batch, sequence, heads, head dim; innermost dim contiguous):
 *   q, out : [B][Sq][Hq][D]          k, v : [B][Sk][Hkv][D]          lse : [B][Hq][Sq] fp32
 *   Query head h reads KV head h / (Hq / Hkv) (contiguous groups).
 *   Query row i sits at absolute position i + (Sk - Sq) (bottom-right alignment).
 *
 * Masks (mask_kind):
 *   SDPA_MASK_NONE     every key visible.
 *   SDPA_MASK_CAUSAL   key j visible from query position p iff j <= p.
 *   SDPA_MASK_SLIDING  key j visible iff 0 <= p - j < window (window >= Sk equals CAUSAL,
 *                      bit for bit). `window` is ignored for the other kinds.
 *   A query row that sees no key gets O = 0 and LSE = -inf.
 *
 * Biases (bias_kind, bias_tbl):
 *   SDPA_BIAS_NONE  bias_tbl must be NULL.
 *   SDPA_BIAS_T5    bias_tbl = fp32 table [Hq][32]; the score of (query position p, key j) in
 *                   head h gets tbl[h][bucket(j - p)], where bucket is the T5 bidirectional
 *                   scheme: 16 buckets per sign of j - p (keys after the query use buckets
 *                   16..31), distances 0..7 exact, 8..127 log-spaced, >= 128 (in fact >= 91)
 *                   saturating at the last bucket of the half.
 *   SDPA_BIAS_FULL  bias_tbl = [B][Hq][Sq][Sk] in the input dtype (bf16 for sdpa_fwd and
 *                   sdpa_fwd_bf16_f32out, fp32 for sdpa_fwd_f32).
 *   SDPA_BIAS_ALIBI bias_tbl = fp32 slopes [Hq]; the score of (query position p, key j) in head
 *                   h gets -slope[h] * |p - j| (ALiBi, named in the FAT5 README's bias list;
 *                   under a causal mask this is slope * (j - p)).
 *   SDPA_BIAS_T5U   bias_tbl = fp32 table [Hq][32] with T5 unidirectional (decoder) buckets:
 *                   keys at or after the query use bucket 0, a key n positions back bucket n
 *                   below 16, then log-spaced to 31 (reached at n = 113).
 *
 * Conventions for every entry point:
 *   - All pointers are DEVICE pointers owned by the caller. The library allocates nothing,
 *     keeps nothing after returning, and writes every element of out and lse (the one
 *     exception, sdpa_decode_noalloc, uses a static per-GPU scratch array instead).
 *   - q, k, v, out and a full bias must be 16-byte aligned; lse 4-byte aligned.
 *   - stream is a hipStream_t (NULL = the default stream). The call only enqueues work; inputs
 *     must stay alive until the stream has finished it.
 *   - Returns SDPA_OK or the first failed check; on error nothing is launched. No exception
 *     crosses this boundary. Launch failures return SDPA_ERR_LAUNCH.
 *   - Thread-safe: no mutable global state besides two per-device caches, each written once:
 *     the compute-unit count that sizes the forward's persistent grid (an atomic) and the
 *     scratch address that sdpa_decode_noalloc resolves under a lock. Results are bitwise
 *     reproducible run to run for a given shape (fixed tile shape chosen from the shape alone,
 *     fixed key order, no atomics; the same bits whatever the grid: one workgroup per work item
 *     or the persistent grid),
 *     the determinism the transformers issue "Transformer models are not deterministic when
 *     using Flash Attention 2" asks of a fused kernel.
 *   - Validation: B, Hq, Hkv, Sq, Sk >= 1; Hq % Hkv == 0; D in {32, 64, 128, 256} (the
 *     head-dim sweep the "jax-gpu-05-attention-gpu" codelab closes with); scale finite;
 *     SLIDING needs window >= 1; bias_tbl non-NULL iff bias_kind != NONE; B*Hq*Sq*D,
 *     B*Hkv*Sk*D (and B*Hq*Sq*Sk for a full bias) below 2^40 elements.
 */
#ifndef SDPA_MI355X_SDPA_H
#define SDPA_MI355X_SDPA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDPA_ABI_VERSION 4

/* Size of the device scratch buffer behind sdpa_decode_noalloc (per GPU): 16 MiB. */
#define SDPA_DECODE_SCRATCH_BYTES (16u << 20)

enum sdpa_mask_kind { SDPA_MASK_NONE = 0, SDPA_MASK_CAUSAL = 1, SDPA_MASK_SLIDING = 2 };
enum sdpa_bias_kind {
    SDPA_BIAS_NONE = 0, SDPA_BIAS_T5 = 1, SDPA_BIAS_FULL = 2, SDPA_BIAS_ALIBI = 3, SDPA_BIAS_T5U = 4
};

enum sdpa_status {
    SDPA_OK = 0,
    SDPA_ERR_NULL = 1,      /* a required pointer is NULL */
    SDPA_ERR_SHAPE = 2,     /* B, Hq, Hkv, Sq or Sk < 1, or a tensor too large */
    SDPA_ERR_HEADS = 3,     /* Hq not a multiple of Hkv */
    SDPA_ERR_HEADDIM = 4,   /* D not in {32, 64, 128, 256} */
    SDPA_ERR_MASK = 5,      /* unknown mask_kind */
    SDPA_ERR_WINDOW = 6,    /* SLIDING with window < 1 */
    SDPA_ERR_BIAS = 7,      /* unknown bias_kind, or bias_tbl NULL/non-NULL against it */
    SDPA_ERR_SCALE = 8,     /* scale not finite */
    SDPA_ERR_ALIGN = 9,     /* a pointer is not aligned as required */
    SDPA_ERR_LAUNCH = 10,   /* the HIP launch reported an error */
    SDPA_ERR_WORKSPACE = 11, /* workspace NULL, misaligned or smaller than required */
    SDPA_ERR_DEVICE = 12     /* current device unknown or its scratch buffer not resolved */
};

/*
 * bf16 forward: q, k, v, out are bf16 (raw 16-bit words); lse fp32. The hot path: bf16 MFMA
 * for Q.K^T and P.V with fp32 accumulation, fp32 online softmax, O rounded to bf16 (nearest
 * even) from exactly the fp32 value sdpa_fwd_bf16_f32out returns.
 */
int sdpa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
             int mask_kind, int window, int bias_kind, const void* bias_tbl, void* stream);

/* Same kernel as sdpa_fwd (bf16 inputs), but out is fp32: [B][Sq][Hq][D] float. */
int sdpa_fwd_bf16_f32out(const void* q, const void* k, const void* v, float* out, float* lse,
                         int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                         int mask_kind, int window, int bias_kind, const void* bias_tbl,
                         void* stream);

/*
 * Workgroups that sdpa_fwd and sdpa_fwd_bf16_f32out launch for this shape, mask and bias on the
 * current device (nothing is read, written or launched). A call forms one output tile per
 * (batch, query head, block of query rows: 256 rows at D = 64 and 128, 128 rows at D = 32 and
 * 256 and for SDPA_BIAS_FULL at D = 64); it launches one
 * workgroup per tile, or, for the kinds built for it (D = 64, or D = 128 with neither
 * SDPA_BIAS_T5 nor SDPA_BIAS_T5U; never SDPA_BIAS_FULL), when B*Hkv is a multiple
 * of 8 and there are at least two tiles per workgroup, a persistent grid of the device's CU
 * count rounded down to a multiple of 8, each workgroup walking the tiles of its XCD. With no
 * device the CU count reads as 0 and the one-per-tile grid is reported. The result does not
 * change the output: both grids give the same bits.
 *   workgroups: host pointer, receives the count. Returns the status sdpa_fwd would give for
 *   these arguments with valid buffers (SDPA_ERR_NULL if workgroups is NULL).
 */
int sdpa_fwd_launch_grid(int B, int Hq, int Hkv, int Sq, int Sk, int D, int mask_kind, int window,
                         int bias_kind, long long* workgroups);

/* fp32 forward (fp32 q, k, v, out, full bias): the high-precision path, fp32 FMA arithmetic. */
int sdpa_fwd_f32(const float* q, const float* k, const float* v, float* out, float* lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                 int mask_kind, int window, int bias_kind, const void* bias_tbl, void* stream);

/*
 * bf16 backward: the gradients of L = sum(dout * out) with respect to q, k and v, where out is
 * the forward above (same shapes, masks, biases, scale and head sharing). The pages use the
 * backward without printing it (FAT5 README: backward TFLOPS of its biased flash kernels;
 * transformers issue "Transformer models are not deterministic when using Flash Attention 2":
 * run-to-run equality of a training step); the formulas are the chain rule through the
 * forward's definition, with P the softmax weights and S the scaled, biased, masked scores:
 *     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
 *     dQ = scale * dS K,  dK = scale * dS^T Q.
 * A KV head shared by G query heads gets the sum of their dK and dV. The biases get no
 * gradient.
 *   q, k, v, out, dout : bf16 (out and lse as written by sdpa_fwd for the same arguments)
 *   dq : [B][Sq][Hq][D]   dk, dv : [B][Sk][Hkv][D]   (bf16 here, fp32 for sdpa_bwd_f32out)
 *   ws : caller-owned device workspace of B*Hq*Sq floats (4-byte aligned); receives
 *        rowsum(dout * out) per query row; its contents on entry do not matter.
 * Two launches on `stream`: dq with the row sums (one workgroup per 256 query rows, 128 at
 * D = 256), then dk and dv (one workgroup per 128 keys of one KV head, 64 at D = 256, looping
 * over the query rows of its G heads).
 * Every output element has exactly one writer and a fixed summation order (query heads
 * ascending, query rows ascending): bitwise reproducible, no atomics. Validation as for
 * sdpa_fwd, plus dout, dq, dk, dv 16-byte aligned and non-NULL, ws non-NULL.
 */
int sdpa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, float* ws,
             int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
             int mask_kind, int window, int bias_kind, const void* bias_tbl, void* stream);

/* Same as sdpa_bwd, with dq, dk, dv in fp32. */
int sdpa_bwd_f32out(const void* q, const void* k, const void* v, const void* out,
                    const float* lse, const void* dout, float* dq, float* dk, float* dv,
                    float* ws, int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                    int mask_kind, int window, int bias_kind, const void* bias_tbl,
                    void* stream);

/*
 * Packed variable-length sequences: n_seqs sequences stored back to back along the token axis,
 * each attending only to itself (a block-diagonal document mask, generated from the offsets;
 * training with packing in the transformers issue "Slowdown in Training Speed Due to SDPA
 * Mask Fix in Version 4.40.0"). Sequence s owns query tokens cu_seqlens_q[s] ..
 * cu_seqlens_q[s+1]-1 and key tokens cu_seqlens_k[s] .. cu_seqlens_k[s+1]-1; inside it the
 * operation, masks (bottom-right alignment with the sequence's own lengths), T5 bias and head
 * sharing are those of sdpa_fwd.
 *   q, out : [total_q][Hq][D]    k, v : [total_k][Hkv][D]    lse : [Hq][total_q] fp32
 *   cu_seqlens_q, cu_seqlens_k : DEVICE int32 arrays of n_seqs + 1 nondecreasing offsets.
 *   max_seqlen_q / max_seqlen_k : upper bounds of the sequences' lengths (they size the grid).
 * bias_kind: NONE or T5 (a full bias has no packed frame: SDPA_ERR_BIAS). The offsets live on
 * the device and are not read by the host: a sequence whose offsets leave [0, total] or exceed
 * the stated maximum lengths is treated as empty (its rows are not written) instead of being
 * read out of bounds. Tokens not covered by any sequence are not written.
 * Same kernel as sdpa_fwd (bitwise: a pack of equal-length sequences gives sdpa_fwd's bits).
 */
int sdpa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int n_seqs, int total_q,
                    int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int D,
                    float scale, int mask_kind, int window, int bias_kind, const void* bias_tbl,
                    void* stream);

/* Same as sdpa_fwd_varlen with fp32 out. */
int sdpa_fwd_varlen_f32out(const void* q, const void* k, const void* v, float* out, float* lse,
                           const int* cu_seqlens_q, const int* cu_seqlens_k, int n_seqs,
                           int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int Hq,
                           int Hkv, int D, float scale, int mask_kind, int window, int bias_kind,
                           const void* bias_tbl, void* stream);

/*
 * KV-cache decode: the forward above (same operation, arguments, layouts, masks, biases, head
 * sharing and outputs) for few query rows against a long key/value cache, the generation
 * setting of the KV-cache section of the Medium post "Simplified Explanation of Attention"
 * (bottom-right alignment: query row i sits at position i + Sk - Sq). Any Sq is accepted; the
 * kernels are built for Sq * Hq / Hkv up to a few 32-row blocks. The key range is split so
 * that every CU streams part of the cache: one launch forms a partial (max, sum, O) per split,
 * a second combines the splits in split order. The split count is a function of
 * (B, Hq, Hkv, Sq, Sk) alone, so results are bitwise reproducible run to run; they are not
 * bitwise equal to sdpa_fwd's (another summation order), both meeting the forward's bars.
 *   ws       : caller-owned device workspace, 16-byte aligned, at least
 *              sdpa_decode_ws_bytes(B, Hq, Hkv, Sq, Sk, D) bytes; contents on entry do not
 *              matter. Error SDPA_ERR_WORKSPACE otherwise.
 *   q, k, v, out: bf16 (sdpa_decode) or bf16 in / fp32 out (sdpa_decode_f32out); lse fp32.
 */
size_t sdpa_decode_ws_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D);

int sdpa_decode(const void* q, const void* k, const void* v, void* out, float* lse, void* ws,
                size_t ws_bytes, int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                int mask_kind, int window, int bias_kind, const void* bias_tbl, void* stream);

int sdpa_decode_f32out(const void* q, const void* k, const void* v, float* out, float* lse,
                       void* ws, size_t ws_bytes, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                       float scale, int mask_kind, int window, int bias_kind,
                       const void* bias_tbl, void* stream);

/*
 * sdpa_decode (bf16 out) for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments, kernels,
 * arithmetic and results (bit for bit) as sdpa_decode, without the workspace: the per-split
 * partial results go to a device scratch array of SDPA_DECODE_SCRATCH_BYTES that the library
 * holds on each GPU it runs on, until the process ends. Its device address is looked up once
 * per device (hipGetSymbolAddress) on the first call there; the current device must be the
 * device of `stream` and of the tensors. The call allocates nothing.
 *   A call whose partial results need more than SDPA_DECODE_SCRATCH_BYTES
 *   (sdpa_decode_ws_bytes(...) > that size and more than one key split) returns
 *   SDPA_ERR_WORKSPACE; SDPA_ERR_DEVICE if the device or its scratch address cannot be found.
 *   The scratch keeps the last call's contents; every value the merge reads is written by the
 *   same call first, so nothing needs clearing. Calls that overlap on one GPU (on different
 *   streams, or from different host threads without ordering) share the scratch and race:
 *   order them on one stream.
 */
int sdpa_decode_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                        int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                        int mask_kind, int window, int bias_kind, const void* bias_tbl,
                        void* stream);

/* Static English text for a status code (never NULL). */
const char* sdpa_status_str(int status);

/* SDPA_ABI_VERSION of the built library. */
int sdpa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MI355X_SDPA_H */
