// C ABI of the fused attention forward and backward (declared in include/sdpa.h): argument
// validation and dispatch to the gfx950 kernels. Every check runs before any HIP call, so an
// invalid call returns its status without touching the device.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "sdpa.h"
#include "sdpa_decode.h"
#include "sdpa_params.h"

namespace sdpa {
hipError_t launch_fwd_bf16(FwdParams p, int D, int mask, int bias, bool out_f32, hipStream_t s);
hipError_t fwd_bf16_workgroups(FwdParams p, int D, int bias, long long* workgroups);
hipError_t launch_fwd_f32(FwdParams p, int D, int mask, int bias, hipStream_t s);
hipError_t launch_bwd_bf16(BwdParams p, int D, int mask, int bias, bool out_f32, hipStream_t s);
hipError_t launch_decode_bf16(DecParams p, int D, int mask, int bias, bool out_f32, hipStream_t s);
hipError_t decode_scratch(void** ptr);
}  // namespace sdpa

namespace {

constexpr long long kMaxElems = 1LL << 40;

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

int validate(const void* q, const void* k, const void* v, const void* out, const float* lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale, int mask_kind,
             int window, int bias_kind, const void* bias_tbl, int elem_bytes) {
    if (!q || !k || !v || !out || !lse) return SDPA_ERR_NULL;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1) return SDPA_ERR_SHAPE;
    if (Hq % Hkv != 0) return SDPA_ERR_HEADS;
    if (D != 32 && D != 64 && D != 128 && D != 256) return SDPA_ERR_HEADDIM;
    if (mask_kind != SDPA_MASK_NONE && mask_kind != SDPA_MASK_CAUSAL &&
        mask_kind != SDPA_MASK_SLIDING)
        return SDPA_ERR_MASK;
    if (mask_kind == SDPA_MASK_SLIDING && window < 1) return SDPA_ERR_WINDOW;
    if (bias_kind < SDPA_BIAS_NONE || bias_kind > SDPA_BIAS_T5U) return SDPA_ERR_BIAS;
    if ((bias_kind == SDPA_BIAS_NONE) != (bias_tbl == nullptr)) return SDPA_ERR_BIAS;
    if (!isfinite(scale)) return SDPA_ERR_SCALE;
    const long long qe = (long long)B * Sq * Hq * D;
    const long long ke = (long long)B * Sk * Hkv * D;
    if (qe >= kMaxElems || ke >= kMaxElems) return SDPA_ERR_SHAPE;
    if (bias_kind == SDPA_BIAS_FULL && (long long)B * Hq * Sq * Sk >= kMaxElems) return SDPA_ERR_SHAPE;
    // one batch of q/out or k/v is addressed with 32-bit element offsets inside the kernels
    if ((long long)Sq * Hq * D >= (1LL << 31) || (long long)Sk * Hkv * D >= (1LL << 31))
        return SDPA_ERR_SHAPE;
    // grid: one workgroup per 64-row (fp32) or 128-row (bf16) query tile of each (b, head)
    if ((long long)B * Hq * ((Sq + 63) / 64) >= (1LL << 31)) return SDPA_ERR_SHAPE;
    if (elem_bytes == 4 && (B > 65535 || Hq > 65535)) return SDPA_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(lse, 4))
        return SDPA_ERR_ALIGN;
    if ((bias_kind == SDPA_BIAS_T5 || bias_kind == SDPA_BIAS_T5U || bias_kind == SDPA_BIAS_ALIBI) &&
        !aligned(bias_tbl, 4))
        return SDPA_ERR_ALIGN;
    if (bias_kind == SDPA_BIAS_FULL && !aligned(bias_tbl, 16)) return SDPA_ERR_ALIGN;
    return SDPA_OK;
}

// The mask kind the kernels run. A sliding window at least as wide as the key range hides
// nothing the causal mask shows (a visible key has pos - j <= Sk - 1 < window), so it runs the
// causal kernels: exactly the causal result and the causal speed, which the transformers issue
// on the SDPA mask fix asks of a window equal to the sequence length.
int kernel_mask(int mask_kind, int window, int Sk) {
    return (mask_kind == SDPA_MASK_SLIDING && window >= Sk) ? SDPA_MASK_CAUSAL : mask_kind;
}

sdpa::FwdParams make_params(const void* q, const void* k, const void* v, void* out, float* lse,
                            int B, int Hq, int Hkv, int Sq, int Sk, float scale, int mask_kind,
                            int window, const void* bias_tbl) {
    sdpa::FwdParams p{};
    p.q = q; p.k = k; p.v = v; p.out = out; p.lse = lse; p.bias = bias_tbl;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Sq = Sq; p.Sk = Sk;
    p.G = Hq / Hkv;
    p.off = Sk - Sq;
    // Sliding windows wider than the key range are the causal mask: clamp so window
    // arithmetic stays in range (the visible set is unchanged).
    p.window = (mask_kind == SDPA_MASK_SLIDING) ? (window > Sk ? Sk + 1 : window) : 0;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    return p;
}

int validate_bwd(const void* q, const void* k, const void* v, const void* out,
                 const float* lse, const void* dout, const void* dq, const void* dk,
                 const void* dv, const float* ws, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                 float scale, int mask_kind, int window, int bias_kind, const void* bias_tbl) {
    if (!dout || !dq || !dk || !dv || !ws) return SDPA_ERR_NULL;
    int st = validate(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, window,
                      bias_kind, bias_tbl, 2);
    if (st != SDPA_OK) return st;
    // grid of the dK/dV kernel: one workgroup per 128 keys (64 at D = 256) of each (b, KV head)
    if ((long long)B * Hkv * ((Sk + 63) / 64) >= (1LL << 31)) return SDPA_ERR_SHAPE;
    if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        !aligned(ws, 4))
        return SDPA_ERR_ALIGN;
    return SDPA_OK;
}

sdpa::BwdParams make_bwd_params(const void* q, const void* k, const void* v, const void* out,
                                const float* lse, const void* dout, void* dq, void* dk,
                                void* dv, float* ws, int B, int Hq, int Hkv, int Sq, int Sk,
                                float scale, int mask_kind, int window, const void* bias_tbl) {
    const sdpa::FwdParams f = make_params(q, k, v, const_cast<void*>(out), const_cast<float*>(lse),
                                          B, Hq, Hkv, Sq, Sk, scale, mask_kind, window, bias_tbl);
    sdpa::BwdParams p{};
    p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse; p.dout = dout;
    p.dq = dq; p.dk = dk; p.dv = dv; p.delta = ws; p.bias = bias_tbl;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Sq = Sq; p.Sk = Sk;
    p.G = f.G; p.off = f.off; p.window = f.window;
    p.scale = f.scale; p.scale_log2 = f.scale_log2;
    return p;
}

bool dec_shape_ok(int B, int Hq, int Hkv, int Sq, int Sk, int D) {
    return B >= 1 && Hq >= 1 && Hkv >= 1 && Sq >= 1 && Sk >= 1 && Hq % Hkv == 0 &&
           (D == 32 || D == 64 || D == 128 || D == 256) && (long long)Sq * (Hq / Hkv) < (1LL << 30);
}

// Checks of a decode call that need no workspace; *splits receives the key-split count.
int validate_decode(const void* q, const void* k, const void* v, const void* out,
                    const float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                    float scale, int mask_kind, int window, int bias_kind, const void* bias_tbl,
                    long long* splits) {
    int st = validate(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, window,
                      bias_kind, bias_tbl, 2);
    if (st != SDPA_OK) return st;
    const int G = Hq / Hkv;
    if ((long long)Sq * G >= (1LL << 30)) return SDPA_ERR_SHAPE;
    // grids: split kernel B * Hkv * row blocks * splits, merge kernel up to 4 per row block
    const long long blocks = (long long)B * Hkv * sdpa::dec_row_blocks(G, Sq);
    *splits = sdpa::dec_splits(B, Hkv, G, Sq, Sk);
    if (blocks * (*splits > 4 ? *splits : 4) >= (1LL << 31)) return SDPA_ERR_SHAPE;
    return SDPA_OK;
}

// Launch of a validated decode call with its partial-result buffer `ws`.
int run_decode(const void* q, const void* k, const void* v, void* out, float* lse, void* ws,
               int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale, int mask_kind,
               int window, int bias_kind, const void* bias_tbl, void* stream, bool out_f32) {
    const sdpa::FwdParams f = make_params(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, scale,
                                          mask_kind, window, bias_tbl);
    sdpa::DecParams p{};
    p.q = q; p.k = k; p.v = v; p.out = out; p.lse = lse; p.ws = (float*)ws; p.bias = bias_tbl;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Sq = Sq; p.Sk = Sk;
    p.G = f.G; p.off = f.off; p.window = f.window;
    p.scale = f.scale; p.scale_log2 = f.scale_log2;
    hipError_t e = sdpa::launch_decode_bf16(p, D, kernel_mask(mask_kind, window, Sk), bias_kind, out_f32,
                                            (hipStream_t)stream);
    return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

int decode_common(const void* q, const void* k, const void* v, void* out, float* lse, void* ws,
                  size_t ws_bytes, int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                  int mask_kind, int window, int bias_kind, const void* bias_tbl, void* stream,
                  bool out_f32) {
    long long splits = 0;
    int st = validate_decode(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, window,
                             bias_kind, bias_tbl, &splits);
    if (st != SDPA_OK) return st;
    if (!ws || !aligned(ws, 16) ||
        ws_bytes < sdpa::dec_ws_floats(B, Hkv, Hq / Hkv, Sq, Sk, D) * sizeof(float))
        return SDPA_ERR_WORKSPACE;
    return run_decode(q, k, v, out, lse, ws, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, window,
                      bias_kind, bias_tbl, stream, out_f32);
}

int varlen_common(const void* q, const void* k, const void* v, void* out, float* lse,
                  const int* cu_q, const int* cu_k, int n_seqs, int total_q, int total_k,
                  int max_q, int max_k, int Hq, int Hkv, int D, float scale, int mask_kind,
                  int window, int bias_kind, const void* bias_tbl, void* stream, bool out_f32) {
    if (!cu_q || !cu_k) return SDPA_ERR_NULL;
    if (n_seqs < 1 || total_q < 1 || total_k < 1 || max_q < 1 || max_k < 1) return SDPA_ERR_SHAPE;
    if (bias_kind == SDPA_BIAS_FULL) return SDPA_ERR_BIAS;
    // the per-token checks of the dense forward, on one packed "batch" of total tokens
    int st = validate(q, k, v, out, lse, 1, Hq, Hkv, total_q, total_k, D, scale, mask_kind,
                      window, bias_kind, bias_tbl, 2);
    if (st != SDPA_OK) return st;
    // grid: one workgroup per 128- or 256-row query tile of each (sequence, head)
    if ((long long)n_seqs * Hq * ((max_q + 127) / 128) >= (1LL << 31)) return SDPA_ERR_SHAPE;
    if (!aligned(cu_q, 4) || !aligned(cu_k, 4)) return SDPA_ERR_ALIGN;
    sdpa::FwdParams p = make_params(q, k, v, out, lse, n_seqs, Hq, Hkv, max_q, max_k, scale,
                                    mask_kind, window, bias_tbl);
    p.cu_q = cu_q;
    p.cu_k = cu_k;
    p.total_q = total_q;
    p.total_k = total_k;
    hipError_t e = sdpa::launch_fwd_bf16(p, D, kernel_mask(mask_kind, window, max_k), bias_kind, out_f32,
                                         (hipStream_t)stream);
    return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

}  // namespace

static_assert(sdpa::kDecodeScratchBytes == SDPA_DECODE_SCRATCH_BYTES, "scratch size");

extern "C" {

int sdpa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int n_seqs, int total_q,
                    int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int D,
                    float scale, int mask_kind, int window, int bias_kind, const void* bias_tbl,
                    void* stream) {
    return varlen_common(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, n_seqs, total_q, total_k,
                         max_seqlen_q, max_seqlen_k, Hq, Hkv, D, scale, mask_kind, window,
                         bias_kind, bias_tbl, stream, false);
}

int sdpa_fwd_varlen_f32out(const void* q, const void* k, const void* v, float* out, float* lse,
                           const int* cu_seqlens_q, const int* cu_seqlens_k, int n_seqs,
                           int total_q, int total_k, int max_seqlen_q, int max_seqlen_k, int Hq,
                           int Hkv, int D, float scale, int mask_kind, int window, int bias_kind,
                           const void* bias_tbl, void* stream) {
    return varlen_common(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, n_seqs, total_q, total_k,
                         max_seqlen_q, max_seqlen_k, Hq, Hkv, D, scale, mask_kind, window,
                         bias_kind, bias_tbl, stream, true);
}

size_t sdpa_decode_ws_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int D) {
    if (!dec_shape_ok(B, Hq, Hkv, Sq, Sk, D)) return 0;
    return sdpa::dec_ws_floats(B, Hkv, Hq / Hkv, Sq, Sk, D) * sizeof(float);
}

int sdpa_decode(const void* q, const void* k, const void* v, void* out, float* lse, void* ws,
                size_t ws_bytes, int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                int mask_kind, int window, int bias_kind, const void* bias_tbl, void* stream) {
    return decode_common(q, k, v, out, lse, ws, ws_bytes, B, Hq, Hkv, Sq, Sk, D, scale,
                         mask_kind, window, bias_kind, bias_tbl, stream, false);
}

int sdpa_decode_f32out(const void* q, const void* k, const void* v, float* out, float* lse,
                       void* ws, size_t ws_bytes, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                       float scale, int mask_kind, int window, int bias_kind,
                       const void* bias_tbl, void* stream) {
    return decode_common(q, k, v, out, lse, ws, ws_bytes, B, Hq, Hkv, Sq, Sk, D, scale,
                         mask_kind, window, bias_kind, bias_tbl, stream, true);
}

int sdpa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
             int Hkv, int Sq, int Sk, int D, float scale, int mask_kind, int window,
             int bias_kind, const void* bias_tbl, void* stream) {
    int st = validate(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, window,
                      bias_kind, bias_tbl, 2);
    if (st != SDPA_OK) return st;
    sdpa::FwdParams p = make_params(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, scale, mask_kind,
                                    window, bias_tbl);
    hipError_t e = sdpa::launch_fwd_bf16(p, D, kernel_mask(mask_kind, window, Sk), bias_kind, false,
                                         (hipStream_t)stream);
    return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

int sdpa_fwd_bf16_f32out(const void* q, const void* k, const void* v, float* out, float* lse,
                         int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                         int mask_kind, int window, int bias_kind, const void* bias_tbl,
                         void* stream) {
    int st = validate(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, window,
                      bias_kind, bias_tbl, 2);
    if (st != SDPA_OK) return st;
    sdpa::FwdParams p = make_params(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, scale, mask_kind,
                                    window, bias_tbl);
    hipError_t e = sdpa::launch_fwd_bf16(p, D, kernel_mask(mask_kind, window, Sk), bias_kind, true,
                                         (hipStream_t)stream);
    return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

int sdpa_fwd_f32(const float* q, const float* k, const float* v, float* out, float* lse, int B,
                 int Hq, int Hkv, int Sq, int Sk, int D, float scale, int mask_kind, int window,
                 int bias_kind, const void* bias_tbl, void* stream) {
    int st = validate(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, window,
                      bias_kind, bias_tbl, 4);
    if (st != SDPA_OK) return st;
    sdpa::FwdParams p = make_params(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, scale, mask_kind,
                                    window, bias_tbl);
    hipError_t e = sdpa::launch_fwd_f32(p, D, kernel_mask(mask_kind, window, Sk), bias_kind, (hipStream_t)stream);
    return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

int sdpa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, float* ws, int B, int Hq, int Hkv,
             int Sq, int Sk, int D, float scale, int mask_kind, int window, int bias_kind,
             const void* bias_tbl, void* stream) {
    int st = validate_bwd(q, k, v, out, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, Sq, Sk, D, scale,
                          mask_kind, window, bias_kind, bias_tbl);
    if (st != SDPA_OK) return st;
    sdpa::BwdParams p = make_bwd_params(q, k, v, out, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, Sq,
                                        Sk, scale, mask_kind, window, bias_tbl);
    hipError_t e = sdpa::launch_bwd_bf16(p, D, kernel_mask(mask_kind, window, Sk), bias_kind, false,
                                         (hipStream_t)stream);
    return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

int sdpa_bwd_f32out(const void* q, const void* k, const void* v, const void* out,
                    const float* lse, const void* dout, float* dq, float* dk, float* dv,
                    float* ws, int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                    int mask_kind, int window, int bias_kind, const void* bias_tbl,
                    void* stream) {
    int st = validate_bwd(q, k, v, out, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, Sq, Sk, D, scale,
                          mask_kind, window, bias_kind, bias_tbl);
    if (st != SDPA_OK) return st;
    sdpa::BwdParams p = make_bwd_params(q, k, v, out, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, Sq,
                                        Sk, scale, mask_kind, window, bias_tbl);
    hipError_t e = sdpa::launch_bwd_bf16(p, D, kernel_mask(mask_kind, window, Sk), bias_kind, true,
                                         (hipStream_t)stream);
    return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

int sdpa_decode_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                        int B, int Hq, int Hkv, int Sq, int Sk, int D, float scale,
                        int mask_kind, int window, int bias_kind, const void* bias_tbl,
                        void* stream) {
    long long splits = 0;
    int st = validate_decode(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, window,
                             bias_kind, bias_tbl, &splits);
    if (st != SDPA_OK) return st;
    // a single split writes the output directly and leaves the partial-result buffer unused
    if (splits > 1 && sdpa::dec_ws_floats(B, Hkv, Hq / Hkv, Sq, Sk, D) * sizeof(float) >
                          (size_t)SDPA_DECODE_SCRATCH_BYTES)
        return SDPA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (sdpa::decode_scratch(&ws) != hipSuccess) return SDPA_ERR_DEVICE;
    return run_decode(q, k, v, out, lse, ws, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, window,
                      bias_kind, bias_tbl, stream, false);
}

int sdpa_fwd_launch_grid(int B, int Hq, int Hkv, int Sq, int Sk, int D, int mask_kind,
                         int window, int bias_kind, long long* workgroups) {
    if (!workgroups) return SDPA_ERR_NULL;
    // the shape checks of sdpa_fwd, with stand-in buffers (nothing is read or launched)
    alignas(16) static const unsigned char stand_in[16] = {0};
    const void* b = stand_in;
    int st = validate(b, b, b, b, (const float*)b, B, Hq, Hkv, Sq, Sk, D, 1.0f, mask_kind,
                      window, bias_kind, bias_kind == SDPA_BIAS_NONE ? nullptr : b, 2);
    if (st != SDPA_OK) return st;
    const sdpa::FwdParams p = make_params(b, b, b, const_cast<void*>(b), (float*)b, B, Hq, Hkv,
                                          Sq, Sk, 1.0f, mask_kind, window,
                                          bias_kind == SDPA_BIAS_NONE ? nullptr : b);
    long long wg = 0;
    if (sdpa::fwd_bf16_workgroups(p, D, bias_kind, &wg) != hipSuccess) return SDPA_ERR_HEADDIM;
    *workgroups = wg;
    return SDPA_OK;
}

const char* sdpa_status_str(int status) {
    switch (status) {
        case SDPA_OK: return "ok";
        case SDPA_ERR_NULL: return "a required pointer is NULL";
        case SDPA_ERR_SHAPE: return "invalid or too large shape (B, Hq, Hkv, Sq, Sk)";
        case SDPA_ERR_HEADS: return "Hq is not a multiple of Hkv";
        case SDPA_ERR_HEADDIM: return "head dim D must be 32, 64, 128 or 256";
        case SDPA_ERR_MASK: return "unknown mask_kind";
        case SDPA_ERR_WINDOW: return "sliding window must be >= 1";
        case SDPA_ERR_BIAS: return "unknown bias_kind or bias_tbl inconsistent with it";
        case SDPA_ERR_SCALE: return "scale is not finite";
        case SDPA_ERR_ALIGN: return "pointer misaligned (q/k/v/out/full bias need 16 bytes)";
        case SDPA_ERR_LAUNCH: return "HIP kernel launch failed";
        case SDPA_ERR_WORKSPACE: return "workspace NULL, misaligned (16 bytes) or too small";
        case SDPA_ERR_DEVICE: return "current device unknown or its scratch buffer not found";
        default: return "unknown status";
    }
}

int sdpa_abi_version(void) { return SDPA_ABI_VERSION; }

}  // extern "C"
