"""MI355X (gfx950) fused scaled-dot-product attention forward and its gradients.

Thin Python binding over the C ABI in include/sdpa.h (libsdpa_mi355x.so, built in-tree by
scaled_dot_product_03_amd.build). This module only marshals arguments: torch supplies device
memory and the current stream, every step of the attention runs in the HIP kernels. There is no
fallback: if the library is missing, calls raise.

    out, lse = fwd(q, k, v, mask="causal")           # q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D]
    dq, dk, dv = bwd(q, k, v, out, lse, dout, mask="causal")
    out, lse = decode(q_new, k_cache, v_cache, mask="causal")   # few rows, long cache
    out, lse = fwd_varlen(q_packed, k_packed, v_packed, cu_q, cu_k, max_q, max_k)

Layout follows the "jax-gpu-05-attention-gpu" codelab, section 3 (batch, sequence, heads,
head dim). lse is [B, Hq, Sq] fp32 (natural log).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libsdpa_mi355x.so"

MASK_NONE, MASK_CAUSAL, MASK_SLIDING = 0, 1, 2
BIAS_NONE, BIAS_T5, BIAS_FULL, BIAS_ALIBI, BIAS_T5U = 0, 1, 2, 3, 4
_MASKS = {"none": MASK_NONE, "causal": MASK_CAUSAL, "sliding": MASK_SLIDING}
_BIASES = {"none": BIAS_NONE, "t5": BIAS_T5, "full": BIAS_FULL, "alibi": BIAS_ALIBI,
           "t5u": BIAS_T5U}

SDPA_OK = 0
STATUS_NAMES = {0: "SDPA_OK", 1: "SDPA_ERR_NULL", 2: "SDPA_ERR_SHAPE", 3: "SDPA_ERR_HEADS",
                4: "SDPA_ERR_HEADDIM", 5: "SDPA_ERR_MASK", 6: "SDPA_ERR_WINDOW",
                7: "SDPA_ERR_BIAS", 8: "SDPA_ERR_SCALE", 9: "SDPA_ERR_ALIGN",
                10: "SDPA_ERR_LAUNCH", 11: "SDPA_ERR_WORKSPACE", 12: "SDPA_ERR_DEVICE"}

# symbols exported by the library (must match include/sdpa.h)
ENTRY_POINTS = ("sdpa_fwd", "sdpa_fwd_bf16_f32out", "sdpa_fwd_f32", "sdpa_bwd",
                "sdpa_bwd_f32out", "sdpa_decode_ws_bytes", "sdpa_decode", "sdpa_decode_f32out",
                "sdpa_fwd_varlen", "sdpa_fwd_varlen_f32out", "sdpa_decode_noalloc",
                "sdpa_fwd_launch_grid", "sdpa_status_str", "sdpa_abi_version")
ABI_VERSION = 4
DECODE_SCRATCH_BYTES = 16 << 20     # SDPA_DECODE_SCRATCH_BYTES

_lib = None


class SdpaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def lib_path() -> str:
    return os.path.join(PKG, LIB_NAME)


def load():
    """Load the shared library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m scaled_dot_product_03_amd.build`")
    # torch first: the library must bind to the HIP runtime torch already uses (torch ships its
    # own copy under the same soname). Loaded before torch, the library would pull in the
    # system runtime and the process would end up with two HIP runtimes, whose streams, device
    # state and errors are not each other's.
    import torch  # noqa: F401
    L = ctypes.CDLL(path)
    fwd_args = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [ctypes.c_float] + \
               [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_void_p]
    for name in ("sdpa_fwd", "sdpa_fwd_bf16_f32out", "sdpa_fwd_f32"):
        fn = getattr(L, name)
        fn.argtypes = fwd_args
        fn.restype = ctypes.c_int
    bwd_args = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 6 + [ctypes.c_float] + \
               [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_void_p]
    for name in ("sdpa_bwd", "sdpa_bwd_f32out"):
        fn = getattr(L, name)
        fn.argtypes = bwd_args
        fn.restype = ctypes.c_int
    L.sdpa_decode_ws_bytes.argtypes = [ctypes.c_int] * 6
    L.sdpa_decode_ws_bytes.restype = ctypes.c_size_t
    L.sdpa_fwd_launch_grid.argtypes = [ctypes.c_int] * 9 + [ctypes.POINTER(ctypes.c_longlong)]
    L.sdpa_fwd_launch_grid.restype = ctypes.c_int
    dec_args = [ctypes.c_void_p] * 6 + [ctypes.c_size_t] + [ctypes.c_int] * 6 + \
               [ctypes.c_float] + [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_void_p]
    for name in ("sdpa_decode", "sdpa_decode_f32out"):
        fn = getattr(L, name)
        fn.argtypes = dec_args
        fn.restype = ctypes.c_int
    L.sdpa_decode_noalloc.argtypes = fwd_args
    L.sdpa_decode_noalloc.restype = ctypes.c_int
    vl_args = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 8 + [ctypes.c_float] + \
              [ctypes.c_int] * 3 + [ctypes.c_void_p, ctypes.c_void_p]
    for name in ("sdpa_fwd_varlen", "sdpa_fwd_varlen_f32out"):
        fn = getattr(L, name)
        fn.argtypes = vl_args
        fn.restype = ctypes.c_int
    L.sdpa_status_str.argtypes = [ctypes.c_int]
    L.sdpa_status_str.restype = ctypes.c_char_p
    L.sdpa_abi_version.argtypes = []
    L.sdpa_abi_version.restype = ctypes.c_int
    _lib = L
    return L


def status_str(status: int) -> str:
    return load().sdpa_status_str(status).decode()


def call_raw(entry: str, q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, window,
             bias_kind, bias, stream) -> int:
    """Call an entry point with raw integer pointers; returns the status code."""
    fn = getattr(load(), entry)
    return fn(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, D, ctypes.c_float(scale), mask_kind, window,
              bias_kind, bias, stream)


def call_raw_bwd(entry: str, q, k, v, out, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, Sq, Sk, D,
                 scale, mask_kind, window, bias_kind, bias, stream) -> int:
    """Call a backward entry point with raw integer pointers; returns the status code."""
    fn = getattr(load(), entry)
    return fn(q, k, v, out, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, Sq, Sk, D,
              ctypes.c_float(scale), mask_kind, window, bias_kind, bias, stream)


def call_raw_decode(entry: str, q, k, v, out, lse, ws, ws_bytes, B, Hq, Hkv, Sq, Sk, D, scale,
                    mask_kind, window, bias_kind, bias, stream) -> int:
    """Call a decode entry point with raw integer pointers; returns the status code."""
    fn = getattr(load(), entry)
    return fn(q, k, v, out, lse, ws, ws_bytes, B, Hq, Hkv, Sq, Sk, D, ctypes.c_float(scale),
              mask_kind, window, bias_kind, bias, stream)


def call_raw_varlen(entry: str, q, k, v, out, lse, cu_q, cu_k, n_seqs, total_q, total_k,
                    max_q, max_k, Hq, Hkv, D, scale, mask_kind, window, bias_kind, bias,
                    stream) -> int:
    """Call a packed-sequence entry point with raw integer pointers; returns the status."""
    fn = getattr(load(), entry)
    return fn(q, k, v, out, lse, cu_q, cu_k, n_seqs, total_q, total_k, max_q, max_k, Hq, Hkv, D,
              ctypes.c_float(scale), mask_kind, window, bias_kind, bias, stream)


def decode_ws_bytes(B, Hq, Hkv, Sq, Sk, D) -> int:
    """Workspace bytes sdpa_decode needs for this shape (0 for an invalid shape)."""
    return int(load().sdpa_decode_ws_bytes(B, Hq, Hkv, Sq, Sk, D))


def fwd_launch_grid(B, Hq, Hkv, Sq, Sk, D, *, mask="causal", window=0, bias_kind="none") -> int:
    """Workgroups the bf16 forward launches for this shape on the current device: one per
    query tile, or the persistent grid (CU count rounded down to a multiple of 8)."""
    L = load()
    wg = ctypes.c_longlong(0)
    st = L.sdpa_fwd_launch_grid(B, Hq, Hkv, Sq, Sk, D, _kind(mask, _MASKS, "mask"), window,
                                _kind(bias_kind, _BIASES, "bias kind"), ctypes.byref(wg))
    if st != 0:
        raise SdpaError(st, L.sdpa_status_str(st).decode())
    return int(wg.value)


def _kind(val, table, what):
    if isinstance(val, str):
        if val not in table:
            raise ValueError(f"unknown {what} {val!r}")
        return table[val]
    return int(val)


def _check_qkv(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, S, H, D]")
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if (Bk, Dk) != (B, D) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch between q, k, v")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError("q, k, v must be contiguous cuda tensors on one device")
    return B, Sq, Hq, D, Sk, Hkv


def _check_buf(t, name, shape, dtype, device):
    """A caller-supplied output or workspace tensor: it must have exactly the shape and dtype
    the entry point writes, live on the inputs' device and be contiguous. The C ABI only sees
    a raw pointer, so this is the last place a wrong buffer can be caught before the kernels
    write through it."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device \
            or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape "
                         f"{list(shape)} on {device} (got {t.dtype} {list(t.shape)} on "
                         f"{t.device}, contiguous={t.is_contiguous()})")
    return t


def _check_ws(t, name, nbytes, device):
    """A caller-supplied workspace: contiguous, on the inputs' device, at least `nbytes`."""
    have = t.numel() * t.element_size()
    if t.device != device or not t.is_contiguous() or have < nbytes:
        raise ValueError(f"{name} must be a contiguous tensor of at least {nbytes} bytes on "
                         f"{device} (got {have} bytes on {t.device}, "
                         f"contiguous={t.is_contiguous()})")
    return t


def _bias_ptr(bk, bias, dtype, B, Hq, Sq, Sk):
    import torch

    if bk in (BIAS_T5, BIAS_T5U):
        if bias is None or bias.dtype != torch.float32 or tuple(bias.shape) != (Hq, 32) \
                or not bias.is_contiguous() or not bias.is_cuda:
            raise ValueError("t5 bias must be a contiguous cuda fp32 [Hq, 32] table")
        return bias.data_ptr()
    if bk == BIAS_ALIBI:
        if bias is None or bias.dtype != torch.float32 or tuple(bias.shape) != (Hq,) \
                or not bias.is_contiguous() or not bias.is_cuda:
            raise ValueError("alibi bias must be a contiguous cuda fp32 [Hq] slope table")
        return bias.data_ptr()
    if bk == BIAS_FULL:
        if bias is None or bias.dtype != dtype or tuple(bias.shape) != (B, Hq, Sq, Sk) \
                or not bias.is_contiguous() or not bias.is_cuda:
            raise ValueError("full bias must be a contiguous cuda [B, Hq, Sq, Sk] tensor "
                             "in the input dtype")
        return bias.data_ptr()
    if bias is not None:
        raise ValueError("bias given with bias_kind='none'")
    return None


def fwd(q, k, v, *, scale: Optional[float] = None, mask="causal", window: int = 0,
        bias_kind="none", bias=None, out=None, lse=None, out_dtype=None, stream=None):
    """Fused attention forward on the current HIP stream. Returns (out, lse).

    q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D]: contiguous cuda tensors, all bf16 or all fp32.
    mask: "none" | "causal" | "sliding" (window keys, including the query's own position).
    bias_kind: "none" | "t5" / "t5u" (bias = fp32 table [Hq, 32], bidirectional or decoder
    buckets) | "alibi" (bias = fp32 slopes [Hq]) | "full" (bias [B, Hq, Sq, Sk] in the input
    dtype). out_dtype: torch.float32 with bf16 inputs selects the fp32 epilogue.
    """
    import torch

    L = load()
    B, Sq, Hq, D, Sk, Hkv = _check_qkv(q, k, v)
    mk = _kind(mask, _MASKS, "mask")
    bk = _kind(bias_kind, _BIASES, "bias kind")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if q.dtype == torch.bfloat16:
        odt = out_dtype or torch.bfloat16
        entry = "sdpa_fwd" if odt == torch.bfloat16 else "sdpa_fwd_bf16_f32out"
        if odt not in (torch.bfloat16, torch.float32):
            raise ValueError("out_dtype must be bf16 or fp32")
    elif q.dtype == torch.float32:
        odt = torch.float32
        entry = "sdpa_fwd_f32"
        if out_dtype not in (None, torch.float32):
            raise ValueError("fp32 inputs produce fp32 output")
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    bias_ptr = _bias_ptr(bk, bias, q.dtype, B, Hq, Sq, Sk)
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=odt, device=q.device)
    _check_buf(out, "out", (B, Sq, Hq, D), odt, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _check_buf(lse, "lse", (B, Hq, Sq), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = getattr(L, entry)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), B, Hq, Hkv, Sq, Sk, D, ctypes.c_float(scale), mk,
                           int(window), bk, bias_ptr, stream)
    if st != SDPA_OK:
        raise SdpaError(st, L.sdpa_status_str(st).decode())
    return out, lse


def bwd(q, k, v, out, lse, dout, *, scale: Optional[float] = None, mask="causal",
        window: int = 0, bias_kind="none", bias=None, grad_dtype=None, ws=None, dq=None,
        dk=None, dv=None, stream=None):
    """Gradients (dq, dk, dv) of sum(dout * out) on the current HIP stream.

    q, k, v, out, dout bf16 (out, lse from fwd with the same arguments); lse [B, Hq, Sq] fp32.
    grad_dtype: torch.bfloat16 (default) or torch.float32 for dq, dk, dv. ws: optional fp32
    workspace of B*Hq*Sq elements (allocated here when None).
    """
    import torch

    L = load()
    B, Sq, Hq, D, Sk, Hkv = _check_qkv(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError("the backward takes bf16 q, k, v")
    _check_buf(out, "out", (B, Sq, Hq, D), torch.bfloat16, q.device)
    _check_buf(dout, "dout", (B, Sq, Hq, D), torch.bfloat16, q.device)
    _check_buf(lse, "lse", (B, Hq, Sq), torch.float32, q.device)
    mk = _kind(mask, _MASKS, "mask")
    bk = _kind(bias_kind, _BIASES, "bias kind")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    gdt = grad_dtype or torch.bfloat16
    if gdt not in (torch.bfloat16, torch.float32):
        raise ValueError("grad_dtype must be bf16 or fp32")
    entry = "sdpa_bwd" if gdt == torch.bfloat16 else "sdpa_bwd_f32out"
    bias_ptr = _bias_ptr(bk, bias, q.dtype, B, Hq, Sq, Sk)
    if dq is None:
        dq = torch.empty((B, Sq, Hq, D), dtype=gdt, device=q.device)
    if dk is None:
        dk = torch.empty((B, Sk, Hkv, D), dtype=gdt, device=q.device)
    if dv is None:
        dv = torch.empty((B, Sk, Hkv, D), dtype=gdt, device=q.device)
    _check_buf(dq, "dq", (B, Sq, Hq, D), gdt, q.device)
    _check_buf(dk, "dk", (B, Sk, Hkv, D), gdt, q.device)
    _check_buf(dv, "dv", (B, Sk, Hkv, D), gdt, q.device)
    if ws is None:
        ws = torch.empty((B * Hq * Sq,), dtype=torch.float32, device=q.device)
    if ws.dtype != torch.float32:
        raise ValueError("ws must be an fp32 tensor")
    _check_ws(ws, "ws", 4 * B * Hq * Sq, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = getattr(L, entry)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                           dv.data_ptr(), ws.data_ptr(), B, Hq, Hkv, Sq, Sk, D,
                           ctypes.c_float(scale), mk, int(window), bk, bias_ptr, stream)
    if st != SDPA_OK:
        raise SdpaError(st, L.sdpa_status_str(st).decode())
    return dq, dk, dv


def decode(q, k, v, *, scale: Optional[float] = None, mask="causal", window: int = 0,
           bias_kind="none", bias=None, out=None, lse=None, out_dtype=None, ws=None,
           stream=None):
    """Split-key decode on the current HIP stream (few query rows against a long K/V cache).
    Same arguments and results as fwd for bf16 inputs; ws is an optional uint8 device buffer
    of at least decode_ws_bytes(...) bytes (allocated here when None)."""
    import torch

    L = load()
    B, Sq, Hq, D, Sk, Hkv = _check_qkv(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError("decode takes bf16 q, k, v")
    mk = _kind(mask, _MASKS, "mask")
    bk = _kind(bias_kind, _BIASES, "bias kind")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    odt = out_dtype or torch.bfloat16
    if odt not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be bf16 or fp32")
    entry = "sdpa_decode" if odt == torch.bfloat16 else "sdpa_decode_f32out"
    bias_ptr = _bias_ptr(bk, bias, q.dtype, B, Hq, Sq, Sk)
    need = decode_ws_bytes(B, Hq, Hkv, Sq, Sk, D)
    if ws is None:
        ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    _check_ws(ws, "ws", need, q.device)
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=odt, device=q.device)
    _check_buf(out, "out", (B, Sq, Hq, D), odt, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _check_buf(lse, "lse", (B, Hq, Sq), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = getattr(L, entry)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(), B, Hq,
                           Hkv, Sq, Sk, D, ctypes.c_float(scale), mk, int(window), bk, bias_ptr,
                           stream)
    if st != SDPA_OK:
        raise SdpaError(st, L.sdpa_status_str(st).decode())
    return out, lse


def decode_noalloc(q, k, v, out, lse, *, scale: Optional[float] = None, mask="causal",
                   window: int = 0, bias_kind="none", bias=None, stream=None):
    """decode() for callers that cannot allocate: same results, bit for bit, as decode() with
    bf16 output, but the per-split partials go to the library's static per-GPU scratch array
    instead of a workspace. The caller passes the outputs: out [B, Sq, Hq, D] bf16 and
    lse [B, Hq, Sq] fp32; nothing is allocated here or in the library. Calls that overlap on one
    GPU share the scratch: issue them on one stream."""
    import torch

    L = load()
    B, Sq, Hq, D, Sk, Hkv = _check_qkv(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError("decode takes bf16 q, k, v")
    _check_buf(out, "out", (B, Sq, Hq, D), torch.bfloat16, q.device)
    _check_buf(lse, "lse", (B, Hq, Sq), torch.float32, q.device)
    mk = _kind(mask, _MASKS, "mask")
    bk = _kind(bias_kind, _BIASES, "bias kind")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    bias_ptr = _bias_ptr(bk, bias, q.dtype, B, Hq, Sq, Sk)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = L.sdpa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, Hq, Hkv, Sq, Sk, D, ctypes.c_float(scale), mk,
                               int(window), bk, bias_ptr, stream)
    if st != SDPA_OK:
        raise SdpaError(st, L.sdpa_status_str(st).decode())
    return out, lse


def fwd_varlen(q, k, v, cu_q, cu_k, max_seqlen_q: int, max_seqlen_k: int, *,
               scale: Optional[float] = None, mask="causal", window: int = 0, bias_kind="none",
               bias=None, out=None, lse=None, out_dtype=None, stream=None):
    """Packed variable-length sequences on the current HIP stream. Returns (out, lse).

    q [total_q, Hq, D], k/v [total_k, Hkv, D] contiguous bf16 cuda tensors; cu_q, cu_k int32
    cuda tensors of n + 1 offsets; lse is [Hq, total_q]. bias_kind "none" or "t5".
    """
    import torch

    L = load()
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or tuple(k.shape) != tuple(v.shape):
        raise ValueError("q [total_q, Hq, D], k and v [total_k, Hkv, D] expected")
    total_q, Hq, D = q.shape
    total_k, Hkv, Dk = k.shape
    if Dk != D or q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must be bf16 with one head dim")
    for t in (q, k, v, cu_q, cu_k):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("inputs must be contiguous cuda tensors")
    if cu_q.dtype != torch.int32 or cu_k.dtype != torch.int32 or cu_q.numel() != cu_k.numel():
        raise ValueError("cu_q and cu_k must be int32 tensors of equal length")
    n = cu_q.numel() - 1
    mk = _kind(mask, _MASKS, "mask")
    bk = _kind(bias_kind, _BIASES, "bias kind")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    odt = out_dtype or torch.bfloat16
    entry = "sdpa_fwd_varlen" if odt == torch.bfloat16 else "sdpa_fwd_varlen_f32out"
    if bk == BIAS_FULL:
        raise ValueError("packed sequences take no full bias")
    bias_ptr = _bias_ptr(bk, bias, q.dtype, 1, Hq, 1, 1)
    if odt not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be bf16 or fp32")
    if out is None:
        out = torch.empty((total_q, Hq, D), dtype=odt, device=q.device)
    _check_buf(out, "out", (total_q, Hq, D), odt, q.device)
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    _check_buf(lse, "lse", (Hq, total_q), torch.float32, q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    st = getattr(L, entry)(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), cu_q.data_ptr(), cu_k.data_ptr(), n, total_q, total_k,
                           int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, D,
                           ctypes.c_float(scale), mk, int(window), bk, bias_ptr, stream)
    if st != SDPA_OK:
        raise SdpaError(st, L.sdpa_status_str(st).decode())
    return out, lse
