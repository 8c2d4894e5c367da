"""fp64 CPU oracle for the gradients of the attention forward (dQ, dK, dV).

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import it. It shares no code with the HIP path.

What it computes: the gradients of L = sum(dO * O) with respect to Q, K and V, where O is the
forward of sdpa_ref (the four steps of scaled dot-product attention of the
"jax-gpu-05-attention-gpu" codelab, section 1, with the masks, biases and head sharing of the
forward oracle). The pages use the backward pass without printing it: the FAT5 README reports
backward TFLOPS of its biased flash kernels, and the transformers issue "Transformer models are
not deterministic when using Flash Attention 2" is about run-to-run equality of a
training step. The formulas are the chain rule through the definition, for one (batch,
query head) with P = softmax(S) row-wise and S = scale * Q K^T + bias (masked entries -inf):

    dV   = P^T dO                       (O = P V)
    dP   = dO V^T
    dS   = P * (dP - rowsum(dO * O))    (softmax Jacobian: rowsum(P * dP) = rowsum(dO * O))
    dQ   = scale * dS K
    dK   = scale * dS^T Q

A K/V head shared by G query heads (GQA / MQA, codelab section 9) receives the sum of the G
heads' dK and dV. Masked pairs have P = 0 and contribute nothing; a row with no visible key
has O = 0 and zero gradients. The bias is an input here and gets no gradient.

Readings: R1-R5 and R8 of the forward oracle; in addition
  R14 the gradients are those of the exact fp64 forward (no bf16 rounding of P or O): the
      GPU path's rounding is part of its error budget, not of the definition.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

from .sdpa_ref import (BIAS_ALIBI, BIAS_FULL, BIAS_NONE, BIAS_T5, BIAS_T5U, t5_bucket,
                       t5u_bucket, visible)


def _bias(bias_kind, bias, b, h, q_pos, Sk):
    if bias_kind == BIAS_NONE:
        return 0.0
    if bias_kind == BIAS_T5:
        rel = np.arange(Sk, dtype=np.int64)[None, :] - np.asarray(q_pos, np.int64)[:, None]
        return bias[h][t5_bucket(rel)]
    if bias_kind == BIAS_FULL:
        return bias[b, h]
    rel = np.arange(Sk, dtype=np.int64)[None, :] - np.asarray(q_pos, np.int64)[:, None]
    if bias_kind == BIAS_ALIBI:
        return -float(bias[h]) * np.abs(rel).astype(np.float64)
    if bias_kind == BIAS_T5U:
        return bias[h][t5u_bucket(rel)]
    raise ValueError(f"unknown bias kind {bias_kind}")


def head_backward(q_h, k_h, v_h, do_h, q_pos, scale, mask_kind, window, bias_h=0.0):
    """Gradients for one (batch, query head): q_h [Sq, D], k_h / v_h [Sk, D], do_h [Sq, D].

    Returns (dq_h [Sq, D], dk_h [Sk, D], dv_h [Sk, D]) of L = sum(do_h * O).
    """
    Sk = k_h.shape[0]
    s = (q_h @ k_h.T) * scale + bias_h
    s = np.where(visible(q_pos, Sk, mask_kind, window), s, -np.inf)
    m = s.max(axis=1)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m[:, None])
    den = e.sum(axis=1, keepdims=True)
    p = np.divide(e, den, out=np.zeros_like(e), where=den > 0)     # softmax rows (0 if empty)
    o = p @ v_h
    dv = p.T @ do_h
    dp = do_h @ v_h.T
    ds = p * (dp - (do_h * o).sum(axis=1, keepdims=True))
    dq = scale * (ds @ k_h)
    dk = scale * (ds.T @ q_h)
    return dq, dk, dv


def sdpa_backward(q, k, v, dout, *, scale: float, mask_kind: int, window: int = 0,
                  bias_kind: int = BIAS_NONE, bias=None, threads: Optional[int] = None,
                  kv_heads: Optional[Sequence[tuple]] = None):
    """(dq [B, Sq, Hq, D], dk [B, Sk, Hkv, D], dv [B, Sk, Hkv, D]) in float64.

    q, dout [B, Sq, Hq, D]; k, v [B, Sk, Hkv, D]; bias as in the forward oracle. `kv_heads`
    optionally restricts the work to a list of (b, kv_head) pairs (their G query heads' dq rows
    and the pair's dk, dv; everything else stays 0). `threads` runs pairs on a thread pool.
    """
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    q_pos = np.arange(Sq, dtype=np.int64) + (Sk - Sq)          # R2
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    pairs = list(kv_heads) if kv_heads is not None else [(b, kh) for b in range(B)
                                                           for kh in range(Hkv)]

    def one(pair):
        b, kh = pair
        for h in range(kh * G, (kh + 1) * G):                 # R3: the group of kv head kh
            g_q, g_k, g_v = head_backward(q[b, :, h, :], k[b, :, kh, :], v[b, :, kh, :],
                                          dout[b, :, h, :], q_pos, scale, mask_kind, window,
                                          _bias(bias_kind, bias, b, h, q_pos, Sk))
            dq[b, :, h, :] = g_q
            dk[b, :, kh, :] += g_k
            dv[b, :, kh, :] += g_v

    nthr = threads or 1
    if nthr <= 1:
        for pr in pairs:
            one(pr)
    else:
        with ThreadPoolExecutor(max_workers=nthr) as ex:
            list(ex.map(one, pairs))
    return dq, dk, dv
