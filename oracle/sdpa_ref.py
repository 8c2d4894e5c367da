"""fp64 CPU oracle for the scaled-dot-product attention forward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import it. It shares no code with the HIP path.

What it computes (one (batch, query-head) at a time, plain steps, no blocking beyond
independent query rows):

  * the four steps of scaled dot-product attention -- score Q.K^T, scale by 1/sqrt(d_k) and
    softmax over keys, weighted sum of V, output with Q's shape -- as defined in the
    "jax-gpu-05-attention-gpu" codelab, section 1 ("Dikkat nasil calisir?") and its naive
    implementation in section 4, and in the Medium post "Simplified Explanation of Attention",
    steps 1-4 of "Scaled Dot-Product Attention";
  * an additive bias on the scores before the softmax: a full [B, H, Sq, Sk] tensor, or a T5
    bucketed relative-position bias looked up from a [H, 32] table (FAT5 / flashT5 README,
    list of supported attention biases);
  * a causal mask (codelab section 7, is_causal=True) and a sliding-window causal mask
    (transformers issue "Slowdown in Training Speed Due to SDPA Mask Fix in Version 4.40.0");
  * GQA / MQA head sharing, K/V heads broadcast over query-head groups (codelab section 9);
  * the row log-sum-exp of the final (scaled, biased, masked) scores.

Readings where the pages are silent (each also listed in the design notes):
  R1 sliding window: key j is visible from query position p iff 0 <= p - j < window, so a
     query sees exactly `window` keys including itself; window >= Sk equals plain causal.
  R2 causal alignment when Sq != Sk: bottom-right, query row i sits at position
     p = i + (Sk - Sq) (the KV-cache reading of the Medium post's KV-cache section).
  R3 GQA grouping: query head h uses KV head h // (Hq // Hkv) (codelab section 9: "each
     shared by 4 query heads", contiguous groups).
  R4 T5 bucket: the T5 bidirectional scheme -- 32 buckets split 16/16 by the sign of the
     relative position j - p, 8 exact buckets per half, the rest log-spaced up to distance 128
     and saturating beyond. Written here as the T5 real-valued log formula in fp64.
  R5 T5 table layout: fp32 [Hq][32], row h holds the 32 bucket values of head h.
  R8 a query row with no visible key gives O = 0 and LSE = -inf.
  R9 LSE = natural log of sum_j exp(s'_ij) where s' includes scale and bias.
  R19 ALiBi (named in the FAT5 README's list of attention biases, not defined there): the
     score of (query position p, key j) in head h gets -slope[h] * |p - j|, slopes an fp32
     [Hq] table given by the caller (for causal rows this is the ALiBi paper's
     slope * (j - p)).
  R20 T5 unidirectional (decoder) buckets: keys at or after the query share bucket 0; a key
     n = p - j positions back gets bucket n for n < 16, else 16 + floor(16 log(n/16) / log 8)
     capped at 31 (the T5 formula with bidirectional=False, 32 buckets, max distance 128).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

MASK_NONE, MASK_CAUSAL, MASK_SLIDING = 0, 1, 2
BIAS_NONE, BIAS_T5, BIAS_FULL, BIAS_ALIBI, BIAS_T5U = 0, 1, 2, 3, 4

T5_NUM_BUCKETS = 32
T5_MAX_DISTANCE = 128

# Row chunk: query rows are independent in the definition, so they are processed in chunks only
# to bound the memory of the [rows, Sk] score block.
_ROW_CHUNK = 512


def t5_bucket(rel) -> np.ndarray:
    """T5 bidirectional relative-position bucket of rel = key_position - query_position.

    Reading R4 (the pages name the scheme -- T5-like relative position encoding, FAT5 README --
    but do not print it). Half of the 32 buckets go to keys after the query (rel > 0). Within a
    half, distances n < 8 get their own bucket; larger n get
        8 + floor( log(n / 8) / log(128 / 8) * (16 - 8) ),
    capped at 15, i.e. log-spaced from 8 to 128 and saturating beyond 128.
    """
    rel = np.asarray(rel, dtype=np.int64)
    half = T5_NUM_BUCKETS // 2            # 16 buckets per direction
    max_exact = half // 2                 # 8 exact buckets
    n = np.abs(rel)
    nn = np.maximum(n, max_exact).astype(np.float64)   # log only evaluated where n >= 8
    large = max_exact + np.floor(np.log(nn / max_exact)
                                 / math.log(T5_MAX_DISTANCE / max_exact)
                                 * (half - max_exact)).astype(np.int64)
    large = np.minimum(large, half - 1)
    bucket = np.where(n < max_exact, n, large)
    return bucket + np.where(rel > 0, half, 0)


def t5u_bucket(rel) -> np.ndarray:
    """T5 unidirectional bucket of rel = key_position - query_position (R20), the T5
    real-valued formula in fp64: n = max(-rel, 0); n below 16 exact; otherwise
    16 + floor(16 * log(n / 16) / log(128 / 16)), capped at 31."""
    rel = np.asarray(rel, dtype=np.int64)
    n = np.maximum(-rel, 0)
    nf = np.maximum(n, 1).astype(np.float64)
    large = 16 + np.floor(np.log(nf / 16.0) / math.log(128.0 / 16.0) * 16.0).astype(np.int64)
    return np.where(n < 16, n, np.minimum(large, 31))


def visible(q_pos: np.ndarray, Sk: int, mask_kind: int, window: int) -> np.ndarray:
    """Boolean [n, Sk]: may query at absolute position q_pos[r] see key j?  (R1, R2)"""
    j = np.arange(Sk, dtype=np.int64)[None, :]
    p = np.asarray(q_pos, dtype=np.int64)[:, None]
    if mask_kind == MASK_NONE:
        return np.ones((p.shape[0], Sk), dtype=bool)
    if mask_kind == MASK_CAUSAL:
        return j <= p
    if mask_kind == MASK_SLIDING:
        return (j <= p) & (p - j < window)
    raise ValueError(f"unknown mask kind {mask_kind}")


def attend_rows(q_rows: np.ndarray, k_head: np.ndarray, v_head: np.ndarray, q_pos: np.ndarray,
                scale: float, mask_kind: int, window: int,
                bias_rows: Optional[np.ndarray] = None):
    """Attention for a set of query rows of one (batch, head).

    q_rows [n, D], k_head / v_head [Sk, D], q_pos [n] absolute query positions, bias_rows
    [n, Sk] (additive, already gathered) or None. All float64.
    Returns (out [n, D], lse [n]).
    """
    Sk = k_head.shape[0]
    # Step 1, score: each query against every key.  Step 2, scale by 1/sqrt(d_k) (given).
    s = (q_rows @ k_head.T) * scale
    # Additive bias on the scaled scores (FAT5 README: attention biases).
    if bias_rows is not None:
        s = s + bias_rows
    # Mask: invisible pairs get -inf, i.e. weight exactly 0 after the softmax.
    s = np.where(visible(q_pos, Sk, mask_kind, window), s, -np.inf)
    # Step 3, softmax over keys, with its log-normaliser.
    m = s.max(axis=1)
    has_key = np.isfinite(m)
    m_safe = np.where(has_key, m, 0.0)
    p = np.exp(s - m_safe[:, None])
    denom = p.sum(axis=1)
    # Step 4, weighted sum of the value rows.
    num = p @ v_head
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(has_key[:, None], num / np.where(has_key, denom, 1.0)[:, None], 0.0)
        lse = np.where(has_key, m_safe + np.log(np.where(has_key, denom, 1.0)), -np.inf)
    return out, lse


def attention_weights(q_rows, k_head, q_pos, scale, mask_kind, window, bias_rows=None):
    """The softmax weights P [n, Sk] of the same definition (for invariant checks)."""
    s = (q_rows @ k_head.T) * scale
    if bias_rows is not None:
        s = s + bias_rows
    s = np.where(visible(q_pos, k_head.shape[0], mask_kind, window), s, -np.inf)
    m = s.max(axis=1)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m[:, None])
    d = p.sum(axis=1, keepdims=True)
    return np.divide(p, d, out=np.zeros_like(p), where=d > 0)


def _bias_rows(bias_kind, bias, b, h, q_pos, rows, Sk):
    if bias_kind == BIAS_NONE:
        return None
    if bias_kind == BIAS_T5:
        rel = np.arange(Sk, dtype=np.int64)[None, :] - np.asarray(q_pos, np.int64)[:, None]
        return bias[h][t5_bucket(rel)]          # table [Hq][32]
    if bias_kind == BIAS_FULL:
        return bias[b, h][np.asarray(rows)]     # [B, Hq, Sq, Sk]
    rel = np.arange(Sk, dtype=np.int64)[None, :] - np.asarray(q_pos, np.int64)[:, None]
    if bias_kind == BIAS_ALIBI:
        return -float(bias[h]) * np.abs(rel).astype(np.float64)     # slopes [Hq] (R19)
    if bias_kind == BIAS_T5U:
        return bias[h][t5u_bucket(rel)]                              # table [Hq][32] (R20)
    raise ValueError(f"unknown bias kind {bias_kind}")


def sdpa_rows(q, k, v, b: int, h: int, rows: Sequence[int], *, scale: float, mask_kind: int,
              window: int = 0, bias_kind: int = BIAS_NONE, bias=None):
    """Selected output rows of one (batch b, query head h).

    q [B, Sq, Hq, D], k / v [B, Sk, Hkv, D] float64 (layout of codelab section 3: batch,
    sequence, heads, head dim); bias: [Hq, 32] table for T5, [B, Hq, Sq, Sk] for full.
    Returns (out [len(rows), D], lse [len(rows)]).
    """
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    kh = h // (Hq // Hkv)                       # R3
    rows = np.asarray(rows, dtype=np.int64)
    q_pos = rows + (Sk - Sq)                    # R2
    return attend_rows(q[b, rows, h, :], k[b, :, kh, :], v[b, :, kh, :], q_pos, scale,
                       mask_kind, window, _bias_rows(bias_kind, bias, b, h, q_pos, rows, Sk))


def sdpa_forward(q, k, v, *, scale: float, mask_kind: int, window: int = 0,
                 bias_kind: int = BIAS_NONE, bias=None, threads: Optional[int] = None,
                 heads: Optional[Sequence[tuple]] = None):
    """Full forward: out [B, Sq, Hq, D] (Q's shape) and lse [B, Hq, Sq], both float64.

    `heads` optionally restricts the work to a list of (b, h) pairs (other entries stay 0 /
    -inf). `threads` runs (b, h) pairs on a thread pool (numpy releases the GIL in matmul).
    """
    B, Sq, Hq, D = q.shape
    out = np.zeros((B, Sq, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq, Sq), -np.inf, dtype=np.float64)
    pairs = list(heads) if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]

    def one(bh):
        b, h = bh
        for r0 in range(0, Sq, _ROW_CHUNK):
            rows = np.arange(r0, min(Sq, r0 + _ROW_CHUNK))
            o, l = sdpa_rows(q, k, v, b, h, rows, scale=scale, mask_kind=mask_kind,
                             window=window, bias_kind=bias_kind, bias=bias)
            out[b, rows, h, :] = o
            lse[b, h, rows] = l

    nthr = threads or 1
    if nthr <= 1:
        for bh in pairs:
            one(bh)
    else:
        with ThreadPoolExecutor(max_workers=nthr) as ex:
            list(ex.map(one, pairs))
    return out, lse


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1
