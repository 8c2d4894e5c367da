"""fp64 CPU oracle for the attention forward over packed variable-length sequences.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import it. It shares no code with the HIP path.

What it computes: several sequences packed back to back along the token axis (training with
packing, transformers issue "Slowdown in Training Speed Due to SDPA Mask Fix in Version
4.40.0", the SFT trainer's packing=True; dynamic batching of the FAT5 README), each attending
only to itself: the packed problem is the forward of sdpa_ref with a block-diagonal document
mask. Sequence s owns query tokens cu_q[s] .. cu_q[s+1]-1 and key tokens cu_k[s] ..
cu_k[s+1]-1; inside it the masks, biases and head sharing of the forward apply with the
sequence's own lengths (bottom-right alignment R2 per sequence, relative positions for the T5
bias counted inside the sequence).

Readings: R1-R5, R8, R9 of the forward oracle, and
  R18 packed layout: q [total_q, Hq, D], k / v [total_k, Hkv, D] (the forward's layout without
      the batch axis), offsets cu_q / cu_k of n + 1 nondecreasing integers from 0; out has
      q's shape, lse is [Hq, total_q]. A sequence with no query tokens contributes nothing; a
      query token of a sequence with no keys gets O = 0 and LSE = -inf. A full additive bias
      is not defined for packed sequences (no [B, H, Sq, Sk] frame): biases are none or T5.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .sdpa_ref import BIAS_FULL, BIAS_NONE, sdpa_forward


def sdpa_forward_varlen(q, k, v, cu_q, cu_k, *, scale: float, mask_kind: int, window: int = 0,
                        bias_kind: int = BIAS_NONE, bias=None, threads: Optional[int] = None):
    """(out [total_q, Hq, D], lse [Hq, total_q]) in float64: each sequence through the forward
    definition on its own slice (a batch of one)."""
    if bias_kind == BIAS_FULL:
        raise ValueError("a full bias is not defined for packed sequences")
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    total_q, Hq, D = q.shape
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    lse = np.full((Hq, total_q), -np.inf, dtype=np.float64)
    for s in range(len(cu_q) - 1):
        a, b = int(cu_q[s]), int(cu_q[s + 1])
        c, d = int(cu_k[s]), int(cu_k[s + 1])
        if b == a:
            continue
        if d == c:
            continue                      # no keys: O = 0, LSE = -inf (already set)
        o, l = sdpa_forward(q[None, a:b], k[None, c:d], v[None, c:d], scale=scale,
                            mask_kind=mask_kind, window=window, bias_kind=bias_kind,
                            bias=bias, threads=threads)
        out[a:b] = o[0]
        lse[:, a:b] = l[0]
    return out, lse
