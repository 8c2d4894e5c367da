"""Pins for the packed-sequence oracle (oracle.sdpa_forward_varlen), no GPU needed.

The oracle runs each sequence through the forward definition; these checks tie it to things
other than that loop:
  * pure-Python brute force over the packed token axis with a visibility rule written from
    the definition (same sequence, bottom-right positions inside the sequence, window);
  * a library special case: torch's CPU scaled-dot-product attention in float64 over the
    whole pack as one batch, with a block-diagonal mask and T5 bias assembled here with torch;
  * invariants: tokens of one sequence do not change another's outputs (bit for bit);
    sequences without queries or without keys; equal-length packing equals the batched
    forward oracle on the same values.
Planted mistakes (attention across sequences, top-left alignment, a one-token boundary shift)
must each be caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import sdpa_varlen_ref
from test_oracle import t5_bucket_int

TOL = 1e-12


def packed_case(rng, lens_q, lens_k, Hq, Hkv, D, bias_kind):
    tq, tk = sum(lens_q), sum(lens_k)
    q = rng.standard_normal((tq, Hq, D))
    k = rng.standard_normal((tk, Hkv, D))
    v = rng.standard_normal((tk, Hkv, D))
    bias = rng.standard_normal((Hq, 32)) if bias_kind == 1 else None
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int64)
    return q, k, v, bias, cu_q, cu_k


def brute(q, k, v, cu_q, cu_k, scale, mask, window, bias_kind, bias):
    tq, Hq, D = q.shape
    G = Hq // k.shape[1]
    out = np.zeros_like(q)
    lse = np.full((Hq, tq), -np.inf)
    for s in range(len(cu_q) - 1):
        for i in range(int(cu_q[s]), int(cu_q[s + 1])):
            p = (i - int(cu_q[s])) + (int(cu_k[s + 1] - cu_k[s]) - int(cu_q[s + 1] - cu_q[s]))
            for h in range(Hq):
                sc, vs = [], []
                for j in range(int(cu_k[s]), int(cu_k[s + 1])):
                    jj = j - int(cu_k[s])
                    if mask >= 1 and jj > p:
                        continue
                    if mask == 2 and p - jj >= window:
                        continue
                    x = sum(q[i, h, d] * k[j, h // G, d] for d in range(D)) * scale
                    if bias_kind == 1:
                        x += bias[h, t5_bucket_int(jj - p)]
                    sc.append(x)
                    vs.append(v[j, h // G])
                if not sc:
                    continue
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                z = sum(e)
                out[i, h] = sum(w * vv for w, vv in zip(e, vs)) / z
                lse[h, i] = m + math.log(z)
    return out, lse


def torch_pack(q, k, v, cu_q, cu_k, scale, mask, window, bias_kind, bias):
    tq, Hq, D = q.shape
    tk, Hkv = k.shape[0], k.shape[1]
    blocks_vis, blocks_bias = [], []
    for s in range(len(cu_q) - 1):
        nq, nk = int(cu_q[s + 1] - cu_q[s]), int(cu_k[s + 1] - cu_k[s])
        ones = torch.ones(nq, nk, dtype=torch.bool)
        off = nk - nq
        vis = ones if mask == 0 else torch.tril(ones, diagonal=off)
        if mask == 2:
            vis = vis & torch.triu(ones, diagonal=off - window + 1)
        blocks_vis.append(vis.to(torch.float64))
        rel = torch.arange(nk)[None, :] - (torch.arange(nq)[:, None] + off)
        blocks_bias.append(rel.to(torch.float64))
    vis = torch.block_diag(*blocks_vis) > 0.5
    rel = torch.block_diag(*blocks_bias).to(torch.int64)
    am = torch.zeros(Hq, tq, tk, dtype=torch.float64).masked_fill(~vis, float("-inf"))
    if bias_kind == 1:
        idx = torch.tensor([[t5_bucket_int(int(x)) for x in row] for row in rel.tolist()])
        am = am + torch.from_numpy(bias)[:, idx]
    tq_ = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk_ = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv_ = torch.from_numpy(v).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(tq_, tk_, tv_, attn_mask=am[None],
                                                         scale=scale, enable_gqa=True)
    o = o[0].permute(1, 0, 2).numpy()
    # rows with no visible key: torch returns NaN there; the definition gives 0 (R8)
    empty = ~vis.any(dim=1).numpy()
    o[empty] = 0.0
    return o, empty


CASES = [  # lens_q, lens_k, Hq, Hkv, D, mask, window, bias_kind
    ([3, 5, 2], [3, 5, 2], 2, 1, 4, 1, 0, 0),
    ([4, 0, 3], [6, 2, 3], 2, 2, 3, 1, 0, 1),
    ([5, 2, 4], [5, 4, 4], 3, 1, 2, 2, 2, 0),
    ([3, 3], [3, 0], 2, 1, 3, 0, 0, 0),
    ([6, 1, 3], [6, 1, 7], 2, 1, 3, 2, 3, 1),
]


def check_brute():
    rng = np.random.default_rng(31)
    for (lq, lk, Hq, Hkv, D, mask, window, bk) in CASES:
        q, k, v, bias, cu_q, cu_k = packed_case(rng, lq, lk, Hq, Hkv, D, bk)
        got = oracle.sdpa_forward_varlen(q, k, v, cu_q, cu_k, scale=0.7, mask_kind=mask,
                                         window=window, bias_kind=bk, bias=bias)
        ref = brute(q, k, v, cu_q, cu_k, 0.7, mask, window, bk, bias)
        assert np.max(np.abs(got[0] - ref[0])) <= TOL, (lq, lk, mask)
        fin = np.isfinite(ref[1])
        assert np.array_equal(fin, np.isfinite(got[1]))
        assert np.max(np.abs(got[1][fin] - ref[1][fin]), initial=0.0) <= TOL


def check_torch():
    rng = np.random.default_rng(32)
    cases = [([40, 17, 64, 3], [40, 17, 64, 3], 4, 2, 16, 1, 0, 0),
             ([30, 50, 21], [45, 50, 60], 4, 1, 8, 2, 13, 1),
             ([33, 0, 70], [33, 12, 70], 2, 2, 8, 0, 0, 1)]
    for (lq, lk, Hq, Hkv, D, mask, window, bk) in cases:
        q, k, v, bias, cu_q, cu_k = packed_case(rng, lq, lk, Hq, Hkv, D, bk)
        scale = 1.0 / math.sqrt(D)
        got, _ = oracle.sdpa_forward_varlen(q, k, v, cu_q, cu_k, scale=scale, mask_kind=mask,
                                            window=window, bias_kind=bk, bias=bias)
        ref, _ = torch_pack(q, k, v, cu_q, cu_k, scale, mask, window, bk, bias)
        assert np.max(np.abs(got - ref)) <= 1e-12


def test_varlen_brute_force():
    check_brute()


def test_varlen_torch_block_diagonal_special_case():
    check_torch()


def test_sequences_do_not_see_each_other():
    rng = np.random.default_rng(33)
    q, k, v, bias, cu_q, cu_k = packed_case(rng, [20, 30, 25], [20, 30, 25], 4, 2, 8, 1)
    a = oracle.sdpa_forward_varlen(q, k, v, cu_q, cu_k, scale=0.4, mask_kind=1, bias_kind=1,
                                   bias=bias)
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[20:50] += 1.0
    v2[20:50] -= 2.0
    q2[20:50] *= 3.0
    b = oracle.sdpa_forward_varlen(q2, k2, v2, cu_q, cu_k, scale=0.4, mask_kind=1, bias_kind=1,
                                   bias=bias)
    for sl in (slice(0, 20), slice(50, 75)):
        assert np.array_equal(a[0][sl], b[0][sl]) and np.array_equal(a[1][:, sl], b[1][:, sl])
    assert not np.array_equal(a[0][20:50], b[0][20:50])


def test_empty_sequences_and_keyless_rows():
    rng = np.random.default_rng(34)
    q, k, v, _, cu_q, cu_k = packed_case(rng, [0, 4, 3, 0], [5, 0, 3, 2], 2, 1, 4, 0)
    o, l = oracle.sdpa_forward_varlen(q, k, v, cu_q, cu_k, scale=0.5, mask_kind=1)
    assert o.shape == (7, 2, 4) and l.shape == (2, 7)
    assert np.all(o[0:4] == 0.0) and np.all(np.isneginf(l[:, 0:4]))
    assert np.all(np.isfinite(l[:, 4:7]))


def test_equal_lengths_equal_the_batched_forward():
    rng = np.random.default_rng(35)
    B, S, Hq, Hkv, D = 3, 24, 4, 2, 8
    qb = rng.standard_normal((B, S, Hq, D))
    kb = rng.standard_normal((B, S, Hkv, D))
    vb = rng.standard_normal((B, S, Hkv, D))
    cu = np.arange(B + 1) * S
    o, l = oracle.sdpa_forward_varlen(qb.reshape(B * S, Hq, D), kb.reshape(B * S, Hkv, D),
                                      vb.reshape(B * S, Hkv, D), cu, cu, scale=0.3,
                                      mask_kind=2, window=7)
    ob, lb = oracle.sdpa_forward(qb, kb, vb, scale=0.3, mask_kind=2, window=7)
    assert np.array_equal(o, ob.reshape(B * S, Hq, D))
    assert np.array_equal(l, lb.transpose(1, 0, 2).reshape(Hq, B * S))


# ------------------------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# ------------------------------------------------------------------------------------------
def _mutant(kind):
    real = sdpa_varlen_ref.sdpa_forward

    def bad(q, k, v, cu_q, cu_k, *, scale, mask_kind, window=0, bias_kind=0, bias=None,
            threads=None):
        if kind == "no_document_mask":
            o, l = real(q[None], k[None], v[None], scale=scale, mask_kind=mask_kind,
                        window=window, bias_kind=bias_kind, bias=bias)
            return o[0], l[0]
        total_q, Hq, D = q.shape
        out = np.zeros((total_q, Hq, D))
        lse = np.full((Hq, total_q), -np.inf)
        for s in range(len(cu_q) - 1):
            a, b = int(cu_q[s]), int(cu_q[s + 1])
            c, d = int(cu_k[s]), int(cu_k[s + 1])
            if kind == "boundary_shift" and s > 0:
                c -= 1
            if b == a or d == c:
                continue
            qq, kk, vv = q[None, a:b], k[None, c:d], v[None, c:d]
            if kind == "top_left" and (d - c) != (b - a):
                # align row i with key i instead of the last keys
                n = b - a
                kk, vv = k[None, c:c + max(n, 1)], v[None, c:c + max(n, 1)]
            o, l = real(qq, kk, vv, scale=scale, mask_kind=mask_kind, window=window,
                        bias_kind=bias_kind, bias=bias)
            out[a:b] = o[0]
            lse[:, a:b] = l[0]
        return out, lse
    return bad


@pytest.mark.parametrize("kind", ["no_document_mask", "top_left", "boundary_shift"])
def test_pins_catch_varlen_mistakes(monkeypatch, kind):
    monkeypatch.setattr(oracle, "sdpa_forward_varlen", _mutant(kind))
    caught = False
    for chk in (check_brute, check_torch):
        try:
            chk()
        except AssertionError:
            caught = True
            break
    assert caught
