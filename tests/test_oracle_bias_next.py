"""Pins for the oracle's ALiBi bias (R19) and T5 unidirectional buckets (R20), no GPU needed.

  * pure-Python brute force over (b, h, i, j) with both biases computed here from their
    definitions (the bucket by exact integer thresholds, not the oracle's log formula);
  * a library special case: torch's CPU attention in float64 with the bias matrices built
    here with torch ops;
  * the bucket function exhaustively for |rel| < 8192 against its exact integer form
    (thresholds n^16 >= 2^(64 + 3b)), and its properties;
  * ALiBi under a causal mask equals a key-only bias slope * j for O (the -slope * p part is
    constant along a row), with LSE shifted by -slope * p; slope 0 equals no bias;
  * the backward oracle with these biases against finite differences.
Planted mistakes (ALiBi sign, ALiBi without the absolute value, bidirectional buckets for the
decoder table) must each be caught.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import sdpa_ref

THR = []
for _b in range(1, 16):
    _n = 16
    while _n ** 16 < 2 ** (64 + 3 * _b):
        _n += 1
    THR.append(_n)


def t5u_int(rel: int) -> int:
    n = max(-rel, 0)
    return n if n < 16 else 16 + sum(1 for t in THR if n >= t)


def bias_value(kind, bias, h, i_pos, j):
    if kind == 3:
        return -float(bias[h]) * abs(i_pos - j)
    return float(bias[h][t5u_int(j - i_pos)])


def rand(rng, B, Sq, Sk, Hq, Hkv, D, kind):
    q = rng.standard_normal((B, Sq, Hq, D))
    k = rng.standard_normal((B, Sk, Hkv, D))
    v = rng.standard_normal((B, Sk, Hkv, D))
    bias = rng.uniform(0.05, 1.0, Hq) if kind == 3 else rng.standard_normal((Hq, 32))
    return q, k, v, bias


def brute(q, k, v, scale, mask, window, kind, bias):
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    out = np.zeros((B, Sq, Hq, D))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            kh = h * Hkv // Hq
            for i in range(Sq):
                pos = i + Sk - Sq
                sc = []
                for j in range(Sk):
                    if mask >= 1 and j > pos:
                        continue
                    if mask == 2 and pos - j >= window:
                        continue
                    s = sum(q[b, i, h, d] * k[b, j, kh, d] for d in range(D)) * scale
                    sc.append((j, s + bias_value(kind, bias, h, pos, j)))
                if not sc:
                    lse[b, h, i] = -math.inf
                    continue
                m = max(s for _, s in sc)
                w = [(j, math.exp(s - m)) for j, s in sc]
                z = sum(x for _, x in w)
                for d in range(D):
                    out[b, i, h, d] = sum(x * v[b, j, kh, d] for j, x in w) / z
                lse[b, h, i] = m + math.log(z)
    return out, lse


CASES = [  # B, Sq, Sk, Hq, Hkv, D, mask, window, kind
    (1, 5, 5, 2, 1, 3, 1, 0, 3), (1, 4, 7, 2, 2, 3, 0, 0, 3), (1, 6, 6, 2, 1, 2, 2, 3, 3),
    (1, 5, 5, 2, 1, 3, 1, 0, 4), (2, 4, 6, 2, 2, 2, 0, 0, 4), (1, 7, 5, 3, 1, 2, 2, 4, 4)]


def check_brute():
    rng = np.random.default_rng(41)
    for (B, Sq, Sk, Hq, Hkv, D, mask, window, kind) in CASES:
        q, k, v, bias = rand(rng, B, Sq, Sk, Hq, Hkv, D, kind)
        o, l = oracle.sdpa_forward(q, k, v, scale=0.6, mask_kind=mask, window=window,
                                   bias_kind=kind, bias=bias)
        ro, rl = brute(q, k, v, 0.6, mask, window, kind, bias)
        assert np.max(np.abs(o - ro)) <= 1e-12, (kind, mask)
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(l))
        assert np.max(np.abs(l[fin] - rl[fin]), initial=0.0) <= 1e-12


def check_torch():
    rng = np.random.default_rng(42)
    cases = [(2, 64, 64, 4, 2, 16, 1, 0, 3), (1, 70, 90, 4, 1, 8, 0, 0, 3),
             (1, 80, 80, 2, 2, 16, 2, 20, 3), (1, 150, 150, 4, 2, 8, 1, 0, 4),
             (2, 40, 200, 2, 1, 8, 0, 0, 4)]
    for (B, Sq, Sk, Hq, Hkv, D, mask, window, kind) in cases:
        q, k, v, bias = rand(rng, B, Sq, Sk, Hq, Hkv, D, kind)
        scale = 1.0 / math.sqrt(D)
        o, l = oracle.sdpa_forward(q, k, v, scale=scale, mask_kind=mask, window=window,
                                   bias_kind=kind, bias=bias)
        rel = torch.arange(Sk)[None, :] - (torch.arange(Sq)[:, None] + Sk - Sq)
        if kind == 3:
            bm = -torch.from_numpy(bias)[:, None, None] * rel.abs().to(torch.float64)[None]
        else:
            idx = torch.tensor([[t5u_int(int(x)) for x in row] for row in rel.tolist()])
            bm = torch.from_numpy(bias)[:, idx]
        ones = torch.ones(Sq, Sk, dtype=torch.bool)
        vis = ones if mask == 0 else torch.tril(ones, diagonal=Sk - Sq)
        if mask == 2:
            vis = vis & torch.triu(ones, diagonal=Sk - Sq - window + 1)
        am = bm.masked_fill(~vis, float("-inf"))[None].expand(B, Hq, Sq, Sk)
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)
        tk = torch.from_numpy(k).permute(0, 2, 1, 3)
        tv = torch.from_numpy(v).permute(0, 2, 1, 3)
        ro = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=am, scale=scale, enable_gqa=True).permute(0, 2, 1, 3).numpy()
        assert np.max(np.abs(o - ro)) <= 1e-12, (kind, mask)


def test_new_biases_brute_force():
    check_brute()


def test_new_biases_torch_special_case():
    check_torch()


def test_t5u_bucket_exhaustive_and_properties():
    rel = np.arange(-8191, 8192)
    got = oracle.t5u_bucket(rel)
    want = np.array([t5u_int(int(r)) for r in rel])
    assert np.array_equal(got, want)
    assert np.all(got[rel >= 0] == 0)
    n = -rel[rel <= 0][::-1]
    b = oracle.t5u_bucket(-n)
    assert np.all(np.diff(b) >= 0) and b[0] == 0
    assert np.all(b[n < 16] == n[n < 16])
    assert np.all(b[n >= 113] == 31) and b[n == 112][0] == 30
    assert got.min() == 0 and got.max() == 31


def test_alibi_causal_is_key_bias_and_zero_slope_is_no_bias():
    rng = np.random.default_rng(43)
    B, S, Hq, Hkv, D = 2, 40, 4, 2, 8
    q, k, v, slopes = rand(rng, B, S, S, Hq, Hkv, D, 3)
    o, l = oracle.sdpa_forward(q, k, v, scale=0.3, mask_kind=1, bias_kind=3, bias=slopes)
    key_bias = np.broadcast_to(slopes[None, :, None, None] * np.arange(S)[None, None, None, :],
                               (B, Hq, S, S)).copy()
    o2, l2 = oracle.sdpa_forward(q, k, v, scale=0.3, mask_kind=1, bias_kind=2, bias=key_bias)
    assert np.max(np.abs(o - o2)) <= 1e-12
    shift = -slopes[None, :, None] * np.arange(S)[None, None, :]
    assert np.max(np.abs(l - (l2 + shift))) <= 1e-10
    o3, l3 = oracle.sdpa_forward(q, k, v, scale=0.3, mask_kind=0, bias_kind=3,
                                 bias=np.zeros(Hq))
    o4, l4 = oracle.sdpa_forward(q, k, v, scale=0.3, mask_kind=0)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)


def test_backward_with_new_biases_finite_differences():
    rng = np.random.default_rng(44)
    for kind, mask in ((3, 1), (3, 0), (4, 1), (4, 2)):
        q, k, v, bias = rand(rng, 1, 5, 6, 2, 1, 3, kind)
        do = rng.standard_normal(q.shape)
        dq, dk, dv = oracle.sdpa_backward(q, k, v, do, scale=0.7, mask_kind=mask, window=3,
                                          bias_kind=kind, bias=bias)

        def loss(q_, k_, v_):
            o, _ = oracle.sdpa_forward(q_, k_, v_, scale=0.7, mask_kind=mask, window=3,
                                       bias_kind=kind, bias=bias)
            return float(np.sum(do * o))
        eps = 1e-5
        for x, g in ((q, dq), (k, dk), (v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + eps
                lp = loss(q, k, v)
                x[idx] = old - eps
                lm = loss(q, k, v)
                x[idx] = old
                num[idx] = (lp - lm) / (2 * eps)
            assert np.max(np.abs(num - g)) <= 1e-7, (kind, mask)


# ------------------------------------------------------------------------------------------
# planted mistakes
# ------------------------------------------------------------------------------------------
def _mutant(change):
    real = sdpa_ref._bias_rows

    def bad(bias_kind, bias, b, h, q_pos, rows, Sk):
        rel = np.arange(Sk, dtype=np.int64)[None, :] - np.asarray(q_pos, np.int64)[:, None]
        if bias_kind == 3 and change == "alibi_sign":
            return float(bias[h]) * np.abs(rel)
        if bias_kind == 3 and change == "alibi_no_abs":
            return float(bias[h]) * rel
        if bias_kind == 4 and change == "t5u_bidirectional":
            return bias[h][oracle.t5_bucket(rel)]
        return real(bias_kind, bias, b, h, q_pos, rows, Sk)
    return bad


@pytest.mark.parametrize("change", ["alibi_sign", "alibi_no_abs", "t5u_bidirectional"])
def test_pins_catch_new_bias_mistakes(monkeypatch, change):
    monkeypatch.setattr(sdpa_ref, "_bias_rows", _mutant(change))
    caught = False
    for chk in (check_brute, check_torch):
        try:
            chk()
        except AssertionError:
            caught = True
            break
    assert caught
