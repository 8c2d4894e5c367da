"""Pins for the fp64 backward oracle (dQ, dK, dV), no GPU needed.

The backward oracle is trusted because these checks tie it to things other than its formulas:
  * central finite differences of L = sum(dO * O) through the (separately pinned) forward
    oracle, on tiny shapes, for every mask / bias / head-sharing combination;
  * a library special case: torch autograd in float64 through torch's CPU scaled-dot-product
    attention (enable_gqa sums the shared K/V heads' gradients itself), with masks and biases
    built here independently;
  * closed forms: equal V rows give dQ = dK = 0 (O no longer depends on the weights); equal K
    rows give dQ = 0; sum_i Q_i . dQ_i = sum_j K_j . dK_j (both equal scale * sum dS * Q K^T);
    dO = 0 gives zero gradients.
The mutation tests plant plausible mistakes in the oracle and check that a pin catches each.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import sdpa_bwd_ref
from test_oracle import rand_case, t5_bucket_int, torch_band

TOL = 1e-10


def run_bwd(q, k, v, do, scale, mask, window, bk, bias):
    return oracle.sdpa_backward(q, k, v, do, scale=scale, mask_kind=mask, window=window,
                                bias_kind=bk, bias=bias)


def loss(q, k, v, do, scale, mask, window, bk, bias):
    o, _ = oracle.sdpa_forward(q, k, v, scale=scale, mask_kind=mask, window=window,
                               bias_kind=bk, bias=bias)
    return float(np.sum(do * o))


CASES = [  # B, Sq, Sk, Hq, Hkv, D, mask, window, bias_kind
    (1, 5, 5, 2, 1, 3, 0, 0, 0), (1, 5, 7, 2, 2, 3, 1, 0, 0), (1, 6, 6, 2, 1, 2, 2, 3, 0),
    (1, 4, 6, 1, 1, 3, 0, 0, 1), (2, 4, 4, 2, 1, 2, 1, 0, 2), (1, 7, 5, 3, 1, 2, 1, 0, 0)]


def check_finite_differences():
    rng = np.random.default_rng(21)
    eps = 1e-5
    for (B, Sq, Sk, Hq, Hkv, D, mask, window, bk) in CASES:
        q, k, v, bias = rand_case(rng, B, Sq, Sk, Hq, Hkv, D, bk)
        do = rng.standard_normal(q.shape)
        scale = 0.7
        dq, dk, dv = run_bwd(q, k, v, do, scale, mask, window, bk, bias)
        for x, g in ((q, dq), (k, dk), (v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + eps
                lp = loss(q, k, v, do, scale, mask, window, bk, bias)
                x[idx] = old - eps
                lm = loss(q, k, v, do, scale, mask, window, bk, bias)
                x[idx] = old
                num[idx] = (lp - lm) / (2 * eps)
            assert np.max(np.abs(num - g)) <= 1e-7, (B, Sq, Sk, Hq, Hkv, D, mask, window, bk)


def torch_grads(q, k, v, do, scale, mask, window, bk, bias):
    B, Sq, Hq, D = q.shape
    Sk = k.shape[1]
    tq = torch.from_numpy(q).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    am = torch_band(Sq, Sk, mask, window).expand(B, Hq, Sq, Sk).clone()
    if bk == 1:
        rel = np.arange(Sk)[None, :] - (np.arange(Sq)[:, None] + Sk - Sq)
        am = am + torch.from_numpy(bias[:, np.vectorize(t5_bucket_int)(rel)])[None]
    elif bk == 2:
        am = am + torch.from_numpy(bias)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, scale=scale,
                                                         enable_gqa=True)
    o.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    back = lambda t: t.grad.permute(0, 2, 1, 3).numpy()       # noqa: E731
    return back(tq), back(tk), back(tv)


def check_torch_library():
    rng = np.random.default_rng(22)
    cases = [(2, 40, 40, 4, 4, 16, 0, 0, 0), (1, 64, 64, 8, 2, 32, 1, 0, 0),
             (1, 70, 70, 4, 1, 16, 2, 20, 0), (2, 33, 33, 3, 3, 8, 0, 0, 1),
             (1, 30, 30, 2, 2, 16, 0, 0, 2), (1, 50, 50, 2, 1, 8, 2, 50, 1)]
    for (B, Sq, Sk, Hq, Hkv, D, mask, window, bk) in cases:
        q, k, v, bias = rand_case(rng, B, Sq, Sk, Hq, Hkv, D, bk)
        do = rng.standard_normal(q.shape)
        scale = 1.0 / math.sqrt(D)
        got = run_bwd(q, k, v, do, scale, mask, window, bk, bias)
        ref = torch_grads(q, k, v, do, scale, mask, window, bk, bias)
        for a, b in zip(got, ref):
            assert np.max(np.abs(a - b)) <= TOL * max(1.0, np.max(np.abs(b)))


def check_closed_forms():
    rng = np.random.default_rng(23)
    for (B, Sq, Sk, Hq, Hkv, D, mask, window, bk) in CASES + [(1, 20, 24, 4, 2, 8, 1, 0, 1)]:
        q, k, v, bias = rand_case(rng, B, Sq, Sk, Hq, Hkv, D, bk)
        do = rng.standard_normal(q.shape)
        scale = 0.6
        # equal V rows: O = that row whatever the weights, so Q and K get no gradient
        v_eq = np.broadcast_to(v[:, :1], v.shape).copy()
        dq, dk, dv = run_bwd(q, k, v_eq, do, scale, mask, window, bk, bias)
        assert np.max(np.abs(dq)) <= 1e-12 and np.max(np.abs(dk)) <= 1e-12
        # equal K rows with no bias and no mask: uniform weights, dQ = 0
        if bk == 0 and mask == 0:
            k_eq = np.broadcast_to(k[:, :1], k.shape).copy()
            dq, _, _ = run_bwd(q, k_eq, v, do, scale, mask, window, bk, bias)
            assert np.max(np.abs(dq)) <= 1e-12
        # sum Q.dQ == sum K.dK (both scale * sum_ij dS_ij Q_i.K_j)
        dq, dk, dv = run_bwd(q, k, v, do, scale, mask, window, bk, bias)
        a, b = float(np.sum(q * dq)), float(np.sum(k * dk))
        assert abs(a - b) <= 1e-10 * max(1.0, abs(a))
        # dO = 0: no gradient
        z = run_bwd(q, k, v, np.zeros_like(do), scale, mask, window, bk, bias)
        assert all(np.max(np.abs(g)) == 0.0 for g in z)


def test_backward_finite_differences():
    check_finite_differences()


def test_backward_torch_autograd_special_case():
    check_torch_library()


def test_backward_closed_forms():
    check_closed_forms()


def test_backward_kv_heads_restriction():
    rng = np.random.default_rng(24)
    q, k, v, _ = rand_case(rng, 2, 16, 16, 4, 2, 8, 0)
    do = rng.standard_normal(q.shape)
    full = oracle.sdpa_backward(q, k, v, do, scale=0.3, mask_kind=1)
    part = oracle.sdpa_backward(q, k, v, do, scale=0.3, mask_kind=1, kv_heads=[(1, 0)])
    assert np.array_equal(part[0][1, :, 0:2], full[0][1, :, 0:2])
    assert np.array_equal(part[1][1, :, 0], full[1][1, :, 0])
    assert np.max(np.abs(part[2][0])) == 0.0
    thr = oracle.sdpa_backward(q, k, v, do, scale=0.3, mask_kind=1, threads=3)
    assert all(np.array_equal(a, b) for a, b in zip(thr, full))


# ------------------------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# ------------------------------------------------------------------------------------------
ALL = [check_finite_differences, check_torch_library, check_closed_forms]


def _caught(monkeypatch, fn):
    monkeypatch.setattr(sdpa_bwd_ref, "head_backward", fn)
    for chk in ALL:
        try:
            chk()
        except AssertionError:
            return True
    return False


def _mutant(change):
    def bad(q_h, k_h, v_h, do_h, q_pos, scale, mask_kind, window, bias_h=0.0):
        Sk = k_h.shape[0]
        s = (q_h @ k_h.T) * scale + bias_h
        s = np.where(oracle.visible(q_pos, Sk, mask_kind, window), s, -np.inf)
        m = s.max(axis=1)
        m = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(s - m[:, None])
        den = e.sum(axis=1, keepdims=True)
        p = np.divide(e, den, out=np.zeros_like(e), where=den > 0)
        o = p @ v_h
        dv = p.T @ do_h
        dp = do_h @ v_h.T
        corr = (do_h * o).sum(axis=1, keepdims=True)
        if change == "no_softmax_correction":
            corr = 0.0
        ds = p * (dp - corr)
        dq = scale * (ds @ k_h)
        dk = scale * (ds.T @ q_h)
        if change == "dk_without_scale":
            dk = ds.T @ q_h
        if change == "dv_unnormalised":
            dv = e.T @ do_h
        if change == "dq_uses_v":
            dq = scale * (ds @ v_h)
        if change == "correction_by_column":
            ds = p * (dp - (p * dp).sum(axis=0, keepdims=True))
            dq = scale * (ds @ k_h)
            dk = scale * (ds.T @ q_h)
        return dq, dk, dv
    return bad


@pytest.mark.parametrize("change", ["no_softmax_correction", "dk_without_scale", "dv_unnormalised",
                                    "dq_uses_v", "correction_by_column"])
def test_pins_catch_backward_mistakes(monkeypatch, change):
    assert _caught(monkeypatch, _mutant(change))
