"""Pins for the fp64 CPU oracle (runs without a GPU).

The oracle is trusted only because these checks tie it to things other than itself:
  * a pure-Python triple loop written independently here (brute force, tiny shapes);
  * a library special case: torch's CPU flash-attention op in float64, with masks and biases
    built here independently of the oracle;
  * hand-derived closed-form cases (tests/golden/hand_cases.json);
  * invariants the pages fix (rows sum to 1, Q=0 gives the mean of visible V, causal row 0 is
    V[0], window >= Sk equals causal, the causal last row equals the unmasked last row, ...);
  * the T5 bucket against an exact integer formulation, exhaustively.
The mutation tests at the end plant plausible mistakes in the oracle and check that at least one
pin catches each.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import sdpa_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")
TOL = 1e-12


# ------------------------------------------------------------------------------------------
# helpers written independently of the oracle
# ------------------------------------------------------------------------------------------
def t5_bucket_int(rel: int) -> int:
    """Exact integer form of the T5 bidirectional bucket.

    For n >= 8 the real formula is 8 + floor(8*log(n/8)/log 16) = 8 + floor(2*log2(n) - 6),
    i.e. 2 + floor(log2(n^2)) = 1 + bit_length(n^2); capped at 15.
    """
    n = abs(rel)
    b = n if n < 8 else min(15, 1 + (n * n).bit_length())
    return b + (16 if rel > 0 else 0)


def brute_force(q, k, v, scale, mask, window, bias_kind, bias):
    """Plain Python loops over (b, h, i, j); q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] nested lists."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    out = np.zeros((B, Sq, Hq, D))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            kh = h * Hkv // Hq
            for i in range(Sq):
                pos = i + Sk - Sq
                scores = []
                for j in range(Sk):
                    if mask == 1 and j > pos:
                        continue
                    if mask == 2 and (j > pos or pos - j >= window):
                        continue
                    s = sum(float(q[b, i, h, d]) * float(k[b, j, kh, d]) for d in range(D)) * scale
                    if bias_kind == 1:
                        s += float(bias[h][t5_bucket_int(j - pos)])
                    elif bias_kind == 2:
                        s += float(bias[b, h, i, j])
                    scores.append((j, s))
                if not scores:
                    lse[b, h, i] = -math.inf
                    continue
                mx = max(s for _, s in scores)
                w = [(j, math.exp(s - mx)) for j, s in scores]
                z = sum(x for _, x in w)
                for d in range(D):
                    out[b, i, h, d] = sum(x * float(v[b, j, kh, d]) for j, x in w) / z
                lse[b, h, i] = mx + math.log(z)
    return out, lse


def rand_case(rng, B, Sq, Sk, Hq, Hkv, D, bias_kind):
    q = rng.standard_normal((B, Sq, Hq, D))
    k = rng.standard_normal((B, Sk, Hkv, D))
    v = rng.standard_normal((B, Sk, Hkv, D))
    bias = None
    if bias_kind == 1:
        bias = rng.standard_normal((Hq, 32))
    elif bias_kind == 2:
        bias = 0.5 * rng.standard_normal((B, Hq, Sq, Sk))
    return q, k, v, bias


def run_oracle(q, k, v, scale, mask, window, bias_kind, bias):
    return oracle.sdpa_forward(q, k, v, scale=scale, mask_kind=mask, window=window,
                               bias_kind=bias_kind, bias=bias)


# ------------------------------------------------------------------------------------------
# pin checks (plain functions so the mutation tests can re-run them against a broken oracle)
# ------------------------------------------------------------------------------------------
BF_CASES = [
    # (B, Sq, Sk, Hq, Hkv, D, mask, window, bias_kind)
    (1, 5, 5, 2, 2, 3, 0, 0, 0),
    (1, 6, 6, 2, 1, 4, 1, 0, 0),
    (2, 7, 7, 4, 2, 3, 2, 3, 0),
    (1, 4, 9, 2, 1, 2, 1, 0, 1),      # Sq < Sk: bottom-right causal + T5
    (1, 9, 4, 2, 2, 2, 1, 0, 0),      # Sq > Sk: fully masked rows
    (1, 8, 8, 4, 1, 3, 2, 1, 2),      # window 1, MQA, full bias
    (1, 12, 12, 2, 2, 2, 0, 0, 1),    # bidirectional T5
    (2, 6, 10, 3, 1, 5, 2, 4, 2),
    (1, 16, 16, 1, 1, 8, 2, 16, 1),   # window == S
]


def check_brute_force():
    rng = np.random.default_rng(7)
    for (B, Sq, Sk, Hq, Hkv, D, mask, window, bk) in BF_CASES:
        q, k, v, bias = rand_case(rng, B, Sq, Sk, Hq, Hkv, D, bk)
        scale = 1.0 / math.sqrt(D)
        o1, l1 = run_oracle(q, k, v, scale, mask, window, bk, bias)
        o2, l2 = brute_force(q, k, v, scale, mask, window, bk, bias)
        assert np.max(np.abs(o1 - o2)) <= TOL, (B, Sq, Sk, Hq, Hkv, D, mask, window, bk)
        fin = np.isfinite(l2)
        assert np.array_equal(np.isfinite(l1), fin)
        assert np.max(np.abs(l1[fin] - l2[fin]), initial=0.0) <= TOL


def torch_band(Sq, Sk, mask, window):
    """Additive float mask (0 visible / -inf hidden) built with torch.tril/triu."""
    ones = torch.ones(Sq, Sk, dtype=torch.bool)
    off = Sk - Sq
    if mask == 0:
        vis = ones
    else:
        vis = torch.tril(ones, diagonal=off)
        if mask == 2:
            vis = vis & torch.triu(ones, diagonal=off - window + 1)
    return torch.zeros(Sq, Sk, dtype=torch.float64).masked_fill(~vis, float("-inf"))


def torch_ref(q, k, v, scale, mask, window, bias_kind, bias):
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    tq = torch.from_numpy(q).permute(0, 2, 1, 3).contiguous()
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1).contiguous()
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1).contiguous()
    am = torch_band(Sq, Sk, mask, window).expand(B, Hq, Sq, Sk).clone()
    if bias_kind == 1:
        rel = np.arange(Sk)[None, :] - (np.arange(Sq)[:, None] + Sk - Sq)
        idx = np.vectorize(t5_bucket_int)(rel)
        am = am + torch.from_numpy(bias[:, idx])[None]
    elif bias_kind == 2:
        am = am + torch.from_numpy(bias)
    o, l = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        tq, tk, tv, 0.0, False, attn_mask=am, scale=scale)
    return o.permute(0, 2, 1, 3).numpy(), l.numpy()


def check_torch_library():
    rng = np.random.default_rng(11)
    cases = [(2, 64, 64, 4, 4, 16, 0, 0, 0), (1, 96, 96, 8, 2, 32, 1, 0, 0),
             (1, 128, 128, 4, 1, 16, 2, 40, 0), (2, 80, 80, 3, 3, 8, 0, 0, 1),
             (1, 48, 48, 2, 2, 16, 0, 0, 2), (1, 200, 200, 2, 1, 8, 2, 200, 1)]
    for (B, Sq, Sk, Hq, Hkv, D, mask, window, bk) in cases:
        q, k, v, bias = rand_case(rng, B, Sq, Sk, Hq, Hkv, D, bk)
        scale = 1.0 / math.sqrt(D)
        o1, l1 = run_oracle(q, k, v, scale, mask, window, bk, bias)
        o2, l2 = torch_ref(q, k, v, scale, mask, window, bk, bias)
        assert np.max(np.abs(o1 - o2)) <= 1e-12
        assert np.max(np.abs(l1 - l2)) <= 1e-12


def _ev(x):
    if isinstance(x, (int, float)):
        return float(x)
    if "/" in x and "ln" not in x and "sqrt" not in x:
        return float(Fraction(x))
    return float(eval(x, {"__builtins__": {}}, {"ln": math.log, "sqrt": math.sqrt,
                                                 "inf": math.inf}))


def _arr(nested):
    return np.vectorize(_ev, otypes=[np.float64])(np.array(nested, dtype=object))


def check_golden():
    with open(GOLDEN) as f:
        data = json.load(f)
    for c in data["cases"]:
        q = _arr(c["q"])[None]
        k = _arr(c["k"])[None]
        v = _arr(c["v"])[None]
        bias = None
        if c["bias_kind"] == 1:
            bias = np.full((c["Hq"], 32), float(c["t5_fill"]))
            for idx, val in c["t5_entries"].items():
                bias[:, int(idx)] = _ev(val)
        elif c["bias_kind"] == 2:
            bias = _arr(c["bias"])[None]
        o, l = run_oracle(q, k, v, c["scale"], c["mask"], c["window"], c["bias_kind"], bias)
        eo = _arr(c["out"])
        el = _arr(c["lse"])
        assert np.max(np.abs(o[0] - eo)) <= 1e-12, c["name"]
        fin = np.isfinite(el)
        assert np.array_equal(np.isfinite(l[0]), fin), c["name"]
        assert np.max(np.abs(l[0][fin] - el[fin]), initial=0) <= 1e-12, c["name"]
    b = data["t5_bucket_boundaries"]["first_distance_of_bucket"]
    for bucket, n in b.items():
        bucket = int(bucket)
        # key before the query (rel < 0): lower half; key after it: upper half (+16)
        assert sdpa_ref.t5_bucket(-n) == bucket and sdpa_ref.t5_bucket(n) == bucket + 16
        assert sdpa_ref.t5_bucket(-(n - 1)) == bucket - 1


def check_t5_exhaustive():
    n = np.arange(-8191, 8192)
    got = oracle.t5_bucket(n)
    want = np.array([t5_bucket_int(int(x)) for x in n])
    assert np.array_equal(got, want)
    assert oracle.t5_bucket(0) == 0
    pos = oracle.t5_bucket(np.arange(0, 8192))
    neg = oracle.t5_bucket(-np.arange(0, 8192))
    assert np.all(np.diff(neg) >= 0) and np.all(np.diff(pos[1:]) >= 0)
    assert np.array_equal(neg[:8], np.arange(8))
    assert np.all(neg[91:] == 15) and neg[90] == 14
    assert np.array_equal(pos[1:], neg[1:] + 16)
    assert got.min() >= 0 and got.max() < 32


def check_invariants():
    rng = np.random.default_rng(3)
    B, S, Hq, Hkv, D = 2, 40, 4, 2, 16
    q, k, v, _ = rand_case(rng, B, S, S, Hq, Hkv, D, 0)
    sc = 1.0 / math.sqrt(D)
    # softmax rows sum to 1
    for mask, w in [(0, 0), (1, 0), (2, 7)]:
        P = oracle.attention_weights(q[0, :, 0], k[0, :, 0], np.arange(S), sc, mask, w)
        assert np.max(np.abs(P.sum(axis=1) - 1.0)) <= 1e-12
    # Q = 0: mean of the visible value rows, lse = ln(#visible)
    for mask, w in [(0, 0), (1, 0), (2, 5)]:
        o, l = run_oracle(np.zeros_like(q), k, v, sc, mask, w, 0, None)
        for i in range(S):
            lo = 0 if mask != 2 else max(0, i - w + 1)
            hi = S - 1 if mask == 0 else i
            want = v[:, lo:hi + 1].mean(axis=1)            # [B, Hkv, D]
            got = o[:, i]                                   # [B, Hq, D]
            assert np.max(np.abs(got - np.repeat(want, Hq // Hkv, axis=1))) <= 1e-12
            assert np.max(np.abs(l[:, :, i] - math.log(hi - lo + 1))) <= 1e-12
    # causal row 0 is exactly V[0]
    o, _ = run_oracle(q, k, v, sc, 1, 0, 0, None)
    assert np.array_equal(o[:, 0], np.repeat(v[:, 0], Hq // Hkv, axis=1))
    # window >= Sk equals causal (identical arithmetic: masks equal)
    for w in (S, S + 1, 10 * S):
        o2, l2 = run_oracle(q, k, v, sc, 2, w, 0, None)
        oc, lc = run_oracle(q, k, v, sc, 1, 0, 0, None)
        assert np.array_equal(o2, oc) and np.array_equal(l2, lc)
    # window 1: each query sees only itself
    o, l = run_oracle(q, k, v, sc, 2, 1, 0, None)
    assert np.max(np.abs(o - np.repeat(v, Hq // Hkv, axis=2))) <= 1e-12
    # causal last row = unmasked last row (codelab section 7)
    oc, _ = run_oracle(q, k, v, sc, 1, 0, 0, None)
    on, _ = run_oracle(q, k, v, sc, 0, 0, 0, None)
    assert np.max(np.abs(oc[:, -1] - on[:, -1])) <= 1e-12
    assert np.max(np.abs(oc[:, 0] - on[:, 0])) > 1e-3
    # V = 1 gives O = 1
    o, _ = run_oracle(q, k, np.ones_like(v), sc, 1, 0, 0, None)
    assert np.max(np.abs(o - 1.0)) <= 1e-12
    # adding c to every bias: O unchanged, lse + c
    bias = 0.5 * rng.standard_normal((B, Hq, S, S))
    o1, l1 = run_oracle(q, k, v, sc, 1, 0, 2, bias)
    o2, l2 = run_oracle(q, k, v, sc, 1, 0, 2, bias + 3.25)
    assert np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l2 - l1 - 3.25)) <= 1e-12
    tbl = rng.standard_normal((Hq, 32))
    o1, l1 = run_oracle(q, k, v, sc, 0, 0, 1, tbl)
    o2, l2 = run_oracle(q, k, v, sc, 0, 0, 1, tbl - 1.5)
    assert np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l2 - l1 + 1.5)) <= 1e-12
    # GQA = MHA on repeat_interleaved K/V
    G = Hq // Hkv
    og, lg = run_oracle(q, k, v, sc, 1, 0, 0, None)
    om, lm = run_oracle(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), sc, 1, 0, 0, None)
    assert np.array_equal(og, om) and np.array_equal(lg, lm)
    # bidirectional, no bias: invariant under a joint permutation of the key/value rows
    perm = rng.permutation(S)
    o1, l1 = run_oracle(q, k, v, sc, 0, 0, 0, None)
    o2, l2 = run_oracle(q, k[:, perm], v[:, perm], sc, 0, 0, 0, None)
    assert np.max(np.abs(o1 - o2)) <= 1e-12 and np.max(np.abs(l1 - l2)) <= 1e-12
    # scale = 0 behaves like Q = 0
    o1, _ = run_oracle(q, k, v, 0.0, 1, 0, 0, None)
    o2, _ = run_oracle(np.zeros_like(q), k, v, sc, 1, 0, 0, None)
    assert np.max(np.abs(o1 - o2)) <= 1e-12


def brute_force_weights(q_rows, k_head, q_pos, scale, mask, window, bias_rows):
    """Softmax weights P [n, Sk] by plain Python loops (same visibility rules as brute_force)."""
    n, D = q_rows.shape
    Sk = k_head.shape[0]
    P = np.zeros((n, Sk))
    for i in range(n):
        pos = int(q_pos[i])
        vis = []
        for j in range(Sk):
            if mask == 1 and j > pos:
                continue
            if mask == 2 and (j > pos or pos - j >= window):
                continue
            s = sum(float(q_rows[i, d]) * float(k_head[j, d]) for d in range(D)) * scale
            if bias_rows is not None:
                s += float(bias_rows[i, j])
            vis.append((j, s))
        if not vis:
            continue
        mx = max(s for _, s in vis)
        z = sum(math.exp(s - mx) for _, s in vis)
        for j, s in vis:
            P[i, j] = math.exp(s - mx) / z
    return P


WEIGHT_CASES = [
    # (Sq, Sk, D, mask, window, bias_kind, scale)
    (7, 7, 3, 0, 0, 0, 0.6),
    (9, 9, 4, 1, 0, 2, 0.5),
    (10, 10, 3, 2, 3, 1, 0.7),
    (5, 11, 2, 2, 4, 2, 1.3),         # Sq < Sk, bottom-right
    (9, 4, 2, 1, 0, 0, 0.5),          # Sq > Sk: rows without a key are all zero
    (12, 12, 2, 0, 0, 1, -0.4),       # negative scale, T5
]


def check_weights():
    """oracle.attention_weights (the P the gradient error bars use) against brute force, torch's
    CPU softmax over scores built here, and the identity-V link P = attend_rows(V = I)."""
    rng = np.random.default_rng(21)
    for (Sq, Sk, D, mask, window, bk, scale) in WEIGHT_CASES:
        q = rng.standard_normal((Sq, D))
        k = rng.standard_normal((Sk, D))
        pos = np.arange(Sq) + (Sk - Sq)
        bias = None
        if bk == 1:
            tbl = rng.standard_normal(32)
            bias = tbl[np.vectorize(t5_bucket_int)(np.arange(Sk)[None, :] - pos[:, None])]
        elif bk == 2:
            bias = 0.5 * rng.standard_normal((Sq, Sk))
        got = sdpa_ref.attention_weights(q, k, pos, scale, mask, window, bias)
        want = brute_force_weights(q, k, pos, scale, mask, window, bias)
        assert np.max(np.abs(got - want)) <= TOL, (Sq, Sk, mask, window, bk)
        # library special case: torch.softmax of the scores with an additive -inf band
        sc = torch.from_numpy(q) @ torch.from_numpy(k).T * scale + torch_band(Sq, Sk, mask, window)
        if bias is not None:
            sc = sc + torch.from_numpy(bias)
        tp = torch.softmax(sc, dim=-1).numpy()
        tp = np.where(np.isnan(tp), 0.0, tp)          # rows without a visible key
        assert np.max(np.abs(got - tp)) <= TOL
        # the weights are what attend_rows averages V with: V = I returns them exactly
        o, _ = oracle.attend_rows(q, k, np.eye(Sk), pos, scale, mask, window, bias)
        assert np.max(np.abs(got - o)) <= TOL


def check_sampled_rows_match_full():
    rng = np.random.default_rng(5)
    q, k, v, bias = rand_case(rng, 2, 70, 90, 4, 2, 8, 2)
    o, l = run_oracle(q, k, v, 0.3, 2, 25, 2, bias)
    rows = [0, 13, 69]
    for b in range(2):
        for h in range(4):
            ro, rl = oracle.sdpa_rows(q, k, v, b, h, rows, scale=0.3, mask_kind=2, window=25,
                                      bias_kind=2, bias=bias)
            assert np.array_equal(ro, o[b, rows, h]) and np.array_equal(rl, l[b, h, rows])


# ------------------------------------------------------------------------------------------
# tests
# ------------------------------------------------------------------------------------------
def test_oracle_brute_force():
    check_brute_force()


def test_oracle_torch_library_special_case():
    check_torch_library()


def test_oracle_golden_hand_cases():
    check_golden()


def test_oracle_t5_bucket_exhaustive():
    check_t5_exhaustive()


def test_oracle_invariants():
    check_invariants()


def test_oracle_attention_weights():
    check_weights()


def test_oracle_sampled_rows_match_full():
    check_sampled_rows_match_full()


def test_oracle_threads_same_result():
    rng = np.random.default_rng(9)
    q, k, v, _ = rand_case(rng, 2, 33, 33, 4, 2, 8, 0)
    o1, l1 = oracle.sdpa_forward(q, k, v, scale=0.25, mask_kind=1)
    o2, l2 = oracle.sdpa_forward(q, k, v, scale=0.25, mask_kind=1, threads=4)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# ------------------------------------------------------------------------------------------
ALL_CHECKS = [check_brute_force, check_torch_library, check_golden, check_t5_exhaustive,
              check_invariants, check_weights]


def _caught(monkeypatch, name, fn):
    monkeypatch.setattr(sdpa_ref, name, fn)
    for chk in ALL_CHECKS:
        try:
            chk()
        except AssertionError:
            return True
    return False


def test_pins_catch_dropped_scale(monkeypatch):
    orig = sdpa_ref.attend_rows

    def bad(q, k, v, pos, scale, *a, **kw):
        return orig(q, k, v, pos, 1.0, *a, **kw)
    assert _caught(monkeypatch, "attend_rows", bad)


def test_pins_catch_t5_sign_flip(monkeypatch):
    orig = sdpa_ref.t5_bucket
    assert _caught(monkeypatch, "t5_bucket", lambda rel: orig(-np.asarray(rel)))


def test_pins_catch_t5_log_base(monkeypatch):
    def bad(rel):
        rel = np.asarray(rel, dtype=np.int64)
        n = np.abs(rel)
        large = 8 + np.floor(np.log(np.maximum(n, 8) / 8) / math.log(128 / 8) * 7).astype(int)
        return np.where(n < 8, n, np.minimum(large, 15)) + np.where(rel > 0, 16, 0)
    assert _caught(monkeypatch, "t5_bucket", bad)


def test_pins_catch_window_off_by_one(monkeypatch):
    def bad(q_pos, Sk, mask_kind, window):
        j = np.arange(Sk)[None, :]
        p = np.asarray(q_pos)[:, None]
        if mask_kind == 0:
            return np.ones((p.shape[0], Sk), bool)
        if mask_kind == 1:
            return j <= p
        return (j <= p) & (p - j <= window)
    assert _caught(monkeypatch, "visible", bad)


def test_pins_catch_top_left_causal(monkeypatch):
    orig = sdpa_ref.sdpa_rows

    def bad(q, k, v, b, h, rows, **kw):
        # aligns query i with key i even when Sq != Sk
        Sq, Sk = q.shape[1], k.shape[1]
        if Sq == Sk:
            return orig(q, k, v, b, h, rows, **kw)
        kk = k[:, :Sq] if Sk > Sq else k
        vv = v[:, :Sq] if Sk > Sq else v
        return orig(q, kk, vv, b, h, rows, **kw)
    assert _caught(monkeypatch, "sdpa_rows", bad)


def test_pins_catch_wrong_gqa_grouping(monkeypatch):
    def bad(q, k, v, b, h, rows, *, scale, mask_kind, window=0, bias_kind=0, bias=None):
        Sq, Sk, Hkv = q.shape[1], k.shape[1], k.shape[2]
        kh = h % Hkv                         # interleaved instead of contiguous groups
        rows = np.asarray(rows, dtype=np.int64)
        pos = rows + Sk - Sq
        br = sdpa_ref._bias_rows(bias_kind, bias, b, h, pos, rows, Sk)
        return sdpa_ref.attend_rows(q[b, rows, h], k[b, :, kh], v[b, :, kh], pos, scale,
                                    mask_kind, window, br)
    assert _caught(monkeypatch, "sdpa_rows", bad)


def test_pins_catch_transposed_value(monkeypatch):
    orig = sdpa_ref.attend_rows

    def bad(q, k, v, *a, **kw):
        return orig(q, k, k, *a, **kw)        # uses K where V belongs
    assert _caught(monkeypatch, "attend_rows", bad)


def test_pins_catch_lse_log2(monkeypatch):
    orig = sdpa_ref.attend_rows

    def bad(*a, **kw):
        o, l = orig(*a, **kw)
        return o, l / math.log(2)
    assert _caught(monkeypatch, "attend_rows", bad)


# planted mistakes in the softmax weights (the P of the gradient error bars)
def test_pins_catch_weights_dropped_scale(monkeypatch):
    orig = sdpa_ref.attention_weights

    def bad(q, k, pos, scale, *a, **kw):
        return orig(q, k, pos, 1.0, *a, **kw)
    assert _caught(monkeypatch, "attention_weights", bad)


def test_pins_catch_weights_dropped_bias(monkeypatch):
    orig = sdpa_ref.attention_weights

    def bad(q, k, pos, scale, mask, window, bias_rows=None):
        return orig(q, k, pos, scale, mask, window, None)
    assert _caught(monkeypatch, "attention_weights", bad)


def test_pins_catch_weights_wrong_window(monkeypatch):
    orig = sdpa_ref.attention_weights

    def bad(q, k, pos, scale, mask, window, bias_rows=None):
        return orig(q, k, pos, scale, mask, window + 1, bias_rows)
    assert _caught(monkeypatch, "attention_weights", bad)


def test_pins_catch_weights_unnormalised(monkeypatch):
    orig = sdpa_ref.attention_weights

    def bad(*a, **kw):
        p = orig(*a, **kw)
        return p * 1.001
    assert _caught(monkeypatch, "attention_weights", bad)
