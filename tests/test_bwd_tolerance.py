"""CPU checks of the gradient error bars in bwd_check.py (no GPU).

An fp32 / bf16 emulation of a bf16 gradient computation (scores and sums in fp32, P and dS
rounded to bf16 before their products, the dS of each gradient formed from either the fp32 or
the bf16-rounded P, the row constant from a bf16 forward output, P from an fp32 LSE, which is
either the exact one rounded or the log of a sum of bf16 weights) must pass both bars against
the fp64 oracle in every combination; the same emulation with a planted mistake must fail at
least one of them. This pins the bars from both sides: not tighter than the arithmetic
allows, not so loose that a wrong gradient passes.
"""
import numpy as np
import pytest

import oracle
import sdpa_inputs as si
from bwd_check import check_grad, pair_reference

LOG2E = np.float32(1.4426950408889634)


def bf16(x):
    return si.bf16_bits_to_f32(si.f32_to_bf16_bits(np.asarray(x, np.float32)))


def emulate(q, k, v, dout, o16, lse32, b, kvh, scale, mask, window, bias_kind, bias, plant=None,
            p_bf16=(False, True)):
    """fp32 emulation of a bf16 gradient computation for one (b, KV head): returns
    dq [Sq, G, D], dk, dv. p_bf16 = (for dQ, for dK): whether that gradient's dS is formed
    from the bf16-rounded P instead of the fp32 P."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    q_pos = np.arange(Sq) + (Sk - Sq)
    vis = oracle.visible(q_pos, Sk, mask, window + (1 if plant == "window_off_by_one" else 0))
    k_h = k[b, :, kvh].astype(np.float32)
    v_h = v[b, :, kvh].astype(np.float32)
    dq = np.zeros((Sq, G, D), np.float32)
    dk = np.zeros((Sk, D), np.float32)
    dv = np.zeros((Sk, D), np.float32)
    sl2 = np.float32(scale) * LOG2E
    for g in range(G):
        h = kvh * G + g
        q_h = q[b, :, h].astype(np.float32)
        do_h = dout[b, :, h].astype(np.float32)
        x = (q_h @ k_h.T) * sl2
        if bias_kind == oracle.BIAS_T5:
            rel = np.arange(Sk)[None, :] - q_pos[:, None]
            x = x + bias[h][oracle.t5_bucket(rel)].astype(np.float32) * LOG2E
        elif bias_kind == oracle.BIAS_FULL:
            x = x + bias[b, h].astype(np.float32) * LOG2E
        x = np.where(vis, x, -np.inf).astype(np.float32)
        l2 = lse32[b, h] * LOG2E
        l2 = np.where(np.isfinite(l2), l2, np.inf).astype(np.float32)
        with np.errstate(invalid="ignore"):
            p = np.exp2(x - l2[:, None]).astype(np.float32)
        p = np.where(np.isnan(p), 0, p).astype(np.float32)
        delta = np.sum(do_h * o16[b, :, h].astype(np.float32), axis=1, dtype=np.float32)
        if plant == "no_row_constant":
            delta = np.zeros_like(delta)
        dp = do_h @ v_h.T
        ds = p * (dp - delta[:, None])
        pb, dsb = bf16(p), bf16(ds)
        dsb_p = bf16(pb * (dp - delta[:, None]))
        dsb_k = dsb_p if p_bf16[1] else dsb
        dsb = dsb_p if p_bf16[0] else dsb
        kk = np.roll(k_h, 1, axis=0) if plant == "dq_key_shift" else k_h
        dq[:, g] = np.float32(scale) * (dsb @ kk)
        dk += (np.float32(1.0) if plant == "dk_no_scale" else np.float32(scale)) * (dsb_k.T @ q_h)
        dv += pb.T @ (do_h if plant != "dv_uses_q" else q_h)
    return dq, dk, dv


CASES = [  # B, Sq, Sk, Hq, Hkv, D, mask, window, bias_kind
    (1, 150, 150, 4, 2, 64, oracle.MASK_CAUSAL, 0, oracle.BIAS_NONE),
    (1, 130, 190, 2, 1, 128, oracle.MASK_SLIDING, 40, oracle.BIAS_NONE),
    (1, 120, 120, 2, 2, 64, oracle.MASK_NONE, 0, oracle.BIAS_T5),
    (1, 96, 96, 2, 2, 64, oracle.MASK_NONE, 0, oracle.BIAS_FULL),
]


def _lse_bf16_sum(q, k, extra, wl):
    """An fp32 LSE formed like a bf16 forward's: the log of an fp32 sum of bf16-rounded
    weights over fp32 scores."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    q_pos = np.arange(Sq) + (Sk - Sq)
    vis = oracle.visible(q_pos, Sk, wl.mask_kind, wl.window)
    out = np.zeros((B, Hq, Sq), np.float32)
    for b in range(B):
        for h in range(Hq):
            s = (q[b, :, h].astype(np.float32) @ k[b, :, h // G].astype(np.float32).T
                 ) * np.float32(wl.scale)
            if wl.bias_kind == oracle.BIAS_T5:
                rel = np.arange(Sk)[None, :] - q_pos[:, None]
                s = s + extra[h][oracle.t5_bucket(rel)].astype(np.float32)
            elif wl.bias_kind == oracle.BIAS_FULL:
                s = s + extra[b, h].astype(np.float32)
            s = np.where(vis, s, -np.inf).astype(np.float32)
            m = s.max(axis=1)
            w = bf16(np.exp(s - m[:, None]).astype(np.float32))
            out[b, h] = m + np.log(np.sum(w, axis=1, dtype=np.float32))
    return out


def _case(c, seed, lse_bf16=False):
    B, Sq, Sk, Hq, Hkv, D, mask, window, bk = c
    wl = si.Workload("tol", B, Hq, Hkv, Sq, Sk, D, "bf16", mask, window=window, bias_kind=bk,
                     seed=seed)
    inp = si.make_inputs(wl)
    q, k, v, extra = inp.as_f64()
    do = si.bf16_bits_to_f64(si.make_dout(wl))
    o, lse = oracle.sdpa_forward(q, k, v, scale=wl.scale, mask_kind=mask, window=window,
                                 bias_kind=bk, bias=extra)
    o16 = bf16(o.astype(np.float32)).astype(np.float64)           # the forward's bf16 output
    lse32 = lse.astype(np.float32)                                  # and its fp32 LSE
    if lse_bf16:
        lse32 = _lse_bf16_sum(q, k, extra, wl)
    return wl, q, k, v, extra, do, o16, lse32


def _verdict(c, seed, plant, p_bf16=(False, True), lse_bf16=False):
    wl, q, k, v, extra, do, o16, lse32 = _case(c, seed, lse_bf16)
    G = wl.Hq // wl.Hkv
    for kvh in range(wl.Hkv):
        ref = pair_reference(q, k, v, do, o16, lse32.astype(np.float64), 0, kvh, scale=wl.scale,
                             mask_kind=wl.mask_kind, window=wl.window, bias_kind=wl.bias_kind,
                             bias=extra)
        got = emulate(q, k, v, do, o16, lse32, 0, kvh, wl.scale, wl.mask_kind, wl.window,
                      wl.bias_kind, extra, plant, p_bf16)
        assert got[0].shape == (wl.Sq, G, wl.D)
        for name, g, r, bd in (("dq", got[0], ref["dq"], ref["bound_dq"]),
                               ("dk", got[1], ref["dk"], ref["bound_dk"]),
                               ("dv", got[2], ref["dv"], ref["bound_dv"])):
            check_grad(name, g.astype(np.float64), r, bd)


@pytest.mark.parametrize("p_bf16", [(False, False), (False, True), (True, True)],
                         ids=["p32", "dk_pbf16", "both_pbf16"])
@pytest.mark.parametrize("c", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_emulated_kernel_rounding_passes(c, p_bf16):
    _verdict(c, 77, None, p_bf16)


@pytest.mark.parametrize("c", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_emulated_bf16_sum_lse_passes(c):
    _verdict(c, 79, None, (True, True), lse_bf16=True)


@pytest.mark.parametrize("plant", ["no_row_constant", "dq_key_shift", "dk_no_scale", "dv_uses_q",
                                   "window_off_by_one"])
def test_planted_mistakes_fail(plant):
    c = CASES[1] if plant == "window_off_by_one" else CASES[0]
    with pytest.raises(AssertionError):
        _verdict(c, 78, plant)
