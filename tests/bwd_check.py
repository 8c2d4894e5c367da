"""Reference values and error bars for the attention gradients (dQ, dK, dV) of the HIP path.

The reference is the fp64 oracle (oracle.sdpa_backward) on the same bf16 inputs. The bars come
from one rounding model of a bf16 gradient computation, the same for every mask, bias, head
dim and kernel variant (nothing here depends on how the kernels split the work). With
u = 2^-8 (unit roundoff of bf16, round to nearest even) and f = 2^-24 (fp32):

  * Scores, exponentials, products and sums are fp32. P is recomputed from the forward's fp32
    LSE and may be rounded to bf16 before it forms dS (for dQ and for dK alike: the model
    takes the looser of the two choices), and dS is rounded to bf16 once as a matrix-core
    operand; each rounding has relative error <= u.
  * The forward's LSE is the log of a sum of bf16-rounded weights over fp32 scores, so its
    error is bounded a priori: u (the weights) + Sk f (the fp32 sum) + the P-weighted fp32
    score error + fp32 rounding of the log. That bound enters P as a relative error; the
    measured LSE of the forward must lie within it (checked here, not used to set the bar).
  * The row constant rowsum(dO * O) uses the bf16 forward output O~ the caller passes in
    (its own input): its error is sum_d |dO| |O~ - O| plus fp32 rounding.
  * First-order propagation of these through dS = P (dP - D), dQ = scale dS K,
    dK = scale dS^T Q, dV = P^T dO, with a worst-case fp32 accumulation term (terms * f),
    gives an element-wise bound: every element must lie within it (check 1).
  * The rounding errors of distinct terms are independent and of either sign, so the
    root-mean-square error of a whole gradient tensor stays well below u of its rms value:
    check 2 requires ||err||_2 <= u ||ref||_2.
The bf16-output entry point must return exactly the round-to-nearest-even of the fp32-output
entry point's values (same kernels, same fp32 results, one final rounding) -- check 3 lives
in the tests.
"""
from __future__ import annotations

import numpy as np

import oracle

U_BF16 = 2.0 ** -8
F32 = 2.0 ** -24
EXP2_REL = 2.0 ** -21
RMS_BAR = U_BF16


def _bias_rows(bias_kind, bias, b, h, q_pos, Sk):
    if bias_kind == oracle.BIAS_NONE:
        return None
    rel = np.arange(Sk, dtype=np.int64)[None, :] - q_pos[:, None]
    if bias_kind == oracle.BIAS_T5:
        return bias[h][oracle.t5_bucket(rel)]
    if bias_kind == oracle.BIAS_T5U:
        return bias[h][oracle.t5u_bucket(rel)]
    if bias_kind == oracle.BIAS_ALIBI:
        return -float(bias[h]) * np.abs(rel).astype(np.float64)
    return bias[b, h]


def pair_reference(q, k, v, dout, o_gpu, lse_gpu, b, kvh, *, scale, mask_kind, window,
                   bias_kind, bias):
    """Oracle gradients and element-wise bounds for one (batch b, KV head kvh).

    q, dout, o_gpu [B, Sq, Hq, D], k, v [B, Sk, Hkv, D], lse_gpu [B, Hq, Sq]: float64 arrays
    (o_gpu and lse_gpu are the GPU forward's outputs, the backward's inputs). Returns a dict
    with dq [Sq, G, D] (the G query heads of kvh), dk, dv [Sk, D], and bound_dq / bound_dk /
    bound_dv of the same shapes.
    """
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    dq_ref, dk_ref, dv_ref = oracle.sdpa_backward(
        q, k, v, dout, scale=scale, mask_kind=mask_kind, window=window, bias_kind=bias_kind,
        bias=bias, kv_heads=[(b, kvh)])
    q_pos = np.arange(Sq, dtype=np.int64) + (Sk - Sq)
    k_h, v_h = k[b, :, kvh], v[b, :, kvh]
    ak, av = np.abs(k_h), np.abs(v_h)
    sc = abs(scale)
    bq = np.zeros((Sq, G, D))
    bk = np.zeros((Sk, D))
    bv = np.zeros((Sk, D))
    n_kv_terms = G * Sq
    for g in range(G):
        h = kvh * G + g
        q_h, do_h = q[b, :, h], dout[b, :, h]
        brow = _bias_rows(bias_kind, bias, b, h, q_pos, Sk)
        o, lse = oracle.attend_rows(q_h, k_h, v_h, q_pos, scale, mask_kind, window, brow)
        p = oracle.attention_weights(q_h, k_h, q_pos, scale, mask_kind, window, brow)
        delta = np.sum(do_h * o, axis=1)
        dp = do_h @ v_h.T
        ds = p * (dp - delta[:, None])
        ado = np.abs(do_h)
        og = o_gpu[b, :, h]
        # row constant from the bf16 output, fp32 sum over D
        e_delta = (np.sum(ado * np.abs(og - o), axis=1)
                   + D * F32 * np.sum(np.abs(do_h * og), axis=1))
        # fp32 score error, and the a-priori bound on the forward's LSE error
        s_full = q_h @ k_h.T * scale + (0.0 if brow is None else brow)
        e_s = sc * D * F32 * (np.abs(q_h) @ ak.T) + 4 * F32 * np.abs(np.where(p > 0, s_full, 0))
        fin = np.isfinite(lse)
        lse0 = np.where(fin, lse, 0.0)
        e_lse = np.where(fin, U_BF16 * (1 + U_BF16) + Sk * F32 + np.sum(p * e_s, axis=1)
                         + 4 * F32 * np.abs(lse0), 0.0)
        lse_g = lse_gpu[b, h]
        assert np.array_equal(np.isfinite(lse_g), fin), "forward LSE: -inf rows differ"
        dlse = np.abs(np.where(fin, lse_g, 0.0) - lse0)
        assert np.all(dlse <= e_lse), (
            f"forward LSE error {dlse.max():.3g} beyond its a-priori bound {e_lse.min():.3g}")
        # relative error of the recomputed P (before any bf16 rounding)
        eps_p = e_s + e_lse[:, None] + 4 * F32 * np.abs(lse0)[:, None] + EXP2_REL
        eps_p = np.where(p > 0, eps_p, 0.0)
        e_dp = D * F32 * (ado @ av.T)
        # P rounded to bf16 before it forms dS: dS = rnd(rnd(P) (dP - D))
        e_p = (eps_p + U_BF16 * (1 + eps_p)) * p
        d_ds = e_p * np.abs(dp - delta[:, None]) + p * (e_dp + e_delta[:, None])
        e_ds = (1 + U_BF16) * d_ds + U_BF16 * np.abs(ds)
        e_ds_k = e_ds
        ads = np.abs(ds) + e_ds
        bq[:, g] = sc * (e_ds @ ak + Sk * F32 * (ads @ ak)) + F32 * np.abs(dq_ref[b, :, h])
        aq = np.abs(q_h)
        bk += sc * (e_ds_k.T @ aq + n_kv_terms * F32 * ((np.abs(ds) + e_ds_k).T @ aq))
        bv += e_p.T @ ado + n_kv_terms * F32 * ((p + e_p).T @ ado)
    bk += F32 * np.abs(dk_ref[b, :, kvh])
    bv += F32 * np.abs(dv_ref[b, :, kvh])
    return dict(dq=dq_ref[b, :, kvh * G:(kvh + 1) * G], dk=dk_ref[b, :, kvh],
                dv=dv_ref[b, :, kvh], bound_dq=bq, bound_dk=bk, bound_dv=bv)


def check_grad(name, got, ref, bound):
    """Checks 1 and 2 for one gradient tensor; returns (max err, max err / bound, rms ratio)."""
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite gradient"
    over = err > bound
    worst = float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
    assert not over.any(), (
        f"{name}: {int(over.sum())} elements outside the element-wise bound "
        f"(worst err/bound {worst:.3g}, first at {np.argwhere(over)[0].tolist()})")
    rn = float(np.sqrt(np.sum(ref * ref)))
    re = float(np.sqrt(np.sum(err * err)))
    ratio = re / rn if rn > 0 else 0.0
    # a gradient that is exactly zero (e.g. every row sees a single key, so dS = 0) has no
    # rms scale: the element-wise bound (fp32 rounding of dP and the row constant) decides
    if rn > 0:
        assert re <= RMS_BAR * rn, f"{name}: rms error {ratio:.3g} of rms value > 2^-8"
    return float(err.max()) if err.size else 0.0, worst, ratio
