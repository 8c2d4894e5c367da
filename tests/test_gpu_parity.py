"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same values.

Small cases are compared element by element over the whole output; they span several query
and key tiles and end in ragged tails. The full-size workloads run in exactly the launch
configuration the benchmark times and are checked on sampled rows the oracle computes one by
one.

Bars: bf16 inputs -> max-abs <= 1e-2 and mean-abs <= 1e-3, judged on the fp32 epilogue of the
same kernel (sdpa_fwd_bf16_f32out), whose bf16 rounding must equal sdpa_fwd's output bit for
bit; sdpa_fwd itself is also checked against the oracle with allclose(rtol=1e-2, atol=1e-2)
(the codelab's bf16 comparison, section 6). fp32 inputs -> max-abs <= 1e-5.
"""
import numpy as np
import pytest

import oracle
import sdpa_inputs as si
from helpers import (BF16_MAX_ABS, BF16_MEAN_ABS, F32_MAX_ABS, errors, oracle_full,
                     out_to_f64, run_gpu, sample_rows, to_device)

pytestmark = pytest.mark.gpu

W = si.WORKLOADS

SMALL_BF16 = [
    si.small(W["c2"], B=1, Hq=8, Hkv=2, Sq=700, Sk=700, window=700, name_suffix="s700_w_eq_s"),
    si.small(W["c2"], B=1, Hq=8, Hkv=2, Sq=700, Sk=700, window=190, name_suffix="s700_w190"),
    si.small(W["c3"], B=1, Hq=4, Hkv=1, Sq=1000, Sk=1000, window=256, name_suffix="s1000_w256"),
    si.small(W["c3c"], B=1, Hq=4, Hkv=1, Sq=1000, Sk=1000, name_suffix="s1000"),
    si.small(W["c4t5"], B=2, Hq=3, Hkv=3, Sq=333, Sk=333, name_suffix="s333"),
    si.small(W["c4full"], B=2, Hq=3, Hkv=3, Sq=333, Sk=333, name_suffix="s333"),
    si.small(W["c4full"], B=1, Hq=2, Hkv=2, Sq=256, Sk=264, name_suffix="s256_264"),
    si.small(W["c5mha"], B=2, Hq=8, Hkv=8, Sq=513, Sk=513, name_suffix="s513"),
    si.small(W["c5gqa"], B=2, Hq=8, Hkv=2, Sq=513, Sk=513, name_suffix="s513"),
    si.small(W["c5mqa"], B=2, Hq=8, Hkv=1, Sq=513, Sk=513, name_suffix="s513"),
    # bottom-right causal with Sq < Sk, and Sq > Sk (first rows see no key)
    si.small(W["c5gqa"], B=1, Hq=4, Hkv=2, Sq=100, Sk=300, name_suffix="q100_k300"),
    si.small(W["c5gqa"], B=1, Hq=4, Hkv=2, Sq=300, Sk=100, name_suffix="q300_k100"),
    si.small(W["c2"], B=1, Hq=4, Hkv=2, Sq=77, Sk=333, window=64, name_suffix="q77_k333_w64"),
    # D = 64 with masks, D = 128 with biases
    si.small(W["c4t5"], B=1, Hq=4, Hkv=2, Sq=300, Sk=300, name_suffix="causal_t5").replace(
        mask_kind=si.MASK_CAUSAL),
    si.small(W["c4full"], B=1, Hq=2, Hkv=1, Sq=200, Sk=200, name_suffix="sliding_full").replace(
        mask_kind=si.MASK_SLIDING, window=50),
    si.small(W["c2"], B=1, Hq=4, Hkv=4, Sq=256, Sk=256, name_suffix="t5_d128").replace(
        bias_kind=si.BIAS_T5, mask_kind=si.MASK_NONE),
    si.small(W["c2"], B=1, Hq=2, Hkv=2, Sq=1, Sk=1, name_suffix="single"),
    si.small(W["c2"], B=1, Hq=2, Hkv=1, Sq=5, Sk=3, window=1, name_suffix="window1"),
    # bidirectional D = 128 without bias; T5 and sliding with Sq != Sk
    si.small(W["c2"], B=2, Hq=4, Hkv=2, Sq=300, Sk=300, name_suffix="none_d128").replace(
        mask_kind=si.MASK_NONE),
    si.small(W["c4t5"], B=1, Hq=3, Hkv=3, Sq=150, Sk=400, name_suffix="t5_q150_k400"),
    si.small(W["c2"], B=1, Hq=4, Hkv=1, Sq=200, Sk=520, window=150, name_suffix="q200_k520_w150"),
    # negative and zero softmax scale (sign flip of the Q fragment; smallest normal float)
    si.small(W["c2"], B=1, Hq=4, Hkv=2, Sq=260, Sk=260, window=100,
             name_suffix="neg_scale").replace(scale_override=-0.07),
    si.small(W["c3c"], B=1, Hq=2, Hkv=1, Sq=200, Sk=200, name_suffix="neg_scale").replace(
        scale_override=-0.2),
    si.small(W["c4t5"], B=1, Hq=2, Hkv=2, Sq=140, Sk=140, name_suffix="neg_scale").replace(
        scale_override=-0.1),
    si.small(W["c4full"], B=1, Hq=2, Hkv=2, Sq=136, Sk=136, name_suffix="neg_scale").replace(
        scale_override=-0.1),
    # full bias at D = 64 (its own 4-slot ring): 1, 2, 3 and 5 key tiles (the ring's start and
    # wrap), a ragged last query tile, a band that starts past key tile 0, Sq < Sk causal
    si.small(W["c4full"], B=1, Hq=2, Hkv=2, Sq=300, Sk=64, name_suffix="q300_k64"),
    si.small(W["c4full"], B=1, Hq=2, Hkv=2, Sq=300, Sk=128, name_suffix="q300_k128"),
    si.small(W["c4full"], B=1, Hq=2, Hkv=2, Sq=300, Sk=192, name_suffix="q300_k192"),
    si.small(W["c4full"], B=2, Hq=2, Hkv=1, Sq=520, Sk=320, name_suffix="q520_k320"),
    si.small(W["c4full"], B=1, Hq=2, Hkv=2, Sq=600, Sk=600, name_suffix="sliding_w200").replace(
        mask_kind=si.MASK_SLIDING, window=200),
    si.small(W["c4full"], B=1, Hq=2, Hkv=2, Sq=256, Sk=512, name_suffix="causal_q256_k512").replace(
        mask_kind=si.MASK_CAUSAL),
    si.small(W["c3c"], B=1, Hq=2, Hkv=1, Sq=200, Sk=200, name_suffix="zero_scale").replace(
        scale_override=0.0),
    si.small(W["c4t5"], B=1, Hq=2, Hkv=2, Sq=140, Sk=140, name_suffix="zero_scale").replace(
        scale_override=0.0),
    # ALiBi and T5 decoder buckets (bidirectional, causal, sliding; GQA; Sq != Sk)
    si.small(W["c2alibi"], B=1, Hq=8, Hkv=2, Sq=600, Sk=600, name_suffix="s600"),
    si.small(W["c2alibi"], B=2, Hq=4, Hkv=4, Sq=300, Sk=300, name_suffix="none").replace(
        mask_kind=si.MASK_NONE),
    si.small(W["c2alibi"], B=1, Hq=4, Hkv=1, Sq=200, Sk=500, name_suffix="sliding_q200_k500"
             ).replace(mask_kind=si.MASK_SLIDING, window=150),
    si.small(W["c2alibi"], B=1, Hq=4, Hkv=2, Sq=256, Sk=256, name_suffix="d64_neg").replace(
        D=64, scale_override=-0.1),
    # the masked ALiBi path keeps the per-row part of the bias out of the scores: zero scale
    # (floored score scale), rows that see no key, D = 64 sliding with a key prefix
    si.small(W["c2alibi"], B=1, Hq=4, Hkv=2, Sq=260, Sk=260, name_suffix="zero_scale").replace(
        scale_override=0.0),
    si.small(W["c2alibi"], B=1, Hq=4, Hkv=2, Sq=300, Sk=100, name_suffix="q300_k100"),
    si.small(W["c2alibi"], B=1, Hq=8, Hkv=1, Sq=230, Sk=610, name_suffix="d64_sliding_q230_k610"
             ).replace(D=64, mask_kind=si.MASK_SLIDING, window=97),
    si.small(W["c4t5u"], B=2, Hq=3, Hkv=3, Sq=333, Sk=333, name_suffix="s333"),
    si.small(W["c4t5u"], B=1, Hq=4, Hkv=2, Sq=300, Sk=300, name_suffix="none").replace(
        mask_kind=si.MASK_NONE),
    si.small(W["c4t5u"], B=1, Hq=4, Hkv=2, Sq=150, Sk=400, name_suffix="d128_q150_k400"
             ).replace(D=128),
    # head dims 32 and 256: every mask and bias kind, GQA / MQA, ragged tails, Sq != Sk
    si.small(W["c2d32"], B=2, Hq=8, Hkv=2, Sq=333, Sk=333, name_suffix="s333"),
    si.small(W["c2d32"], B=1, Hq=4, Hkv=1, Sq=300, Sk=520, name_suffix="sliding_q300_k520"
             ).replace(mask_kind=si.MASK_SLIDING, window=150),
    si.small(W["c2d32"], B=1, Hq=3, Hkv=3, Sq=270, Sk=270, name_suffix="t5_none").replace(
        mask_kind=si.MASK_NONE, bias_kind=si.BIAS_T5),
    si.small(W["c2d32"], B=1, Hq=2, Hkv=2, Sq=200, Sk=264, name_suffix="full_none").replace(
        mask_kind=si.MASK_NONE, bias_kind=si.BIAS_FULL),
    si.small(W["c2d32"], B=1, Hq=4, Hkv=2, Sq=300, Sk=100, name_suffix="alibi_q300_k100"
             ).replace(bias_kind=si.BIAS_ALIBI),
    si.small(W["c2d32"], B=1, Hq=4, Hkv=4, Sq=260, Sk=260, name_suffix="t5u_neg").replace(
        bias_kind=si.BIAS_T5U, scale_override=-0.15),
    si.small(W["c2d256"], B=2, Hq=8, Hkv=2, Sq=333, Sk=333, name_suffix="s333"),
    si.small(W["c2d256"], B=1, Hq=4, Hkv=1, Sq=300, Sk=520, name_suffix="sliding_q300_k520"
             ).replace(mask_kind=si.MASK_SLIDING, window=150),
    si.small(W["c2d256"], B=1, Hq=3, Hkv=3, Sq=270, Sk=270, name_suffix="t5_none").replace(
        mask_kind=si.MASK_NONE, bias_kind=si.BIAS_T5),
    si.small(W["c2d256"], B=1, Hq=2, Hkv=2, Sq=200, Sk=264, name_suffix="full_none").replace(
        mask_kind=si.MASK_NONE, bias_kind=si.BIAS_FULL),
    si.small(W["c2d256"], B=1, Hq=2, Hkv=1, Sq=130, Sk=197, name_suffix="full_causal_odd_sk"
             ).replace(bias_kind=si.BIAS_FULL),
    si.small(W["c2d256"], B=1, Hq=4, Hkv=2, Sq=300, Sk=100, name_suffix="alibi_q300_k100"
             ).replace(bias_kind=si.BIAS_ALIBI),
    si.small(W["c2d256"], B=1, Hq=4, Hkv=4, Sq=260, Sk=260, name_suffix="t5u_neg").replace(
        bias_kind=si.BIAS_T5U, scale_override=-0.15),
    si.small(W["c2d256"], B=1, Hq=2, Hkv=1, Sq=150, Sk=150, name_suffix="zero_scale").replace(
        scale_override=0.0),
]

SMALL_F32 = [
    W["c1"],
    W["c1"].replace(name="c1_sliding_gqa_d128", Hq=4, Hkv=2, Sq=200, Sk=200, D=128,
                    mask_kind=si.MASK_SLIDING, window=77),
    W["c1"].replace(name="c1_t5_none", Hq=3, Hkv=3, Sq=150, Sk=150, mask_kind=si.MASK_NONE,
                    bias_kind=si.BIAS_T5),
    W["c1"].replace(name="c1_full_causal_q_lt_k", B=2, Hq=2, Hkv=1, Sq=90, Sk=170,
                    bias_kind=si.BIAS_FULL),
    W["c1"].replace(name="c1_q_gt_k", Sq=170, Sk=90),
    W["c1"].replace(name="c1_neg_scale_none", mask_kind=si.MASK_NONE, scale_override=-0.1),
    W["c1"].replace(name="c1_zero_scale", scale_override=0.0),
    W["c1"].replace(name="c1_alibi_gqa", Hq=4, Hkv=2, bias_kind=si.BIAS_ALIBI),
    W["c1"].replace(name="c1_t5u_none", mask_kind=si.MASK_NONE, bias_kind=si.BIAS_T5U, Sk=170),
    W["c1"].replace(name="c1_d32_sliding_gqa", Hq=4, Hkv=2, Sq=150, Sk=150, D=32,
                    mask_kind=si.MASK_SLIDING, window=40),
    W["c1"].replace(name="c1_d32_t5", D=32, bias_kind=si.BIAS_T5),
    W["c1"].replace(name="c1_d256_causal", D=256, Sq=150, Sk=150),
    W["c1"].replace(name="c1_d256_full_none", D=256, mask_kind=si.MASK_NONE,
                    bias_kind=si.BIAS_FULL, Sq=90, Sk=130),
    # several row blocks and key tiles with ragged ends; in the key tiles at the window's edges
    # some waves of a workgroup see no key of their share
    W["c1"].replace(name="c1_mqa_sliding_t5_ragged", B=2, Hq=4, Hkv=1, Sq=300, Sk=333,
                    mask_kind=si.MASK_SLIDING, window=100, bias_kind=si.BIAS_T5),
    W["c1"].replace(name="c1_d128_full_gqa_none", Hq=4, Hkv=2, Sq=130, Sk=97, D=128,
                    mask_kind=si.MASK_NONE, bias_kind=si.BIAS_FULL),
    W["c1"].replace(name="c1_d256_t5u_sliding", Sq=100, Sk=140, D=256,
                    mask_kind=si.MASK_SLIDING, window=50, bias_kind=si.BIAS_T5U),
    W["c1"].replace(name="c1_d32_alibi_causal_long", Sq=257, Sk=513, D=32,
                    bias_kind=si.BIAS_ALIBI),
]


def _check_bf16(sdpa, wl, inp, dev, ref_o, ref_l, rows=None, heads=None):
    import torch
    o32, l32 = run_gpu(sdpa, wl, dev, out_f32=True)
    o16, l16 = run_gpu(sdpa, wl, dev, out_f32=False)
    # the bf16 path is exactly the rounding of the fp32 epilogue, and shares its LSE
    assert torch.equal(o16, o32.to(torch.bfloat16)), "bf16 out != RNE(fp32 out)"
    assert torch.equal(l16, l32), "lse differs between epilogues"
    go, gl, g16 = out_to_f64(o32), out_to_f64(l32), out_to_f64(o16)
    if rows is not None:
        go = np.stack([go[b, rows, h] for b, h in heads])
        g16 = np.stack([g16[b, rows, h] for b, h in heads])
        gl = np.stack([gl[b, h, rows] for b, h in heads])
    mo, ao = errors(go, ref_o)
    ml, al = errors(gl, ref_l)
    print(f"{wl.name}: O max {mo:.3e} mean {ao:.3e} | LSE max {ml:.3e} mean {al:.3e}")
    assert mo <= BF16_MAX_ABS and ao <= BF16_MEAN_ABS, (mo, ao)
    assert ml <= BF16_MAX_ABS and al <= BF16_MEAN_ABS, (ml, al)
    fin = np.isfinite(ref_o)
    assert np.allclose(g16[fin], ref_o[fin], rtol=1e-2, atol=1e-2)


@pytest.mark.parametrize("wl", SMALL_BF16, ids=[w.name for w in SMALL_BF16])
def test_parity_bf16_small(gpu_lib, wl):
    inp = si.make_inputs(wl)
    ref_o, ref_l = oracle_full(inp)
    _check_bf16(gpu_lib, wl, inp, to_device(inp), ref_o, ref_l)


@pytest.mark.parametrize("wl", SMALL_F32, ids=[w.name for w in SMALL_F32])
def test_parity_f32(gpu_lib, wl):
    inp = si.make_inputs(wl)
    ref_o, ref_l = oracle_full(inp)
    o, l = run_gpu(gpu_lib, wl, to_device(inp))
    mo, ao = errors(out_to_f64(o), ref_o)
    ml, al = errors(out_to_f64(l), ref_l)
    print(f"{wl.name}: O max {mo:.3e} | LSE max {ml:.3e}")
    assert mo <= F32_MAX_ABS and ml <= F32_MAX_ABS


FULL = ["c2", "c3", "c3c", "c4t5", "c4full", "c5mha", "c5gqa", "c5mqa", "c2alibi", "c4t5u", "c2d32",
        "c2d256"]


@pytest.mark.parametrize("key", FULL)
def test_parity_full_size_sampled(gpu_lib, key):
    """Full-size workload, launched exactly as the benchmark does; oracle on sampled rows."""
    import torch
    wl = W[key]
    inp = si.make_inputs(wl)
    dev = to_device(inp)
    q, k, v, extra = inp.as_f64()
    rng = np.random.default_rng(sum(map(ord, key)))
    heads = [(0, 0), (wl.B - 1, wl.Hq - 1)] + \
        [(int(rng.integers(wl.B)), int(rng.integers(wl.Hq))) for _ in range(4)]
    rows = sample_rows(wl.Sq, 24, seed=len(key))
    ref_o, ref_l = [], []
    for b, h in heads:
        o, l = oracle.sdpa_rows(q, k, v, b, h, rows, scale=float(np.float32(wl.scale)),
                                mask_kind=wl.mask_kind, window=wl.window,
                                bias_kind=wl.bias_kind, bias=extra)
        ref_o.append(o)
        ref_l.append(l)
    _check_bf16(gpu_lib, wl, inp, dev, np.stack(ref_o), np.stack(ref_l), rows=rows, heads=heads)
    del dev
    torch.cuda.empty_cache()
