"""GPU parity of the split-key decode (sdpa_decode / sdpa_decode_f32out, through the C ABI)
against the fp64 oracle: the same forward definition, few query rows against a long cache.

Bars as for the forward: max-abs <= 1e-2 and mean-abs <= 1e-3 on the fp32 output and the LSE,
and the bf16 output equal to the round-to-nearest-even of the fp32 output bit for bit. Small
cases cover one split and many, every mask and bias kind, GQA / MQA / MHA row blocks (one and
several 32-row blocks), ragged caches, negative and zero scales; the full-size decode workloads
are checked on sampled heads. Determinism: 100 repeated calls are bitwise identical.
"""
import numpy as np
import pytest

import oracle
import sdpa_inputs as si
from helpers import BF16_MAX_ABS, BF16_MEAN_ABS, errors, oracle_full, out_to_f64, to_device

pytestmark = pytest.mark.gpu

W = si.WORKLOADS
BASE = W["dec"]

SMALL = [
    BASE.replace(name="dec_b2_g4_q1_k5000", B=2, Hq=8, Hkv=2, Sk=5000),
    BASE.replace(name="dec_b1_g4_q1_k300_single_split", B=1, Hq=8, Hkv=2, Sk=300),
    BASE.replace(name="dec_mqa_g32_q1_k3000", B=1, Hq=32, Hkv=1, Sk=3000),
    BASE.replace(name="dec_mha_q1_k2500", B=2, Hq=4, Hkv=4, Sk=2500),
    BASE.replace(name="dec_g8_q4_k4100", B=1, Hq=16, Hkv=2, Sq=4, Sk=4100),
    BASE.replace(name="dec_g8_q9_k3000_two_blocks", B=1, Hq=8, Hkv=1, Sq=9, Sk=3000),
    BASE.replace(name="dec_g4_q3_k1_tiny", B=1, Hq=4, Hkv=1, Sq=3, Sk=1),
    BASE.replace(name="dec_q6_k4_rows_without_keys", B=1, Hq=4, Hkv=2, Sq=6, Sk=4),
    BASE.replace(name="dec_none_k2000", B=1, Hq=8, Hkv=2, Sq=2, Sk=2000,
                 mask_kind=si.MASK_NONE),
    BASE.replace(name="dec_sliding_w300_q4_k5000", B=1, Hq=8, Hkv=2, Sq=4, Sk=5000,
                 mask_kind=si.MASK_SLIDING, window=300),
    BASE.replace(name="dec_sliding_w1_q3_k700", B=1, Hq=4, Hkv=2, Sq=3, Sk=700,
                 mask_kind=si.MASK_SLIDING, window=1),
    BASE.replace(name="dec_t5_d64_q2_k3000", B=2, Hq=6, Hkv=3, Sq=2, Sk=3000, D=64,
                 mask_kind=si.MASK_NONE, bias_kind=si.BIAS_T5),
    BASE.replace(name="dec_t5_causal_q5_k1000", B=1, Hq=4, Hkv=2, Sq=5, Sk=1000,
                 bias_kind=si.BIAS_T5),
    BASE.replace(name="dec_full_bias_q3_k2001", B=1, Hq=4, Hkv=2, Sq=3, Sk=2001,
                 bias_kind=si.BIAS_FULL),
    BASE.replace(name="dec_full_bias_d64_none_q1_k4096", B=2, Hq=4, Hkv=4, Sq=1, Sk=4096, D=64,
                 mask_kind=si.MASK_NONE, bias_kind=si.BIAS_FULL),
    BASE.replace(name="dec_neg_scale_q2_k3000", B=1, Hq=8, Hkv=2, Sq=2, Sk=3000,
                 scale_override=-0.08),
    BASE.replace(name="dec_zero_scale_t5_q2_k900", B=1, Hq=4, Hkv=2, Sq=2, Sk=900,
                 bias_kind=si.BIAS_T5, scale_override=0.0),
    BASE.replace(name="dec_alibi_q1_k5000", B=2, Hq=8, Hkv=2, Sk=5000, bias_kind=si.BIAS_ALIBI),
    BASE.replace(name="dec_alibi_none_q3_k2000", B=1, Hq=8, Hkv=2, Sq=3, Sk=2000,
                 mask_kind=si.MASK_NONE, bias_kind=si.BIAS_ALIBI),
    BASE.replace(name="dec_t5u_d64_q2_k3000", B=1, Hq=6, Hkv=2, Sq=2, Sk=3000, D=64,
                 bias_kind=si.BIAS_T5U),
    # D = 256 (two-slot ring): one and several splits, several row blocks, masks and biases
    BASE.replace(name="dec_d256_b2_g4_q1_k5000", B=2, Hq=8, Hkv=2, Sk=5000, D=256),
    BASE.replace(name="dec_d256_q9_k3000_two_blocks", B=1, Hq=8, Hkv=1, Sq=9, Sk=3000, D=256),
    BASE.replace(name="dec_d256_single_split_k200", B=1, Hq=4, Hkv=2, Sq=2, Sk=200, D=256),
    BASE.replace(name="dec_d256_sliding_t5_q4_k4100", B=1, Hq=8, Hkv=2, Sq=4, Sk=4100, D=256,
                 mask_kind=si.MASK_SLIDING, window=300, bias_kind=si.BIAS_T5),
    BASE.replace(name="dec_d256_full_bias_none_q3_k2001", B=1, Hq=4, Hkv=2, Sq=3, Sk=2001,
                 D=256, mask_kind=si.MASK_NONE, bias_kind=si.BIAS_FULL),
    BASE.replace(name="dec_d256_alibi_neg_q2_k3000", B=1, Hq=8, Hkv=2, Sq=2, Sk=3000, D=256,
                 bias_kind=si.BIAS_ALIBI, scale_override=-0.05),
    # D = 32 (one head-dim fragment)
    BASE.replace(name="dec_d32_b2_g4_q1_k5000", B=2, Hq=8, Hkv=2, Sk=5000, D=32),
    BASE.replace(name="dec_d32_q9_k3000_two_blocks", B=1, Hq=8, Hkv=1, Sq=9, Sk=3000, D=32),
    BASE.replace(name="dec_d32_single_split_k200", B=1, Hq=4, Hkv=2, Sq=2, Sk=200, D=32),
    BASE.replace(name="dec_d32_sliding_t5u_q4_k4100", B=1, Hq=8, Hkv=2, Sq=4, Sk=4100, D=32,
                 mask_kind=si.MASK_SLIDING, window=300, bias_kind=si.BIAS_T5U),
    BASE.replace(name="dec_d32_full_bias_none_q3_k2001", B=1, Hq=4, Hkv=2, Sq=3, Sk=2001,
                 D=32, mask_kind=si.MASK_NONE, bias_kind=si.BIAS_FULL),
]


def run(sdpa, wl, dev, f32):
    import torch
    q, k, v, bias = dev
    out, lse = sdpa.decode(q, k, v, scale=wl.scale, mask=wl.mask_kind, window=wl.window,
                           bias_kind=wl.bias_kind, bias=bias,
                           out_dtype=torch.float32 if f32 else torch.bfloat16)
    torch.cuda.synchronize()
    return out, lse


def check(sdpa, wl, ref_o, ref_l, heads=None):
    import torch
    inp = si.make_inputs(wl)
    dev = to_device(inp)
    o32, l32 = run(sdpa, wl, dev, True)
    o16, l16 = run(sdpa, wl, dev, False)
    assert torch.equal(o16, o32.to(torch.bfloat16)), "bf16 out != RNE(fp32 out)"
    assert torch.equal(l16, l32), "lse differs between epilogues"
    go, gl = out_to_f64(o32), out_to_f64(l32)
    if heads is not None:
        go = np.stack([go[b, :, h] for b, h in heads])
        gl = np.stack([gl[b, h] for b, h in heads])
    mo, ao = errors(go, ref_o)
    ml, al = errors(gl, ref_l)
    print(f"{wl.name}: O max {mo:.3e} mean {ao:.3e} | LSE max {ml:.3e} mean {al:.3e}",
          flush=True)
    assert mo <= BF16_MAX_ABS and ao <= BF16_MEAN_ABS, (mo, ao)
    assert ml <= BF16_MAX_ABS and al <= BF16_MEAN_ABS, (ml, al)


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_decode_parity_small(gpu_lib, wl):
    ref_o, ref_l = oracle_full(si.make_inputs(wl))
    check(gpu_lib, wl, ref_o, ref_l)


@pytest.mark.parametrize("key", ["dec", "decmqa", "decsw", "decd256"])
def test_decode_parity_full_size_sampled(gpu_lib, key):
    """Full-size decode workload as the benchmark launches it; the oracle on sampled heads
    (all query rows of each)."""
    import torch
    wl = W[key]
    inp = si.make_inputs(wl)
    q, k, v, extra = inp.as_f64()
    rng = np.random.default_rng(len(key))
    heads = [(0, 0), (wl.B - 1, wl.Hq - 1)] + \
        [(int(rng.integers(wl.B)), int(rng.integers(wl.Hq))) for _ in range(6)]
    ref_o, ref_l = [], []
    for b, h in heads:
        o, l = oracle.sdpa_rows(q, k, v, b, h, list(range(wl.Sq)),
                                scale=float(np.float32(wl.scale)), mask_kind=wl.mask_kind,
                                window=wl.window, bias_kind=wl.bias_kind, bias=extra)
        ref_o.append(o)
        ref_l.append(l)
    check(gpu_lib, wl, np.stack(ref_o), np.stack(ref_l), heads=heads)
    torch.cuda.empty_cache()


def test_decode_bitwise_determinism_100_runs(gpu_lib):
    import torch
    wl = W["dec"]
    q, k, v, _ = to_device(si.make_inputs(wl))
    ws = torch.empty((gpu_lib.decode_ws_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.Sk, wl.D),),
                     dtype=torch.uint8, device="cuda")
    o0, l0 = gpu_lib.decode(q, k, v, mask="causal", ws=ws)
    o0, l0 = o0.clone(), l0.clone()
    for _ in range(99):
        o, l = gpu_lib.decode(q, k, v, mask="causal", ws=ws)
        assert torch.equal(o, o0) and torch.equal(l, l0)
    torch.cuda.synchronize()
    print(f"{wl.name}: decode deterministic over 100 runs", flush=True)

