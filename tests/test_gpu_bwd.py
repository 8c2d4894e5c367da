"""GPU parity of the attention gradients: sdpa_bwd / sdpa_bwd_f32out (through the C ABI) against
the fp64 oracle (oracle.sdpa_backward) on the same bf16 inputs.

The gradient kernels take the GPU forward's own bf16 output and fp32 LSE, as a training step
would. Bars (derived in bwd_check.py): every element of dQ, dK, dV within its element-wise
first-order error bound, and the rms error of each tensor at most 2^-8 of its rms value; the
bf16-output entry point returns exactly the round-to-nearest-even of the fp32-output one.
Small cases compare whole tensors (every (batch, KV head) pair); the full-size workloads run
in the launch configuration the benchmark times and are checked on whole (batch, KV head)
pairs. Determinism: 100 repeated backward passes are bitwise identical.
"""
import numpy as np
import pytest

import sdpa_inputs as si
from bwd_check import check_grad, pair_reference
from helpers import out_to_f64, to_device
from test_gpu_parity import SMALL_BF16 as _SMALL_FWD

SMALL_BF16 = list(_SMALL_FWD)

pytestmark = pytest.mark.gpu

W = si.WORKLOADS


def run_fwd_bwd(sdpa, wl, dev, dout_dev, grad_f32=True):
    import torch
    q, k, v, bias = dev
    out, lse = sdpa.fwd(q, k, v, scale=wl.scale, mask=wl.mask_kind, window=wl.window,
                        bias_kind=wl.bias_kind, bias=bias)
    gdt = torch.float32 if grad_f32 else torch.bfloat16
    dq, dk, dv = sdpa.bwd(q, k, v, out, lse, dout_dev, scale=wl.scale, mask=wl.mask_kind,
                          window=wl.window, bias_kind=wl.bias_kind, bias=bias, grad_dtype=gdt)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def dout_device(wl):
    import torch
    return torch.from_numpy(si.make_dout(wl).view(np.int16)).cuda().view(torch.bfloat16)


def check_pairs(sdpa, wl, pairs):
    import torch
    inp = si.make_inputs(wl)
    dev = to_device(inp)
    dod = dout_device(wl)
    out, lse, dq, dk, dv = run_fwd_bwd(sdpa, wl, dev, dod, grad_f32=True)
    _, _, dq16, dk16, dv16 = run_fwd_bwd(sdpa, wl, dev, dod, grad_f32=False)
    for a32, a16, name in ((dq, dq16, "dq"), (dk, dk16, "dk"), (dv, dv16, "dv")):
        assert torch.equal(a16, a32.to(torch.bfloat16)), f"{name}: bf16 != RNE(fp32)"
    q, k, v, extra = inp.as_f64()
    do = si.bf16_bits_to_f64(si.make_dout(wl))
    o_g, l_g = out_to_f64(out), out_to_f64(lse)
    gq, gk, gv = out_to_f64(dq), out_to_f64(dk), out_to_f64(dv)
    G = wl.Hq // wl.Hkv
    worst = {"dq": [0, 0, 0], "dk": [0, 0, 0], "dv": [0, 0, 0]}
    for b, kvh in pairs:
        ref = pair_reference(q, k, v, do, o_g, l_g, b, kvh, scale=wl.scale,
                             mask_kind=wl.mask_kind, window=wl.window, bias_kind=wl.bias_kind,
                             bias=extra)
        gq_pair = gq[b, :, kvh * G:(kvh + 1) * G]
        res = {"dq": check_grad("dq", gq_pair, ref["dq"], ref["bound_dq"]),
               "dk": check_grad("dk", gk[b, :, kvh], ref["dk"], ref["bound_dk"]),
               "dv": check_grad("dv", gv[b, :, kvh], ref["dv"], ref["bound_dv"])}
        for key, r in res.items():
            worst[key] = [max(x, y) for x, y in zip(worst[key], r)]
    print(wl.name + ": " + " | ".join(
        f"{k} max {v[0]:.2e} err/bound {v[1]:.2f} rms {v[2]:.2e}" for k, v in worst.items()),
        flush=True)


@pytest.mark.parametrize("wl", SMALL_BF16, ids=[w.name for w in SMALL_BF16])
def test_bwd_parity_small(gpu_lib, wl):
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.Hkv)]
    check_pairs(gpu_lib, wl, pairs)


FULL = ["c2", "c3", "c4t5", "c4full", "c5mha", "c5gqa", "c2alibi", "c4t5u", "c2d32", "c2d256"]


@pytest.mark.parametrize("key", FULL)
def test_bwd_parity_full_size_pairs(gpu_lib, key):
    """Full-size workload; the oracle checks the last (batch, KV head) pair completely (the
    first for the MHA sweep point as well)."""
    import torch
    wl = W[key]
    pairs = [(wl.B - 1, wl.Hkv - 1)]
    if key in ("c5mha", "c4t5"):
        pairs.append((0, 0))
    check_pairs(gpu_lib, wl, pairs)
    torch.cuda.empty_cache()


def test_bwd_bitwise_determinism_100_runs(gpu_lib):
    import torch
    wl = W["c2"]
    inp = si.make_inputs(wl)
    dev = to_device(inp)
    dod = dout_device(wl)
    q, k, v, bias = dev
    out, lse = gpu_lib.fwd(q, k, v, scale=wl.scale, mask=wl.mask_kind, window=wl.window)
    ref = gpu_lib.bwd(q, k, v, out, lse, dod, scale=wl.scale, mask=wl.mask_kind,
                      window=wl.window)
    ref = [t.clone() for t in ref]
    for _ in range(99):
        got = gpu_lib.bwd(q, k, v, out, lse, dod, scale=wl.scale, mask=wl.mask_kind,
                          window=wl.window)
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
    torch.cuda.synchronize()
    print(f"{wl.name}: backward deterministic over 100 runs", flush=True)


def test_bwd_sliding_window_ge_seqlen_is_causal_bitwise(gpu_lib):
    import torch
    wl = si.small(W["c2"], B=1, Hq=8, Hkv=2, Sq=600, Sk=700, window=700, name_suffix="w_eq")
    inp = si.make_inputs(wl)
    q, k, v, _ = to_device(inp)
    dod = dout_device(wl)
    out, lse = gpu_lib.fwd(q, k, v, mask="causal")
    a = gpu_lib.bwd(q, k, v, out, lse, dod, mask="causal")
    for w in (700, 701, 5000):
        b = gpu_lib.bwd(q, k, v, out, lse, dod, mask="sliding", window=w)
        for x, y in zip(a, b):
            assert torch.equal(x, y), w

