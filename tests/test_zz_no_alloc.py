"""sdpa_decode_noalloc: the decode entry point for callers that cannot allocate.

Called through the C ABI with raw device pointers, it must return exactly what sdpa_decode
(the same kernels with a caller-owned workspace) returns, bit for bit, on two calls in a row,
the second with a smaller input (the scratch keeps the first call's partials), and meet the
forward's bars against the fp64 oracle. Validation happens before any HIP call, so the refusals
below need no GPU.
"""
import numpy as np
import pytest

import oracle
import sdpa_inputs as si
import scaled_dot_product_03_amd as sdpa
from helpers import BF16_MAX_ABS, BF16_MEAN_ABS, errors, oracle_full, out_to_f64, to_device

BASE = si.WORKLOADS["dec"]
P = 0x10000          # fake, aligned, never-dereferenced device address


def call_noalloc(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, D, scale, mask_kind, window, bias_kind,
                 bias, stream):
    import ctypes
    return sdpa.load().sdpa_decode_noalloc(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, D,
                                           ctypes.c_float(scale), mask_kind, window, bias_kind,
                                           bias, stream)


def test_noalloc_refuses_before_any_hip_call():
    good = dict(q=P, k=P, v=P, out=P, lse=P, B=1, Hq=4, Hkv=2, Sq=1, Sk=4096, D=128,
                scale=0.1, mask_kind=1, window=0, bias_kind=0, bias=None, stream=None)
    for kw, code in [(dict(q=None), 1), (dict(B=0), 2), (dict(Hkv=3), 3), (dict(D=96), 4),
                     (dict(mask_kind=7), 5), (dict(mask_kind=2, window=0), 6),
                     (dict(bias_kind=1), 7), (dict(scale=float("inf")), 8),
                     (dict(out=P + 2), 9)]:
        a = dict(good, **kw)
        assert call_noalloc(**a) == code, kw
    # partials beyond the scratch: 255 groups of one row block, 2 splits, D = 256
    a = dict(good, B=255, Hq=1, Hkv=1, Sq=1, Sk=1024, D=256)
    need = sdpa.decode_ws_bytes(255, 1, 1, 1, 1024, 256)
    assert need > sdpa.DECODE_SCRATCH_BYTES
    assert call_noalloc(**a) == 11


def test_scratch_covers_the_decode_workloads():
    for key in ("dec", "decmqa", "decsw", "decd256"):
        w = si.WORKLOADS[key]
        assert sdpa.decode_ws_bytes(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D) \
            <= sdpa.DECODE_SCRATCH_BYTES, key


def _pair(wl, dev):
    """(noalloc out, lse) and (sdpa_decode out, lse) on the same inputs, through the C ABI."""
    import torch
    q, k, v, bias = dev
    stream = torch.cuda.current_stream().cuda_stream
    bias_ptr = None if bias is None else bias.data_ptr()
    outs = []
    for entry in ("noalloc", "decode"):
        out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((wl.B, wl.Hq, wl.Sq), float("nan"), dtype=torch.float32,
                         device="cuda")
        if entry == "noalloc":
            st = call_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.Sk, wl.D, wl.scale,
                              wl.mask_kind, wl.window, wl.bias_kind, bias_ptr, stream)
        else:
            need = sdpa.decode_ws_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.Sk, wl.D)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
            st = sdpa.call_raw_decode("sdpa_decode", q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      out.data_ptr(), lse.data_ptr(), ws.data_ptr(), need,
                                      wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.Sk, wl.D, wl.scale,
                                      wl.mask_kind, wl.window, wl.bias_kind, bias_ptr, stream)
        assert st == 0, (entry, sdpa.status_str(st))
        torch.cuda.synchronize()
        outs.append((out, lse))
    return outs


@pytest.mark.gpu
def test_noalloc_equals_decode_two_calls_second_smaller(gpu_lib):
    import torch
    first = BASE.replace(name="noalloc_b4_g4_k8192", B=4, Hq=32, Hkv=8, Sq=1, Sk=8192)
    second = BASE.replace(name="noalloc_b1_g4_q3_k1500_t5", B=1, Hq=8, Hkv=2, Sq=3, Sk=1500,
                          bias_kind=si.BIAS_T5)
    for wl in (first, second):
        inp = si.make_inputs(wl)
        (o_n, l_n), (o_d, l_d) = _pair(wl, to_device(inp))
        assert torch.equal(o_n, o_d) and torch.equal(l_n, l_d), wl.name
        # the forward's bars against the oracle (bf16 output: the codelab's allclose)
        ro, rl = oracle_full(inp)
        got = out_to_f64(o_n)
        assert np.allclose(got, ro, rtol=BF16_MAX_ABS, atol=BF16_MAX_ABS), wl.name
        el = errors(out_to_f64(l_n), rl)
        assert el[0] <= BF16_MAX_ABS and el[1] <= BF16_MEAN_ABS, (wl.name, el)
        print(f"{wl.name}: noalloc == decode bit for bit; lse max-abs {el[0]:.2e}")


@pytest.mark.gpu
def test_noalloc_single_split_and_d256(gpu_lib):
    import torch
    for wl in (BASE.replace(name="noalloc_single_split_k300", B=1, Hq=8, Hkv=2, Sk=300),
               BASE.replace(name="noalloc_d256_b2_k3000", B=2, Hq=8, Hkv=2, Sk=3000, D=256)):
        inp = si.make_inputs(wl)
        (o_n, l_n), (o_d, l_d) = _pair(wl, to_device(inp))
        assert torch.equal(o_n, o_d) and torch.equal(l_n, l_d), wl.name


@pytest.mark.gpu
def test_noalloc_binding_allocates_nothing_and_matches(gpu_lib):
    import torch
    wl = BASE.replace(name="noalloc_binding_b2_k4000", B=2, Hq=8, Hkv=2, Sq=2, Sk=4000)
    q, k, v, bias = to_device(si.make_inputs(wl))
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((wl.B, wl.Hq, wl.Sq), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    o, l = gpu_lib.decode_noalloc(q, k, v, out, lse, scale=wl.scale, mask=wl.mask_kind)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert o is out and l is lse
    o2, l2 = gpu_lib.decode(q, k, v, scale=wl.scale, mask=wl.mask_kind)
    assert torch.equal(o, o2) and torch.equal(l, l2)
