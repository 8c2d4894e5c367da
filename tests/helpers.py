"""Shared helpers for the GPU parity tests: move seeded inputs to the device, run the HIP path
through the C ABI binding, run the fp64 oracle on the same values, compare."""
from __future__ import annotations

import numpy as np

import oracle
import sdpa_inputs as si

BF16_MAX_ABS = 1e-2      # stated bar for bf16 inputs: max-abs error
BF16_MEAN_ABS = 1e-3     # and mean-abs error
F32_MAX_ABS = 1e-5       # stated bar for the fp32 path


def to_device(inp: si.Inputs):
    import torch
    wl = inp.wl

    def dev(a):
        if wl.dtype == "bf16" and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    bias = None
    if wl.bias_kind in (si.BIAS_T5, si.BIAS_T5U, si.BIAS_ALIBI):
        bias = torch.from_numpy(inp.t5_table).cuda()
    elif wl.bias_kind == si.BIAS_FULL:
        bias = dev(inp.bias)
    return q, k, v, bias


def run_gpu(sdpa, wl: si.Workload, dev_inputs, out_f32: bool = False):
    import torch
    q, k, v, bias = dev_inputs
    odt = torch.float32 if (out_f32 or wl.dtype == "f32") else torch.bfloat16
    out, lse = sdpa.fwd(q, k, v, scale=wl.scale, mask=wl.mask_kind, window=wl.window,
                        bias_kind=wl.bias_kind, bias=bias, out_dtype=odt)
    torch.cuda.synchronize()
    return out, lse


def out_to_f64(t) -> np.ndarray:
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_full(inp: si.Inputs, threads: int = 0):
    q, k, v, extra = inp.as_f64()
    wl = inp.wl
    return oracle.sdpa_forward(q, k, v, scale=float(np.float32(wl.scale)), mask_kind=wl.mask_kind,
                               window=wl.window, bias_kind=wl.bias_kind, bias=extra,
                               threads=threads or oracle.default_threads())


def errors(got: np.ndarray, want: np.ndarray):
    """(max-abs, mean-abs) over finite entries; infinities must coincide exactly."""
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(got), fin), "non-finite pattern differs"
    assert np.array_equal(got[~fin], want[~fin]), "infinite entries differ"
    if not fin.any():
        return 0.0, 0.0
    d = np.abs(got[fin] - want[fin])
    return float(d.max()), float(d.mean())


def rne_bf16_of_f32(t_f32):
    """bf16 words that round-to-nearest-even of fp32 tensor values gives (torch on device)."""
    import torch
    return t_f32.to(torch.bfloat16)


def sample_rows(Sq: int, n: int, seed: int):
    """Row indices that cover the first rows, tile edges (multiples of 64/128 +-1), the last
    row, plus random ones."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, 129, Sq // 2, Sq - 129, Sq - 128, Sq - 2, Sq - 1]
    rows = {r for r in fixed if 0 <= r < Sq}
    while len(rows) < min(Sq, len(rows) + n):
        rows.add(int(rng.integers(0, Sq)))
    return sorted(rows)
