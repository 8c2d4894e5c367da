"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2] [--sweep]

A step is one fused forward (tile plan, Q load, K/V streaming, Q.K^T, mask/bias, online
softmax, P.V, epilogue: one kernel launch) over one batch of synthetic input already resident
in HBM. The default workload is the Mistral-7B-shaped GQA prefill: B=4, Hq=32, Hkv=8, S=4096,
D=128, bf16, sliding window 4096 (= seqlen, i.e. exactly causal).

Prints ONE JSON line on stdout. `value` is effective TFLOP/s: 4*D flop per visible
(query, key) pair (Q.K^T and P.V), masked pairs excluded, exps not counted. Timing: W untimed
warmup launches, then untimed settle launches in batches of 10 until two consecutive batch
medians agree within 1 % (at least 0.5 s; the GPU clocks ramp up after idling), then exactly K
launches bracketed by device synchronisation (wall clock: `value`, `ms_per_step`), each of them
also bracketed by HIP events on the launch stream (average kernel duration: `roofline`). This
is the repeat-with-device-sync method of the "jax-gpu-05-attention-gpu" codelab, section 8.
The line's `sweep` object carries the same measurement for the other target workloads (the
S = 8192 sliding window and its full-causal comparison, the T5 encoder with bucketed and full
bias, the head-sharing sweep, the tiny fp32 case). The CPU baseline is the fp64 oracle timed on
the same workload on this host's cores.

--sweep additionally times the extra bias kinds and head dims and prints one JSON line per
workload on stderr; --no-sweep times the headline workload only.

--decode measures the split-key decode instead (default workload: one new query row per head
against a 16384-key cache, B16, Mistral-7B heads): a step is one sdpa_decode call (split
kernel + merge kernel); `value` is HBM GB/s over the algorithmic bytes (visible K/V range, q,
out, lse); the roofline is HBM-bound against 8 TB/s. The CPU baseline is the fp64 oracle on
the same rows.

--varlen measures packed variable-length sequences (32768 tokens of Mistral-7B heads in
sequences of seeded log-normal lengths, causal inside each): a step is one sdpa_fwd_varlen
call; `value` is effective TFLOP/s over the visible pairs of all sequences (4*D flop each).

--bwd measures the gradients instead: a step is one sdpa_bwd call (dQ, dK, dV of
sum(dO * O), two kernel launches) on the same workload, with O and the LSE produced by the
forward once before the timed region. `value` counts 10*D flop per visible pair (the five
products S, dP, dV, dQ, dK; the kernels recompute S and dP, which is not counted), and the
roofline entry covers the whole call (both launches) timed with HIP events on its stream.
The CPU baseline is the fp64 gradient oracle on whole (batch, KV head) pairs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import sdpa_inputs as si  # noqa: E402

METRIC = "attention fwd effective TFLOP/s (masked tiles excluded) + % of bf16 MFMA peak"
METRIC_BWD = ("attention bwd (dQ, dK, dV) effective TFLOP/s, 10*D flop per visible pair "
              "(masked tiles excluded) + % of bf16 MFMA peak")
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, published
# kernel sources and the C ABI (which picks the kernel variant) of each profiled path
KERNEL_SOURCES = ["scaled_dot_product_03_amd/csrc/sdpa_fwd_bf16.hip",
                  "scaled_dot_product_03_amd/csrc/sdpa_params.h",
                  "scaled_dot_product_03_amd/csrc/sdpa_api.hip"]
TRAFFIC_FILE = "profiles/sdpa_fwd_bf16_c2_traffic.json"
KERNEL_SOURCES_BWD = ["scaled_dot_product_03_amd/csrc/sdpa_bwd_bf16.hip",
                      "scaled_dot_product_03_amd/csrc/sdpa_device.h",
                      "scaled_dot_product_03_amd/csrc/sdpa_params.h",
                      "scaled_dot_product_03_amd/csrc/sdpa_api.hip"]
TRAFFIC_FILE_BWD = "profiles/sdpa_bwd_bf16_c2_traffic.json"
METRIC_DEC = "attention decode HBM GB/s (visible K/V range + q, out, lse) + % of HBM peak"
KERNEL_SOURCES_DEC = ["scaled_dot_product_03_amd/csrc/sdpa_decode_bf16.hip",
                      "scaled_dot_product_03_amd/csrc/sdpa_decode.h",
                      "scaled_dot_product_03_amd/csrc/sdpa_device.h",
                      "scaled_dot_product_03_amd/csrc/sdpa_params.h",
                      "scaled_dot_product_03_amd/csrc/sdpa_api.hip"]
TRAFFIC_FILE_DEC = "profiles/sdpa_decode_bf16_dec_traffic.json"


def kernel_sha(sources=None) -> str:
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, bwd: bool = False, decode: bool = False):
    """HBM bytes per launch (per call with bwd / decode) measured by rocprofv3 counters, if
    taken on this exact kernel source."""
    path = os.path.join(ROOT, TRAFFIC_FILE_DEC if decode else
                        (TRAFFIC_FILE_BWD if bwd else TRAFFIC_FILE))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    sha = kernel_sha(KERNEL_SOURCES_DEC if decode else
                     (KERNEL_SOURCES_BWD if bwd else KERNEL_SOURCES))
    if rec.get("kernel_sha") != sha or rec.get("workload") != workload:
        return None
    return rec.get("traffic_bytes_per_launch")


def to_device(inp: si.Inputs):
    import torch

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bias = None
    if inp.wl.bias_kind in (si.BIAS_T5, si.BIAS_T5U, si.BIAS_ALIBI):
        bias = torch.from_numpy(inp.t5_table).cuda()
    elif inp.wl.bias_kind == si.BIAS_FULL:
        bias = dev(inp.bias)
    return dev(inp.q), dev(inp.k), dev(inp.v), bias


def settle(launch, stream, warmup: int, min_s: float = 0.5, max_s: float = 4.0,
           batch: int = 10, tol: float = 0.01) -> int:
    """Untimed launches until the GPU clocks have settled: `warmup` launches, then batches of
    `batch` launches, each timed with HIP events on the launch stream, until two consecutive
    batch medians agree within `tol` and at least `min_s` seconds have passed (at most
    `max_s`). Clocks ramp up over the first launches after the GPU idles; without this the
    ramp would fall inside the timed region. Returns the number of launches after `warmup`."""
    import torch
    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    n, prev = 0, None
    t0 = time.perf_counter()
    while True:
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(batch)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(batch)]
        for i in range(batch):
            starts[i].record(stream)
            launch()
            ends[i].record(stream)
        torch.cuda.synchronize()
        n += batch
        med = float(np.median([a.elapsed_time(b) for a, b in zip(starts, ends)]))
        el = time.perf_counter() - t0
        if prev is not None and abs(med - prev) <= tol * prev and el >= min_s:
            return n
        if el >= max_s:
            return n
        prev = med


def timed_launches(launch, stream, steps: int):
    """Exactly `steps` launches between two device synchronisations (wall clock), each
    bracketed by HIP events on the launch stream (per-launch kernel duration). The events are
    recorded inside the timed region, so both statistics describe the same launches."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    return dict(ms_per_step=1e3 * wall / steps, kernel_ms_avg=float(ev.mean()),
                kernel_ms_median=float(np.median(ev)), kernel_ms_min=float(ev.min()),
                kernel_ms_max=float(ev.max()))


def time_workload(sdpa, wl: si.Workload, steps: int, warmup: int, bwd: bool = False,
                  decode: bool = False, min_settle: float = 0.5):
    """Returns dict with ms_per_step (wall, synchronised), kernel_ms_avg / median (events over
    the same launches) and the number of settle launches. With bwd, a step is one gradient
    call (dQ, dK, dV) instead of one forward; with decode, one split-key decode call."""
    import torch
    inp = si.make_inputs(wl)
    q, k, v, bias = to_device(inp)
    del inp
    odt = torch.float32 if wl.dtype == "f32" else q.dtype
    out = torch.empty(q.shape, dtype=odt, device=q.device)
    lse = torch.empty((wl.B, wl.Hq, wl.Sq), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    kw = dict(scale=wl.scale, mask=wl.mask_kind, window=wl.window, bias_kind=wl.bias_kind,
              bias=bias, stream=stream.cuda_stream)
    if bwd:
        sdpa.fwd(q, k, v, out=out, lse=lse, **kw)
        dout = torch.from_numpy(si.make_dout(wl).view(np.int16)).cuda().view(torch.bfloat16)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty((wl.B * wl.Hq * wl.Sq,), dtype=torch.float32, device=q.device)

        def launch():
            sdpa.bwd(q, k, v, out, lse, dout, dq=dq, dk=dk, dv=dv, ws=ws, **kw)
    elif decode:
        wsd = torch.empty((max(16, sdpa.decode_ws_bytes(wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.Sk,
                                                        wl.D)),), dtype=torch.uint8,
                          device=q.device)

        def launch():
            sdpa.decode(q, k, v, out=out, lse=lse, ws=wsd, **kw)
    else:
        def launch():
            sdpa.fwd(q, k, v, out=out, lse=lse, **kw)

    n_settle = settle(launch, stream, warmup, min_s=min_settle)
    t = timed_launches(launch, stream, steps)
    t["settle_launches"] = n_settle
    del q, k, v, bias, out, lse, launch
    torch.cuda.empty_cache()
    return t


def cpu_baseline(wl: si.Workload, budget_s: float = 12.0):
    """The fp64 oracle on the same workload, timed on this host's cores: (batch, head) pairs
    in rounds of `threads` pairs (one pair per thread, BLAS pinned to one thread each) until
    the whole workload is done or the time budget is spent, repeating the workload while less
    than half the budget has elapsed. Effective TFLOP/s over the pairs it finished."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:          # pragma: no cover
        threadpool_limits = None
    threads = oracle.default_threads()
    inp = si.make_inputs(wl)
    q, k, v, extra = inp.as_f64()
    del inp
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.Hq)]
    done = 0
    passes = 0
    t0 = time.perf_counter()
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        while True:
            i = done % len(pairs)
            chunk = pairs[i:i + threads]
            oracle.sdpa_forward(q, k, v, scale=float(np.float32(wl.scale)),
                                mask_kind=wl.mask_kind, window=wl.window,
                                bias_kind=wl.bias_kind, bias=extra, threads=threads,
                                heads=chunk)
            done += len(chunk)
            el = time.perf_counter() - t0
            if done % len(pairs) == 0:
                passes += 1
                if el >= budget_s / 2:
                    break
            if el >= budget_s:
                break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    secs = time.perf_counter() - t0
    per_head = 4.0 * wl.D * si.visible_pairs(wl.Sq, wl.Sk, wl.mask_kind, wl.window)
    what = (f"the whole workload {passes}x" if done % len(pairs) == 0 and passes
            else f"{done} of {len(pairs)} (batch, head) pairs")
    return {"value": per_head * done / secs / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{what} of {wl.name} ({len(pairs)} (batch, head) pairs, all "
                      f"{wl.Sq} query rows each), fp64 numpy, one pair per thread, "
                      f"{secs:.1f} s"}


def cpu_baseline_bwd(wl: si.Workload, budget_s: float = 15.0):
    """The fp64 gradient oracle on the same workload, timed on this host's cores: whole
    (batch, KV head) pairs (all G query heads, all rows), one after the other with BLAS on every
    core, until the workload is done or the budget is spent (at least one pair)."""
    import oracle
    threads = oracle.default_threads()
    inp = si.make_inputs(wl)
    q, k, v, extra = inp.as_f64()
    del inp
    do = si.bf16_bits_to_f64(si.make_dout(wl))
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.Hkv)]
    done = 0
    t0 = time.perf_counter()
    while done < len(pairs):
        oracle.sdpa_backward(q, k, v, do, scale=float(np.float32(wl.scale)),
                             mask_kind=wl.mask_kind, window=wl.window, bias_kind=wl.bias_kind,
                             bias=extra, kv_heads=[pairs[done]])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    secs = time.perf_counter() - t0
    G = wl.Hq // wl.Hkv
    per_pair = 10.0 * wl.D * si.visible_pairs(wl.Sq, wl.Sk, wl.mask_kind, wl.window) * G
    return {"value": per_pair * done / secs / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} of {len(pairs)} (batch, KV head) pairs of {wl.name} (each: "
                      f"{G} query heads x {wl.Sq} rows, dQ, dK, dV), fp64 numpy with BLAS on "
                      f"{threads} threads, {secs:.1f} s"}


def cpu_baseline_decode(wl: si.Workload, budget_s: float = 15.0):
    """The fp64 oracle on the decode workload's rows, timed on this host's cores: (batch, head)
    pairs in rounds of `threads` (one pair per thread, BLAS pinned to one thread each) until
    the workload is done or the budget is spent. GB/s over the same algorithmic bytes."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:          # pragma: no cover
        threadpool_limits = None
    threads = oracle.default_threads()
    inp = si.make_inputs(wl)
    q, k, v, extra = inp.as_f64()
    del inp
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.Hq)]
    done = 0
    t0 = time.perf_counter()
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        while done < len(pairs) and time.perf_counter() - t0 < budget_s:
            chunk = pairs[done:done + threads]
            oracle.sdpa_forward(q, k, v, scale=float(np.float32(wl.scale)),
                                mask_kind=wl.mask_kind, window=wl.window,
                                bias_kind=wl.bias_kind, bias=extra, threads=threads,
                                heads=chunk)
            done += len(chunk)
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    secs = time.perf_counter() - t0
    per_pair = si.algorithmic_bytes_decode(wl) / len(pairs)
    return {"value": per_pair * done / secs / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} of {len(pairs)} (batch, head) pairs of {wl.name} (all {wl.Sq} "
                      f"query rows each), fp64 numpy, one pair per thread, {secs:.1f} s"}


def tile_flops(wl: si.Workload) -> float:
    """FLOP of the matrix work the bf16 kernel performs: 4*D per (row, key) slot of every block
    of 32 query rows x 64 keys it computes, masked slots included. Follows the kernel's tile
    plan: the key range of each 256-row work item, minus the 64-key tiles that a 32-row wave
    skips because the mask hides them completely. One such block is D/4 MFMAs of
    v_mfma_f32_32x32x16_bf16 (32768 flop each: D/8 for the two 32-key halves of S, D/8 for
    the D/32 head-dim blocks of P.V over four 16-key groups), so rocprofv3's SQ_INSTS_MFMA
    times 32768 must equal this count (the profile summaries check it)."""
    off = wl.Sk - wl.Sq
    blocks = 0
    for q0 in range(0, wl.Sq, 256):
        pa, pb = q0 + off, min(q0 + 256, wl.Sq) - 1 + off
        khi, klo = wl.Sk - 1, 0
        if wl.mask_kind != si.MASK_NONE:
            khi = min(khi, pb)
        if wl.mask_kind == si.MASK_SLIDING:
            klo = max(0, pa - wl.window + 1)
        if khi < klo:
            continue
        for wq0 in range(q0, min(q0 + 256, wl.Sq), 32):
            pwa, pwb = wq0 + off, min(wq0 + 31, wl.Sq - 1) + off
            for t in range(klo // 64, khi // 64 + 1):
                j0 = 64 * t
                if wl.mask_kind != si.MASK_NONE and j0 > pwb:
                    continue
                if wl.mask_kind == si.MASK_SLIDING and j0 + 63 <= pwa - wl.window:
                    continue
                blocks += 1
    return 4.0 * wl.D * 32 * 64 * blocks * wl.B * wl.Hq


def bwd_tile_mfmas(wl: si.Workload):
    """MFMA instructions (v_mfma_f32_32x32x16_bf16) the two gradient kernels issue, following
    their tile plans: (dq kernel, dk/dv kernel) per launch.

    dq kernel: work items of 256 query rows (128 at D = 256), 64-key tiles over the item's key
    range; a 32-row wave computes a tile unless the mask hides it completely, issuing per
    32-key half D/16 MFMAs for S, D/16 for dP and 2 * D/32 for dQ. dk/dv kernel: 128 keys per
    workgroup (64 at D = 256), steps of query rows over the G query heads; each 32-key group
    has a dV wave and a dK wave, which skip the 32-row blocks the mask hides completely.
    Without a full bias, and with one at D = 64 (steps of 64 rows; 128 at D = 32, 32 at
    D = 256), the dV wave forms S and P (D/16, then 2 * D/32 for dV) and the dK wave takes
    that P (D/16 for dP, 2 * D/32 for dK); with a full bias at D = 32, 128 and 256 (steps of
    128 rows, 64 at D = 128 and 256) the dK wave forms S itself as well (2 * D/16, then
    2 * D/32)."""
    off, D, W = wl.Sk - wl.Sq, wl.D, wl.window
    G = wl.Hq // wl.Hkv
    causal = wl.mask_kind != si.MASK_NONE
    sliding = wl.mask_kind == si.MASK_SLIDING
    rows = 128 if D == 256 else 256
    per_half = 2 * (D // 16) + 2 * (D // 32)
    dq = 0
    for q0 in range(0, wl.Sq, rows):
        pa, pb = q0 + off, min(q0 + rows, wl.Sq) - 1 + off
        khi, klo = wl.Sk - 1, 0
        if causal:
            khi = min(khi, pb)
        if sliding:
            klo = max(0, pa - W + 1)
        if khi < klo:
            continue
        for wq0 in range(q0, min(q0 + rows, wl.Sq), 32):
            pwa, pwb = wq0 + off, min(wq0 + 31, wl.Sq - 1) + off
            for t in range(klo // 64, khi // 64 + 1):
                j0 = 64 * t
                if causal and j0 > pwb:
                    continue
                if sliding and j0 + 63 <= pwa - W:
                    continue
                dq += 2 * per_half
    handoff = wl.bias_kind != si.BIAS_FULL or D == 64
    if handoff:
        kbq = 32 if D == 256 else (128 if D == 32 else 64)
    else:
        kbq = 64 if D in (128, 256) else 128
    kbk = 64 if D == 256 else 128
    per_dv = D // 16 + 2 * (D // 32)
    per_dk = (1 if handoff else 2) * (D // 16) + 2 * (D // 32)
    dkdv = 0
    for k0 in range(0, wl.Sk, kbk):
        kend = min(k0 + kbk, wl.Sk) - 1
        qlo, qhi = 0, wl.Sq
        if causal:
            qlo = max(0, k0 - off)
        if sliding:
            qhi = min(wl.Sq, kend + min(W, wl.Sk + 1) - off)
        if qhi <= qlo:
            continue
        for kw0 in range(k0, min(k0 + kbk, wl.Sk), 32):
            kwe = min(kw0 + 31, wl.Sk - 1)
            for s0 in range((qlo // kbq) * kbq, qhi, kbq):
                for r0 in range(s0, s0 + kbq, 32):
                    if r0 >= wl.Sq:
                        continue
                    pa, pb = r0 + off, min(r0 + 31, wl.Sq - 1) + off
                    if causal and pb < kw0:
                        continue
                    if sliding and pa - kwe >= min(W, wl.Sk + 1):
                        continue
                    dkdv += G * (per_dv + per_dk)
    return dq * wl.B * wl.Hq, dkdv * wl.B * wl.Hkv


def report(wl: si.Workload, t: dict, bwd: bool = False):
    flops = si.effective_flops(wl) * (2.5 if bwd else 1.0)
    achieved = flops / (t["kernel_ms_avg"] * 1e-3) / 1e12
    return flops, achieved


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None, choices=sorted(si.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--min-settle", type=float, default=0.5, metavar="S",
                    help="least seconds of settle launches before the timed region (counter "
                         "runs use 0: the profiler serialises dispatches)")
    ap.add_argument("--sweep", action="store_true",
                    help="also time the extra bias kinds and head dims (stderr)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="time the headline workload only (no 'sweep' object in the line)")
    ap.add_argument("--bwd", action="store_true",
                    help="time the gradient call (dQ, dK, dV) instead of the forward")
    ap.add_argument("--decode", action="store_true",
                    help="time the split-key decode (workload default: dec)")
    ap.add_argument("--varlen", action="store_true",
                    help="time packed variable-length sequences (workload vl)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of attention, run `steps` device-to-device copies of MIB "
                         "MiB (reference kernel for scaling HBM byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on exactly one GPU (asked for {args.gpus}); "
              "the attention forward has no multi-GPU path", file=sys.stderr)
        return 2

    import torch
    import scaled_dot_product_03_amd as sdpa
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    sdpa.load()

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(7)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n,
                          "launches": args.steps}), flush=True)
        return 0

    if args.varlen:
        return main_varlen(sdpa, si.VARLEN_WORKLOADS["vl"], args)
    wl = si.WORKLOADS[args.workload or ("dec" if args.decode else "c2")]
    if args.bwd:
        return main_bwd(sdpa, wl, args)
    if args.decode:
        return main_decode(sdpa, wl, args)
    t = time_workload(sdpa, wl, args.steps, args.warmup, min_settle=args.min_settle)
    flops, achieved = report(wl, t)
    value = flops / (t["ms_per_step"] * 1e-3) / 1e12
    traffic = load_traffic(wl.name)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_launches": t["settle_launches"],
        "ms_per_step": round(t["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {**wl.describe(), "effective_gflop": round(flops / 1e9, 2),
                   "tile_gflop": round(tile_flops(wl) / 1e9, 2),
                   "tile_tflops": round(tile_flops(wl) / (t["kernel_ms_avg"] * 1e-3) / 1e12, 2),
                   "kernel_ms_avg": round(t["kernel_ms_avg"], 4),
                   "kernel_ms_median": round(t["kernel_ms_median"], 4),
                   "wall_over_kernel": round(t["ms_per_step"] / t["kernel_ms_avg"], 4),
                   "hbm_gbs_algorithmic": round(si.algorithmic_bytes(wl) /
                                                (t["kernel_ms_avg"] * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    if not args.no_sweep:
        line["sweep"] = sweep_forward(sdpa, SWEEP_DEFAULT, args.steps, args.warmup,
                                      args.min_settle)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)

    if args.sweep:
        for key in SWEEP_EXTRA:
            rec = sweep_forward(sdpa, [key], args.steps, args.warmup, args.min_settle)[key]
            print(json.dumps({"workload": key, **si.WORKLOADS[key].describe(), **rec}),
                  file=sys.stderr, flush=True)
    return 0


# the other target workloads, timed in the default run and carried in the line's "sweep"
# object: c2c (the causal twin of the headline), the S = 8192 sliding window and its full-
# causal comparison, the T5 encoder with bucketed and with full bias, the head-sharing sweep,
# and the tiny fp32 case
SWEEP_DEFAULT = ["c2c", "c3", "c3c", "c4t5", "c4full", "c5mha", "c5gqa", "c5mqa", "c1"]
# more index-generated biases and head dims (--sweep, printed on stderr)
SWEEP_EXTRA = ["c2alibi", "c4t5u", "c2d32", "c2d256"]


def sweep_forward(sdpa, keys, steps: int, warmup: int, min_settle: float = 0.5) -> dict:
    """Times each workload like the headline (settle, then `steps` launches with per-launch
    events) and returns {key: record}; adds the sliding/causal time ratios when both sides
    were timed."""
    out = {}
    for key in keys:
        w2 = si.WORKLOADS[key]
        t2 = time_workload(sdpa, w2, steps, warmup, min_settle=min_settle)
        f2, a2 = report(w2, t2)
        rec = {"kernel_ms_avg": round(t2["kernel_ms_avg"], 4),
               "kernel_ms_median": round(t2["kernel_ms_median"], 4),
               "effective_tflops": round(a2, 2),
               "pct_of_bf16_peak": round(100 * a2 / PEAK_BF16_TFLOPS, 2),
               "hbm_gbs_algorithmic": round(si.algorithmic_bytes(w2) /
                                            (t2["kernel_ms_avg"] * 1e-3) / 1e9, 1),
               "settle_launches": t2["settle_launches"]}
        if w2.dtype == "bf16":
            rec["tile_tflops"] = round(tile_flops(w2) / (t2["kernel_ms_avg"] * 1e-3) / 1e12, 2)
        out[key] = rec
    # a sliding window of 4096 at S = 8192 keeps 0.750 of the causal pairs
    if "c3" in out and "c3c" in out:
        out["c3_over_c3c"] = {
            "time_ratio": round(out["c3"]["kernel_ms_avg"] / out["c3c"]["kernel_ms_avg"], 4),
            "pairs_ratio": round(si.effective_flops(si.WORKLOADS["c3"]) /
                                 si.effective_flops(si.WORKLOADS["c3c"]), 4),
            "tile_ratio": round(tile_flops(si.WORKLOADS["c3"]) /
                                tile_flops(si.WORKLOADS["c3c"]), 4)}
    return out


def time_varlen(sdpa, wl, steps: int, warmup: int, min_settle: float = 0.5):
    import torch
    inp = si.make_varlen_inputs(wl)

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    q, k, v = bf(inp.q), bf(inp.k), bf(inp.v)
    cq, ck = torch.from_numpy(inp.cu_q).cuda(), torch.from_numpy(inp.cu_k).cuda()
    m = int(np.diff(inp.cu_q).max())
    out = torch.empty_like(q)
    lse = torch.empty((wl.Hq, q.shape[0]), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()

    def launch():
        sdpa.fwd_varlen(q, k, v, cq, ck, m, m, scale=wl.scale, mask=wl.mask_kind,
                        window=wl.window, out=out, lse=lse, stream=stream.cuda_stream)
    n_settle = settle(launch, stream, warmup, min_s=min_settle)
    t = timed_launches(launch, stream, steps)
    t["settle_launches"] = n_settle
    return t


def cpu_baseline_varlen(wl, budget_s: float = 12.0):
    """The fp64 packed-sequence oracle on whole sequences of the pack, shortest first, until
    the budget is spent; TFLOP/s over their visible pairs."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:          # pragma: no cover
        threadpool_limits = None
    inp = si.make_varlen_inputs(wl)
    q, k, v, _ = inp.as_f64()
    lens = np.diff(inp.cu_q)
    order = np.argsort(lens)
    threads = oracle.default_threads()
    done, flops = 0, 0.0
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    t0 = time.perf_counter()
    try:
        for s in order:
            a, b = int(inp.cu_q[s]), int(inp.cu_q[s + 1])
            oracle.sdpa_forward_varlen(q[a:b], k[a:b], v[a:b], [0, b - a], [0, b - a],
                                       scale=wl.scale, mask_kind=wl.mask_kind, window=wl.window,
                                       threads=threads)
            done += 1
            flops += 4.0 * wl.D * wl.Hq * si.visible_pairs(b - a, b - a, wl.mask_kind,
                                                            wl.window)
            if time.perf_counter() - t0 >= budget_s:
                break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    secs = time.perf_counter() - t0
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} of {len(lens)} sequences of {wl.name} (shortest first, all heads "
                      f"and rows), fp64 numpy, one head per thread (BLAS on one thread each), "
                      f"{secs:.1f} s"}


def main_varlen(sdpa, wl, args) -> int:
    t = time_varlen(sdpa, wl, args.steps, args.warmup, args.min_settle)
    flops = 4.0 * wl.D * wl.Hq * si.varlen_visible_pairs(wl)
    value = flops / (t["ms_per_step"] * 1e-3) / 1e12
    achieved = flops / (t["kernel_ms_avg"] * 1e-3) / 1e12
    line = {
        "metric": "attention fwd over packed sequences, effective TFLOP/s (visible pairs of "
                  "every sequence) + % of bf16 MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_launches": t["settle_launches"],
        "ms_per_step": round(t["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {**wl.describe(), "effective_gflop": round(flops / 1e9, 2),
                   "call_ms_median": round(t["kernel_ms_median"], 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_varlen(wl)
    print(json.dumps(line), flush=True)
    return 0


def main_decode(sdpa, wl: si.Workload, args) -> int:
    t = time_workload(sdpa, wl, args.steps, args.warmup, decode=True,
                      min_settle=args.min_settle)
    nbytes = si.algorithmic_bytes_decode(wl)
    value = nbytes / (t["ms_per_step"] * 1e-3) / 1e9
    achieved = nbytes / (t["kernel_ms_avg"] * 1e-3) / 1e9
    line = {
        "metric": METRIC_DEC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_launches": t["settle_launches"],
        "ms_per_step": round(t["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_hbm_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "config": {**wl.describe(), "pass": "decode (split keys + merge)",
                   "algorithmic_mb": round(nbytes / 1e6, 2),
                   "call_ms_median": round(t["kernel_ms_median"], 4),
                   "call_ms_avg": round(t["kernel_ms_avg"], 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": load_traffic(wl.name, decode=True),
                     "unit_of_work": "one decode call (split kernel + merge kernel)"},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(wl)
    print(json.dumps(line), flush=True)
    if args.sweep:
        for key in ["dec", "decmqa", "decsw", "decd256"]:
            w2 = si.WORKLOADS[key]
            t2 = time_workload(sdpa, w2, args.steps, args.warmup, decode=True,
                               min_settle=args.min_settle)
            nb = si.algorithmic_bytes_decode(w2)
            rec = {"workload": key, "pass": "decode", **w2.describe(),
                   "call_ms_avg": round(t2["kernel_ms_avg"], 4),
                   "call_ms_median": round(t2["kernel_ms_median"], 4),
                   "hbm_gbs": round(nb / (t2["kernel_ms_avg"] * 1e-3) / 1e9, 1),
                   "pct_of_hbm_peak": round(100 * nb / (t2["kernel_ms_avg"] * 1e-3) / 1e9 /
                                            PEAK_HBM_GBS, 2)}
            print(json.dumps(rec), file=sys.stderr, flush=True)
    return 0


def main_bwd(sdpa, wl: si.Workload, args) -> int:
    t = time_workload(sdpa, wl, args.steps, args.warmup, bwd=True, min_settle=args.min_settle)
    flops, achieved = report(wl, t, bwd=True)
    value = flops / (t["ms_per_step"] * 1e-3) / 1e12
    line = {
        "metric": METRIC_BWD,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_launches": t["settle_launches"],
        "ms_per_step": round(t["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {**wl.describe(), "pass": "backward (dQ, dK, dV)",
                   "effective_gflop": round(flops / 1e9, 2),
                   "call_ms_median": round(t["kernel_ms_median"], 4),
                   "call_ms_avg": round(t["kernel_ms_avg"], 4),
                   "hbm_gbs_algorithmic": round(si.algorithmic_bytes_bwd(wl) /
                                                (t["kernel_ms_avg"] * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": load_traffic(wl.name, bwd=True),
                     "unit_of_work": "one gradient call (dQ kernel + dK/dV kernel)"},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_bwd(wl)
    print(json.dumps(line), flush=True)
    if args.sweep:
        for key in ["c2", "c3", "c3c", "c4t5", "c4full", "c5mha", "c5gqa", "c5mqa", "c2alibi",
                    "c4t5u", "c2d32", "c2d256"]:
            w2 = si.WORKLOADS[key]
            t2 = time_workload(sdpa, w2, args.steps, args.warmup, bwd=True,
                               min_settle=args.min_settle)
            f2, a2 = report(w2, t2, bwd=True)
            rec = {"workload": key, "pass": "backward", **w2.describe(),
                   "call_ms_avg": round(t2["kernel_ms_avg"], 4),
                   "call_ms_median": round(t2["kernel_ms_median"], 4),
                   "effective_tflops": round(a2, 2),
                   "pct_of_bf16_peak": round(100 * a2 / PEAK_BF16_TFLOPS, 2)}
            print(json.dumps(rec), file=sys.stderr, flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
