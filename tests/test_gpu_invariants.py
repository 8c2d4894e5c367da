"""GPU determinism and exact invariants of the kernel.

Determinism follows the protocol of the transformers issue "Transformer models are not
deterministic when using Flash Attention 2": repeat the same forward and compare with
torch.equal against the first run (here 100 runs, on both out and LSE).
"""
import numpy as np
import pytest

import sdpa_inputs as si
from helpers import out_to_f64, run_gpu, to_device

pytestmark = pytest.mark.gpu
W = si.WORKLOADS


@pytest.mark.parametrize("key", ["c1", "c2", "c3", "c3c", "c4t5", "c4full", "c5mha", "c5gqa",
                                 "c5mqa", "c2d32", "c2d256"])
def test_bitwise_determinism_100_runs(gpu_lib, key):
    """Every workload at full size, in the launch the benchmark times (c1 runs the fp32
    entry point, the others the bf16 one)."""
    import torch
    wl = W[key]
    inp = si.make_inputs(wl)
    dev = to_device(inp)
    o0, l0 = run_gpu(gpu_lib, wl, dev)
    o0, l0 = o0.clone(), l0.clone()
    same = True
    for _ in range(99):
        o, l = run_gpu(gpu_lib, wl, dev)
        same = same and torch.equal(o, o0) and torch.equal(l, l0)
    assert same
    words = o0.view(torch.int32) if o0.dtype == torch.float32 else o0.view(torch.int16)
    h = int(torch.sum(words.to(torch.int64) * 1000003 % 65521).item())
    print(f"{key}: deterministic over 100 runs, out checksum {h}")


def _sk(wl, **kw):
    return si.small(wl, **kw)


def test_sliding_window_ge_seqlen_is_causal_bitwise(gpu_lib):
    """Window >= seqlen must give exactly the plain causal result (transformers issue on the
    SDPA mask fix: at seqlen == window the result must be that of the causal kernel)."""
    import torch
    for S, w in [(4096, 4096), (700, 700), (700, 5000), (513, 514)]:
        wl = si.small(W["c2"], B=1, Hq=8, Hkv=2, Sq=S, Sk=S, window=w, name_suffix=f"{S}_{w}")
        dev = to_device(si.make_inputs(wl))
        o_s, l_s = run_gpu(gpu_lib, wl, dev)
        o_c, l_c = run_gpu(gpu_lib, wl.replace(mask_kind=si.MASK_CAUSAL), dev)
        assert torch.equal(o_s, o_c) and torch.equal(l_s, l_c), (S, w)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_causal_row0_is_v0_bitwise(gpu_lib, D):
    import torch
    wl = si.small(W["c5gqa"], B=2, Hq=8, Hkv=2, Sq=300, Sk=300, name_suffix="row0").replace(D=D)
    inp = si.make_inputs(wl)
    dev = to_device(inp)
    o, _ = run_gpu(gpu_lib, wl, dev)
    v = dev[2]
    G = wl.Hq // wl.Hkv
    assert torch.equal(o[:, 0], v[:, 0].repeat_interleave(G, dim=1))


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_window1_is_v_bitwise(gpu_lib, D):
    import torch
    wl = si.small(W["c2"], B=1, Hq=4, Hkv=2, Sq=200, Sk=200, window=1, name_suffix="w1").replace(D=D)
    dev = to_device(si.make_inputs(wl))
    o, _ = run_gpu(gpu_lib, wl, dev)
    assert torch.equal(o, dev[2].repeat_interleave(2, dim=2))


@pytest.mark.parametrize("key,D", [("c4t5", 64), ("c2", 128), ("c2d256", 256), ("c2d32", 32)])
def test_ones_value_gives_ones(gpu_lib, key, D):
    import torch
    wl = si.small(W[key], B=1, Hq=2, Hkv=2, Sq=300, Sk=300, name_suffix="v1").replace(D=D)
    q, k, v, bias = to_device(si.make_inputs(wl))
    v = torch.ones_like(v)
    o, _ = run_gpu(gpu_lib, wl, (q, k, v, bias), out_f32=True)
    o16, _ = run_gpu(gpu_lib, wl, (q, k, v, bias), out_f32=False)
    # numerator (P.V) and normaliser both add the same bf16 weights p_hat, in fp32 and in
    # different orders: O = 1 up to the rounding of two sums of <= 300 terms (< 3e-5), and the
    # bf16 output is exactly 1
    assert torch.max(torch.abs(o - 1.0)).item() <= 3e-5
    assert torch.equal(o16, torch.ones_like(o16))


def test_gqa_equals_mha_on_repeated_kv_bitwise(gpu_lib):
    """Head sharing: each query head h reads KV head h // G; giving every query head its own
    copy of that KV head (MHA on repeat_interleave'd K/V) must not change a bit."""
    import torch
    for key, Hq, Hkv in (("c5gqa", 8, 2), ("c5mqa", 8, 1), ("c4t5", 6, 2)):
        wl = si.small(W[key], B=2, Hq=Hq, Hkv=Hkv, Sq=333, Sk=333, name_suffix="rep")
        q, k, v, bias = to_device(si.make_inputs(wl))
        G = Hq // Hkv
        kr = k.repeat_interleave(G, dim=2).contiguous()
        vr = v.repeat_interleave(G, dim=2).contiguous()
        o1, l1 = run_gpu(gpu_lib, wl, (q, k, v, bias))
        o2, l2 = run_gpu(gpu_lib, wl.replace(Hkv=Hq), (q, kr, vr, bias))
        assert torch.equal(o1, o2) and torch.equal(l1, l2), key


def test_zero_query_gives_visible_mean(gpu_lib):
    import torch
    wl = si.small(W["c3"], B=1, Hq=2, Hkv=1, Sq=400, Sk=400, window=37, name_suffix="q0")
    q, k, v, bias = to_device(si.make_inputs(wl))
    q = torch.zeros_like(q)
    o, l = run_gpu(gpu_lib, wl, (q, k, v, bias), out_f32=True)
    vv = v.float()[0, :, 0]                        # [S, D]
    cs = torch.cat([torch.zeros_like(vv[:1]), torch.cumsum(vv.double(), 0)])
    for i in [0, 1, 36, 37, 38, 399]:
        lo = max(0, i - 37 + 1)
        mean = (cs[i + 1] - cs[lo]) / (i + 1 - lo)
        assert torch.max(torch.abs(o[0, i, 0].double() - mean)).item() <= 2e-3
        assert abs(l[0, 0, i].item() - np.log(i + 1 - lo)) <= 1e-5


def test_causal_last_row_equals_unmasked_last_row(gpu_lib):
    """Codelab section 7: the last position attends to every position either way."""
    wl = si.small(W["c5gqa"], B=1, Hq=4, Hkv=2, Sq=257, Sk=257, name_suffix="last")
    dev = to_device(si.make_inputs(wl))
    oc, _ = run_gpu(gpu_lib, wl, dev, out_f32=True)
    on, _ = run_gpu(gpu_lib, wl.replace(mask_kind=si.MASK_NONE), dev, out_f32=True)
    a, c = out_to_f64(oc), out_to_f64(on)
    assert np.max(np.abs(a[:, -1] - c[:, -1])) <= 1e-5
    assert np.max(np.abs(a[:, 0] - c[:, 0])) > 1e-2


_FRESH = r"""
import hashlib, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import torch
import sdpa_inputs as si
import scaled_dot_product_03_amd as sdpa
from helpers import run_gpu, to_device
wl = si.small(si.WORKLOADS["c2"], B=1, Hq=8, Hkv=2, Sq=1000, Sk=1000, window=1000,
              name_suffix="fresh")
o, l = run_gpu(sdpa, wl, to_device(si.make_inputs(wl)))
h = hashlib.sha256(o.view(torch.int16).cpu().numpy().tobytes() +
                   l.cpu().numpy().tobytes()).hexdigest()
print("HASH", h)
"""


def test_bitwise_same_in_a_fresh_process(gpu_lib):
    """The determinism issue compares runs of a training step; besides repeats within one
    process, a second process must produce the same bits (same shape, same launch)."""
    import hashlib
    import os
    import subprocess
    import sys
    import torch
    wl = si.small(W["c2"], B=1, Hq=8, Hkv=2, Sq=1000, Sk=1000, window=1000, name_suffix="fresh")
    o, l = run_gpu(gpu_lib, wl, to_device(si.make_inputs(wl)))
    here = hashlib.sha256(o.view(torch.int16).cpu().numpy().tobytes() +
                          l.cpu().numpy().tobytes()).hexdigest()
    tests = os.path.dirname(os.path.abspath(__file__))
    code = _FRESH.format(root=os.path.dirname(tests), tests=tests)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=180)
    assert r.returncode == 0, r.stderr[-2000:]
    there = [x.split()[1] for x in r.stdout.splitlines() if x.startswith("HASH ")][0]
    print(f"in-process {here[:16]} fresh process {there[:16]}")
    assert here == there


_PERSIST_CASES = {
    "c2": (W["c2"], 2), "c3": (W["c3"], 2), "c4t5": (W["c4t5"], 12), "c5mha": (W["c5mha"], 8),
    "c5mqa": (W["c5mqa"], 1), "c2alibi": (W["c2alibi"], 2), "c4t5u": (W["c4t5u"], 12),
    # ragged query tiles (Sq = 1000: 4 tiles, the last one 232 rows), 512 items
    "ragged": (si.small(W["c5gqa"], B=8, Hq=16, Hkv=8, Sq=1000, Sk=1000, name_suffix="pragged"), 2),
    # keys longer than queries (off = 800) under a sliding window, 768 items
    "prefix_sliding": (si.small(W["c3"], B=16, Hq=16, Hkv=8, Sq=700, Sk=1500, window=600,
                                name_suffix="pprefix"), 2),
    # D = 64 without a bias, causal
    "d64": (si.small(W["c5gqa"], B=8, Hq=16, Hkv=8, Sq=1024, Sk=1024,
                     name_suffix="pd64").replace(D=64), 2),
    # fewer keys than queries under a causal mask (off = -724): the first two query tiles of
    # every (batch, head) see no key and end early inside the work loop
    "empty_items": (si.small(W["c5gqa"], B=8, Hq=16, Hkv=8, Sq=1024, Sk=300,
                             name_suffix="pempty"), 2),
    # a negative softmax scale (the Q fragment's sign is flipped per item)
    "neg_scale": (si.small(W["c5gqa"], B=8, Hq=16, Hkv=8, Sq=1024, Sk=1024,
                           name_suffix="pneg").replace(scale_override=-0.0625), 2),
}


def _launch_grid(sdpa, wl):
    return sdpa.fwd_launch_grid(wl.B, wl.Hq, wl.Hkv, wl.Sq, wl.Sk, wl.D, mask=wl.mask_kind,
                                window=wl.window, bias_kind=wl.bias_kind)


def _persistent_grid():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count // 8 * 8


@pytest.mark.parametrize("case", sorted(_PERSIST_CASES))
def test_persistent_grid_equals_small_launches_bitwise(gpu_lib, case):
    """At these sizes a launch walks its work items on a persistent grid (one workgroup per
    CU, a fixed order of items per workgroup). The same inputs cut into launches of one batch
    and `split_kv` KV heads (with their query heads) are small enough for one workgroup per
    item. Every item is computed by the same code, so out and LSE must agree bit for bit."""
    import torch
    wl, split_kv = _PERSIST_CASES[case]
    tiles = -(-wl.Sq // (256 if wl.D in (64, 128) else 128))
    G = wl.Hq // wl.Hkv
    sub = wl.replace(B=1, Hq=split_kv * G, Hkv=split_kv)
    assert _launch_grid(gpu_lib, wl) == _persistent_grid()          # a persistent launch
    assert _launch_grid(gpu_lib, sub) == split_kv * G * tiles       # one workgroup per item
    inp = si.make_inputs(wl)
    q, k, v, bias = to_device(inp)
    o_all, l_all = run_gpu(gpu_lib, wl, (q, k, v, bias))
    same = True
    for b in range(wl.B):
        for h0 in range(0, wl.Hkv, split_kv):
            qs = q[b:b + 1, :, h0 * G:(h0 + split_kv) * G].contiguous()
            ks = k[b:b + 1, :, h0:h0 + split_kv].contiguous()
            vs = v[b:b + 1, :, h0:h0 + split_kv].contiguous()
            bs = bias[h0 * G:(h0 + split_kv) * G].contiguous() if bias is not None else None
            o, l = run_gpu(gpu_lib, sub, (qs, ks, vs, bs))
            same = same and torch.equal(o[0], o_all[b, :, h0 * G:(h0 + split_kv) * G])
            same = same and torch.equal(l[0], l_all[b, h0 * G:(h0 + split_kv) * G])
    assert same


def _random_persistent_case(seed: int):
    """A seeded random launch that takes the persistent grid: B * Hkv a multiple of 8 and at
    least 512 work items, random head dim, mask, window, bias kind, ragged lengths and a key
    prefix of either sign."""
    rng = np.random.default_rng(seed)
    D = int(rng.choice([64, 128]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    Sq = int(rng.integers(300, 2500))
    Sk = max(1, Sq + int(rng.integers(-200, 800)))
    mask = int(rng.choice([si.MASK_NONE, si.MASK_CAUSAL, si.MASK_SLIDING]))
    window = int(rng.integers(1, Sk + 300)) if mask == si.MASK_SLIDING else 0
    bias = int(rng.choice([si.BIAS_NONE, si.BIAS_ALIBI] + ([si.BIAS_T5, si.BIAS_T5U] if D == 64 else [])))
    tiles = -(-Sq // 256)
    B = 8 // Hkv
    while B * G * Hkv * tiles < 512:
        B += 8 // Hkv
    return W["c5gqa"].replace(name=f"persist_random_{seed}", B=B, Hq=G * Hkv, Hkv=Hkv, Sq=Sq,
                              Sk=Sk, D=D, mask_kind=mask, window=window, bias_kind=bias,
                              seed=9000 + seed % 1000)


@pytest.mark.parametrize("seed", range(20261204, 20261216))
def test_persistent_grid_random_shapes_bitwise(gpu_lib, seed):
    """Random persistent launches against one launch per batch (one workgroup per item, or a
    persistent grid over far fewer items): out and LSE agree bit for bit."""
    import torch
    wl = _random_persistent_case(seed)
    assert _launch_grid(gpu_lib, wl) == _persistent_grid()
    q, k, v, bias = to_device(si.make_inputs(wl))
    o_all, l_all = run_gpu(gpu_lib, wl, (q, k, v, bias))
    sub = wl.replace(B=1)
    same = True
    for b in range(wl.B):
        o, l = run_gpu(gpu_lib, sub, (q[b:b + 1].contiguous(), k[b:b + 1].contiguous(),
                                      v[b:b + 1].contiguous(), bias))
        same = same and torch.equal(o[0], o_all[b]) and torch.equal(l[0], l_all[b])
    assert same, wl
