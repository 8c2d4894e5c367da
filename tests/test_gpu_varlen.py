"""GPU parity of packed variable-length sequences (sdpa_fwd_varlen / _f32out, through the C
ABI) against the fp64 packed-sequence oracle.

Bars as for the forward (max-abs <= 1e-2, mean-abs <= 1e-3 on the fp32 output and the LSE;
bf16 output = round-to-nearest-even of the fp32 output, bit for bit). Cases: ragged lengths
(0, 1, tile edges), queries shorter than keys per sequence, every mask, T5 bias, GQA, D = 64
and 128; the full-size pack checked on sampled sequences and heads. Packing equal-length
sequences must reproduce sdpa_fwd's batched result bit for bit (same kernel, only addressing
differs). Offsets that leave the packed buffers make their sequence empty (its rows untouched)
without disturbing the others.
"""
import numpy as np
import pytest

import oracle
import sdpa_inputs as si
from helpers import BF16_MAX_ABS, BF16_MEAN_ABS, errors, out_to_f64

pytestmark = pytest.mark.gpu

VL = si.VARLEN_WORKLOADS["vl"]


def dev(inp):
    import torch

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    t5 = None if inp.t5_table is None else torch.from_numpy(inp.t5_table).cuda()
    return (bf(inp.q), bf(inp.k), bf(inp.v), torch.from_numpy(inp.cu_q).cuda(),
            torch.from_numpy(inp.cu_k).cuda(), t5)


def run(sdpa, wl, inp, f32):
    import torch
    q, k, v, cq, ck, t5 = dev(inp)
    lq = np.diff(inp.cu_q)
    lk = np.diff(inp.cu_k)
    out, lse = sdpa.fwd_varlen(q, k, v, cq, ck, max(1, int(lq.max())), max(1, int(lk.max())),
                               scale=wl.scale, mask=wl.mask_kind, window=wl.window,
                               bias_kind=wl.bias_kind, bias=t5,
                               out_dtype=torch.float32 if f32 else torch.bfloat16)
    torch.cuda.synchronize()
    return out, lse


def check(sdpa, wl, inp, ref_o, ref_l, sel=None):
    import torch
    o32, l32 = run(sdpa, wl, inp, True)
    o16, l16 = run(sdpa, wl, inp, False)
    assert torch.equal(o16, o32.to(torch.bfloat16)), "bf16 out != RNE(fp32 out)"
    assert torch.equal(l16, l32)
    go, gl = out_to_f64(o32), out_to_f64(l32)
    if sel is not None:
        rows, heads = sel
        go = go[np.ix_(rows, heads)]
        gl = gl[np.ix_(heads, rows)]
    mo, ao = errors(go, ref_o)
    ml, al = errors(gl, ref_l)
    print(f"{wl.name}: O max {mo:.3e} mean {ao:.3e} | LSE max {ml:.3e} mean {al:.3e}",
          flush=True)
    assert mo <= BF16_MAX_ABS and ao <= BF16_MEAN_ABS, (mo, ao)
    assert ml <= BF16_MAX_ABS and al <= BF16_MEAN_ABS, (ml, al)


def small(name, lq, lk=None, **kw):
    kw.setdefault("Hq", 8)
    kw.setdefault("Hkv", 2)
    return (VL.replace(name=name, lengths_override=tuple(lq), **kw), lk)


SMALL = [
    small("vl_ragged_causal", [300, 1, 0, 256, 257, 700, 64]),
    small("vl_ragged_keys_longer", [100, 40, 300], [250, 40, 700]),
    small("vl_queries_longer_than_keys", [90, 300], [50, 120]),
    small("vl_none_mask", [200, 513, 3], mask_kind=si.MASK_NONE),
    small("vl_sliding_w100", [600, 333, 90], mask_kind=si.MASK_SLIDING, window=100),
    small("vl_t5_d64", [400, 129, 77], D=64, Hq=6, Hkv=3, mask_kind=si.MASK_NONE,
          bias_kind=si.BIAS_T5),
    small("vl_t5_causal_gqa", [350, 260], Hq=8, Hkv=2, bias_kind=si.BIAS_T5),
    small("vl_mqa_d128", [500, 31, 250], Hq=8, Hkv=1),
    small("vl_neg_scale", [260, 140], scale_override=-0.09),
    small("vl_alibi_causal", [400, 150, 300], bias_kind=si.BIAS_ALIBI),
    small("vl_t5u_d64", [300, 90], D=64, Hq=6, Hkv=3, bias_kind=si.BIAS_T5U),
    small("vl_d32_ragged_mqa", [300, 1, 129, 257], D=32, Hq=4, Hkv=1),
    small("vl_d256_sliding_t5", [260, 0, 190], [300, 20, 190], D=256, Hq=4, Hkv=2,
          mask_kind=si.MASK_SLIDING, window=70, bias_kind=si.BIAS_T5),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0].name for c in SMALL])
def test_varlen_parity_small(gpu_lib, case):
    wl, lk = case
    inp = si.make_varlen_inputs(wl, key_lengths=lk)
    q, k, v, t5 = inp.as_f64()
    ref_o, ref_l = oracle.sdpa_forward_varlen(q, k, v, inp.cu_q, inp.cu_k, scale=wl.scale,
                                              mask_kind=wl.mask_kind, window=wl.window,
                                              bias_kind=wl.bias_kind, bias=t5,
                                              threads=oracle.default_threads())
    check(gpu_lib, wl, inp, ref_o, ref_l)


def test_varlen_full_size_sampled(gpu_lib):
    inp = si.make_varlen_inputs(VL)
    q, k, v, _ = inp.as_f64()
    lens = np.diff(inp.cu_q)
    rng = np.random.default_rng(5)
    seqs = sorted({0, len(lens) - 1, int(np.argmax(lens)), int(rng.integers(len(lens)))})
    heads = [0, 13, VL.Hq - 1]
    rows = np.concatenate([np.arange(inp.cu_q[s], inp.cu_q[s + 1]) for s in seqs])
    sub_cu = np.concatenate([[0], np.cumsum([lens[s] for s in seqs])])
    qs = np.concatenate([q[inp.cu_q[s]:inp.cu_q[s + 1]] for s in seqs])
    ks = np.concatenate([k[inp.cu_k[s]:inp.cu_k[s + 1]] for s in seqs])
    vs = np.concatenate([v[inp.cu_k[s]:inp.cu_k[s + 1]] for s in seqs])
    ro, rl = oracle.sdpa_forward_varlen(qs, ks, vs, sub_cu, sub_cu, scale=VL.scale,
                                        mask_kind=VL.mask_kind, threads=oracle.default_threads())
    check(gpu_lib, VL, inp, ro[:, heads], rl[heads], sel=(rows, heads))


def test_equal_lengths_reproduce_batched_forward_bitwise(gpu_lib):
    import torch
    B, S, Hq, Hkv = 3, 700, 8, 2
    wl = si.WORKLOADS["c2"].replace(B=B, Hq=Hq, Hkv=Hkv, Sq=S, Sk=S, window=300)
    inp = si.make_inputs(wl)

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    q, k, v = bf(inp.q), bf(inp.k), bf(inp.v)
    o, l = gpu_lib.fwd(q, k, v, scale=wl.scale, mask="sliding", window=300)
    cu = torch.arange(0, (B + 1) * S, S, dtype=torch.int32, device="cuda")
    ov, lv = gpu_lib.fwd_varlen(q.reshape(B * S, Hq, 128), k.reshape(B * S, Hkv, 128),
                                v.reshape(B * S, Hkv, 128), cu, cu, S, S, scale=wl.scale,
                                mask="sliding", window=300)
    torch.cuda.synchronize()
    assert torch.equal(ov, o.reshape(B * S, Hq, 128))
    assert torch.equal(lv, l.permute(1, 0, 2).reshape(Hq, B * S))


def test_offsets_outside_the_buffers_leave_their_sequence_empty(gpu_lib):
    import torch
    wl = VL.replace(name="vl_bad_offsets", lengths_override=(200, 100, 150), Hq=4, Hkv=2)
    inp = si.make_varlen_inputs(wl)
    q, k, v, cq, ck, _ = dev(inp)
    # sequence 1 claims keys past the end of k/v and more than the stated maximum
    bad_k = torch.tensor([0, 200, 5000, 450], dtype=torch.int32, device="cuda")
    out = torch.full((450, 4, 128), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((4, 450), 7.0, dtype=torch.float32, device="cuda")
    gpu_lib.fwd_varlen(q, k, v, cq, bad_k, 200, 200, scale=wl.scale, mask="causal",
                       out=out, lse=lse, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(out[200:300] == 7.0) and torch.all(lse[:, 200:300] == 7.0)
    qf, kf, vf, _ = inp.as_f64()
    ro, rl = oracle.sdpa_forward_varlen(qf[:200], kf[:200], vf[:200], [0, 200], [0, 200],
                                        scale=wl.scale, mask_kind=si.MASK_CAUSAL)
    mo, _ = errors(out_to_f64(out)[:200], ro)
    assert mo <= BF16_MAX_ABS


def test_varlen_bitwise_determinism_100_runs(gpu_lib):
    import torch
    inp = si.make_varlen_inputs(VL)
    q, k, v, cq, ck, _ = dev(inp)
    m = int(np.diff(inp.cu_q).max())
    o0, l0 = gpu_lib.fwd_varlen(q, k, v, cq, ck, m, m)
    o0, l0 = o0.clone(), l0.clone()
    for _ in range(99):
        o, l = gpu_lib.fwd_varlen(q, k, v, cq, ck, m, m)
        assert torch.equal(o, o0) and torch.equal(l, l0)
    torch.cuda.synchronize()
