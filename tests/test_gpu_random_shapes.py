"""Seeded random configurations: the forward (dense and packed), gradient and decode entry
points against the fp64 oracles, at the bars of the fixed-case tests (bf16: max-abs <= 1e-2 and mean-abs <= 1e-3 on the
fp32 epilogue, whose bf16 rounding must equal the bf16 entry point bit for bit; gradients:
element-wise first-order bounds and rms <= 2^-8 of the reference rms).

One seed draws every case: head dim, head sharing (MHA / GQA / MQA), batch, query and key
lengths (ragged tails, Sq below and above Sk, single rows and keys), mask and window, bias
kind and the sign of the softmax scale. The draw is fixed, so each case is a deterministic
regression test; together they cover combinations the hand-picked cases do not list.
"""
import numpy as np
import pytest

import oracle
import sdpa_inputs as si
from helpers import oracle_full, to_device
from test_gpu_bwd import check_pairs
from test_gpu_decode import check as check_decode
from test_gpu_parity import _check_bf16
from test_gpu_varlen import check as check_varlen

pytestmark = pytest.mark.gpu

BASE = si.WORKLOADS["c2c"]


def draw(n, seed, decode=False):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(rng.choice([32, 64, 128, 256]))
        Hkv = int(rng.choice([1, 2, 3]))
        G = int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 3))
        if decode:
            Sq, Sk = int(rng.integers(1, 9)), int(rng.integers(200, 5000))
        else:
            u = rng.random()
            Sq = 1 if u < 0.1 else int(rng.integers(2, 64)) if u < 0.4 else int(rng.integers(64, 420))
            Sk = Sq if rng.random() < 0.5 else int(rng.integers(1, 420))
        mask = int(rng.integers(0, 3))
        window = int(rng.integers(1, 2 * max(Sk, 2))) if mask == si.MASK_SLIDING else 0
        bias = int(rng.integers(0, 5))
        scale = None
        u = rng.random()
        if u < 0.15:
            scale = -float(rng.uniform(0.02, 0.2))
        elif u < 0.2:
            scale = 0.0
        name = (f"rand{i}_d{D}_b{B}_h{Hkv * G}x{Hkv}_q{Sq}_k{Sk}_m{mask}"
                f"{'w' + str(window) if mask == si.MASK_SLIDING else ''}_bias{bias}"
                f"{'' if scale is None else '_s' + format(scale, '.3f')}")
        cases.append(BASE.replace(name=name, B=B, Hq=Hkv * G, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D,
                                  mask_kind=mask, window=window, bias_kind=bias,
                                  seed=9000 + 10 * i + (500 if decode else 0), kv_seed=None,
                                  scale_override=scale))
    return cases


def draw_packs(n, seed):
    """Packed sequences: 1-6 sequences of ragged lengths (some empty), key lengths equal to or
    different from the query lengths, and the forward's masks and index-generated biases."""
    rng = np.random.default_rng(seed)
    base = si.VARLEN_WORKLOADS["vl"]
    cases = []
    for i in range(n):
        ns = int(rng.integers(1, 7))
        lq = [int(x) for x in rng.integers(0, 300, ns)]
        lq[int(rng.integers(ns))] = max(lq[0], 1)          # at least one query token
        lk = lq if rng.random() < 0.5 else [int(x) for x in rng.integers(1, 400, ns)]
        D = int(rng.choice([32, 64, 128, 256]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 4]))
        mask = int(rng.integers(0, 3))
        window = int(rng.integers(1, 300)) if mask == si.MASK_SLIDING else 0
        bias = int(rng.choice([0, 1, 3, 4]))                 # no full bias for packed sequences
        name = f"pack{i}_d{D}_h{Hkv * G}x{Hkv}_n{ns}_m{mask}_bias{bias}"
        wl = base.replace(name=name, lengths_override=tuple(lq), D=D, Hq=Hkv * G, Hkv=Hkv,
                          mask_kind=mask, window=window, bias_kind=bias, seed=9700 + 10 * i)
        cases.append((wl, None if lk is lq else lk))
    return cases


FWD = draw(24, 2024)
PACK = draw_packs(10, 2027)
BWD = draw(12, 2025)
DEC = [w for w in draw(14, 2026, decode=True) if w.bias_kind != si.BIAS_FULL or w.Sq * w.Sk < 4e4]


@pytest.mark.parametrize("wl", FWD, ids=[w.name for w in FWD])
def test_random_forward(gpu_lib, wl):
    inp = si.make_inputs(wl)
    ref_o, ref_l = oracle_full(inp)
    _check_bf16(gpu_lib, wl, inp, to_device(inp), ref_o, ref_l)


@pytest.mark.parametrize("wl", BWD, ids=[w.name for w in BWD])
def test_random_gradients(gpu_lib, wl):
    check_pairs(gpu_lib, wl, [(b, h) for b in range(wl.B) for h in range(wl.Hkv)])


@pytest.mark.parametrize("wl", DEC, ids=[w.name for w in DEC])
def test_random_decode(gpu_lib, wl):
    inp = si.make_inputs(wl)
    ref_o, ref_l = oracle_full(inp)
    check_decode(gpu_lib, wl, ref_o, ref_l)


@pytest.mark.parametrize("case", PACK, ids=[c[0].name for c in PACK])
def test_random_packed(gpu_lib, case):
    wl, lk = case
    inp = si.make_varlen_inputs(wl, key_lengths=lk)
    q, k, v, t5 = inp.as_f64()
    ref_o, ref_l = oracle.sdpa_forward_varlen(q, k, v, inp.cu_q, inp.cu_k, scale=wl.scale,
                                              mask_kind=wl.mask_kind, window=wl.window,
                                              bias_kind=wl.bias_kind, bias=t5,
                                              threads=oracle.default_threads())
    check_varlen(gpu_lib, wl, inp, ref_o, ref_l)
