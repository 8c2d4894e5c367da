"""Work accounting and run contract of bench.py (CPU): the tile-granular FLOP count against
closed forms, and the exits that keep every timed number on one GPU.

The count is the matrix work the bf16 kernel performs (32-row x 64-key blocks, masked slots
included); the profile summary checks it against the MFMA instruction counter.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import sdpa_inputs as si  # noqa: E402

BLOCK = 32 * 64


def blocks(wl):
    return bench.tile_flops(wl) / (4.0 * wl.D * BLOCK * wl.B * wl.Hq)


def test_unmasked_is_dense_rounded_to_tiles():
    wl = si.WORKLOADS["c4t5"]
    assert blocks(wl) == (wl.Sq // 32) * (wl.Sk // 64)
    ragged = wl.replace(Sq=100, Sk=130, B=1, Hq=1, Hkv=1)
    assert blocks(ragged) == 4 * 3          # ceil(100/32) waves x ceil(130/64) tiles


def test_causal_closed_form():
    # rows 32w..32w+31 need key tiles 0 .. floor((32w+31)/64): w = 2k and 2k+1 both need k+1
    for S in (256, 4096, 8192):
        wl = si.WORKLOADS["c2c"].replace(Sq=S, Sk=S, B=1, Hq=1, Hkv=1)
        n = S // 64
        assert blocks(wl) == 2 * n * (n + 1) // 2


def test_window_equal_to_seqlen_is_causal():
    assert bench.tile_flops(si.WORKLOADS["c2"]) == bench.tile_flops(si.WORKLOADS["c2c"])


def test_tile_count_bounds_effective_work():
    for key in ("c2", "c3", "c3c", "c4t5", "c5mqa"):
        wl = si.WORKLOADS[key]
        assert si.effective_flops(wl) <= bench.tile_flops(wl) <= 1.05 * si.effective_flops(wl)


@pytest.mark.parametrize("mask,w,sq,sk", [
    (si.MASK_SLIDING, 1, 300, 333), (si.MASK_SLIDING, 63, 300, 333),
    (si.MASK_SLIDING, 64, 300, 333), (si.MASK_SLIDING, 65, 257, 257),
    (si.MASK_SLIDING, 200, 300, 333), (si.MASK_CAUSAL, 0, 300, 333), (si.MASK_CAUSAL, 0, 70, 500)])
def test_blocks_are_exactly_those_with_a_visible_pair(mask, w, sq, sk):
    # brute force: with Sq <= Sk the kernel computes a 32-row x 64-key block iff some row of
    # it sees some key of it
    wl = si.WORKLOADS["c3"].replace(Sq=sq, Sk=sk, B=1, Hq=1, Hkv=1, window=w, mask_kind=mask)
    off = wl.Sk - wl.Sq
    need = set()
    for i in range(wl.Sq):
        p = i + off
        lo = 0 if mask == si.MASK_CAUSAL else max(0, p - w + 1)
        for j in range(lo, min(p, wl.Sk - 1) + 1):
            need.add((i // 32, j // 64))
    assert blocks(wl) == len(need)


# ------------------------------------------------------------------------------------------
# gradient kernels: MFMA instructions of the tile plans (bench.bwd_tile_mfmas)
# ------------------------------------------------------------------------------------------
def _kv_per_block(D, bias_kind):
    # MFMAs of one 32-row x 32-key block in the dk/dv kernel: the dV wave forms S (D/16) and
    # dV (2 D/32); the dK wave forms dP (D/16) and dK (2 D/32), plus S itself (D/16) where P is
    # not handed over (a full bias at head dims other than 64)
    handoff = bias_kind != si.BIAS_FULL or D == 64
    return (D // 16 + 2 * (D // 32)) + ((1 if handoff else 2) * (D // 16) + 2 * (D // 32))


def test_bwd_unmasked_closed_form():
    for D in (64, 128):
        wl = si.WORKLOADS["c4t5"].replace(B=2, Hq=4, Hkv=2, Sq=512, Sk=768, D=D,
                                          bias_kind=si.BIAS_NONE)
        dq, dkdv = bench.bwd_tile_mfmas(wl)
        G = wl.Hq // wl.Hkv
        per_half = 2 * (D // 16) + 2 * (D // 32)
        assert dq == wl.B * wl.Hq * (wl.Sq // 32) * (wl.Sk // 64) * 2 * per_half
        assert dkdv == wl.B * wl.Hkv * (wl.Sk // 32) * (wl.Sq // 32) * G * _kv_per_block(D, wl.bias_kind)


@pytest.mark.parametrize("mask,w,sq,sk,bias", [
    (si.MASK_CAUSAL, 0, 512, 512, si.BIAS_NONE), (si.MASK_CAUSAL, 0, 256, 640, si.BIAS_NONE),
    (si.MASK_SLIDING, 100, 512, 512, si.BIAS_NONE), (si.MASK_SLIDING, 1, 384, 384, si.BIAS_NONE),
    (si.MASK_SLIDING, 300, 448, 576, si.BIAS_FULL), (si.MASK_CAUSAL, 0, 640, 384, si.BIAS_FULL)])
def test_bwd_blocks_are_exactly_those_with_a_visible_pair(mask, w, sq, sk, bias):
    # brute force over the visibility of every (row, key): with Sq, Sk multiples of 64, the dq
    # kernel computes a 32-row x 64-key block and the dk/dv kernel a 32-row x 32-key block iff
    # some row of it sees some key of it
    wl = si.WORKLOADS["c3"].replace(Sq=sq, Sk=sk, B=1, Hq=2, Hkv=1, window=w, mask_kind=mask,
                                    bias_kind=bias)
    off = wl.Sk - wl.Sq
    dq_blocks, kv_blocks = set(), set()
    for i in range(wl.Sq):
        p = i + off
        for j in range(wl.Sk):
            vis = j <= p if mask != si.MASK_NONE else True
            if mask == si.MASK_SLIDING:
                vis = vis and p - j < w
            if vis:
                dq_blocks.add((i // 32, j // 64))
                kv_blocks.add((i // 32, j // 32))
    D, G = wl.D, 2
    dq, dkdv = bench.bwd_tile_mfmas(wl)
    assert dq == len(dq_blocks) * 2 * (2 * (D // 16) + 2 * (D // 32)) * wl.Hq
    assert dkdv == len(kv_blocks) * _kv_per_block(D, bias) * G


def test_more_than_one_gpu_is_refused_with_a_message(capsys):
    """One GPU only: --gpus N above 1 exits (status 2) and says why, before touching a GPU."""
    assert bench.main(["--gpus", "2"]) == 2
    assert "exactly one GPU" in capsys.readouterr().err


def test_no_gpu_exits_instead_of_falling_back(capsys):
    """Without a visible GPU the benchmark stops (status 1); it never times a CPU path."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert bench.main(["--no-cpu-baseline", "--no-sweep"]) == 1
    assert "no GPU" in capsys.readouterr().err


def _profile_sources(name):
    if name.startswith("sdpa_bwd"):
        return bench.KERNEL_SOURCES_BWD
    if name.startswith("sdpa_decode"):
        return bench.KERNEL_SOURCES_DEC
    return bench.KERNEL_SOURCES


def test_profiles_describe_the_committed_kernels():
    """Every profile summary states the hash of the kernel sources it was taken on; it must be
    the hash of the sources in the tree (a kernel change calls for new profiles), and the
    traffic records the bench line reads must carry the same hash."""
    import json
    import re
    pdir = os.path.join(ROOT, "profiles")
    names = sorted(os.listdir(pdir))
    assert names, "no profiles"
    for name in names:
        path = os.path.join(pdir, name)
        want = bench.kernel_sha(_profile_sources(name))
        if name.endswith(".json"):
            with open(path) as f:
                assert json.load(f)["kernel_sha"] == want, name
        else:
            with open(path) as f:
                m = re.search(r"sha[^:]*\):\s*([0-9a-f]{16})", f.read())
            assert m, f"{name}: no kernel source hash"
            assert m.group(1) == want, name


def test_headline_line_carries_measured_traffic():
    """With the profiles matching the sources, the bench line's roofline entry carries the HBM
    bytes measured by the byte counters (forward, gradients and decode headline workloads)."""
    assert bench.load_traffic(si.WORKLOADS["c2"].name) is not None
    assert bench.load_traffic(si.WORKLOADS["c2"].name, bwd=True) is not None
    dec = [f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.startswith("sdpa_decode")
           and f.endswith(".json")]
    assert dec
