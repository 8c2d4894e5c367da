"""C-ABI checks that need no GPU: the library loads, exports every symbol include/sdpa.h
declares, and every invalid call returns its status before any HIP call (so these calls are
safe on a machine without a GPU: validation fails first and nothing is launched)."""
import ctypes
import math
import os
import re

import pytest

import scaled_dot_product_03_amd as sdpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sdpa.lib_path()):
        from scaled_dot_product_03_amd import build
        build.build()
    return sdpa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sdpa_\w+)\s*\(", text, flags=re.M)


def test_header_declares_entry_points():
    names = declared_functions()
    assert sorted(names) == sorted(sdpa.ENTRY_POINTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.sdpa_abi_version() == sdpa.ABI_VERSION == 4
    for code in range(0, 13):
        s = sdpa.status_str(code)
        assert s and s != "unknown status"
    assert sdpa.status_str(999) == "unknown status"


# fake, aligned, never-dereferenced device addresses
P = 0x10000
GOOD = dict(q=P, k=P, v=P, out=P, lse=P, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, D=64, scale=0.125,
            mask_kind=1, window=0, bias_kind=0, bias=None, stream=None)


def call(entry="sdpa_fwd", **kw):
    a = dict(GOOD)
    a.update(kw)
    return sdpa.call_raw(entry, a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"],
                         a["Hkv"], a["Sq"], a["Sk"], a["D"], a["scale"], a["mask_kind"],
                         a["window"], a["bias_kind"], a["bias"], a["stream"])


BAD_CASES = [
    ("null q", dict(q=None), 1),
    ("null lse", dict(lse=None), 1),
    ("B=0", dict(B=0), 2),
    ("Sk=0", dict(Sk=0), 2),
    ("Hkv=0", dict(Hkv=0), 2),
    ("Hq % Hkv", dict(Hq=6, Hkv=4), 3),
    ("D=96", dict(D=96), 4),
    ("D=512", dict(D=512), 4),
    ("D=16", dict(D=16), 4),
    ("mask 3", dict(mask_kind=3), 5),
    ("mask -1", dict(mask_kind=-1), 5),
    ("sliding window 0", dict(mask_kind=2, window=0), 6),
    ("sliding window -5", dict(mask_kind=2, window=-5), 6),
    ("bias kind 5", dict(bias_kind=5, bias=P), 7),
    ("bias kind -1", dict(bias_kind=-1, bias=P), 7),
    ("alibi without table", dict(bias_kind=3, bias=None), 7),
    ("t5u without table", dict(bias_kind=4, bias=None), 7),
    ("misaligned alibi table", dict(bias_kind=3, bias=P + 2), 9),
    ("t5 without table", dict(bias_kind=1, bias=None), 7),
    ("full without tensor", dict(bias_kind=2, bias=None), 7),
    ("no bias but pointer", dict(bias_kind=0, bias=P), 7),
    ("scale nan", dict(scale=math.nan), 8),
    ("scale inf", dict(scale=math.inf), 8),
    ("misaligned q", dict(q=P + 8), 9),
    ("misaligned out", dict(out=P + 2), 9),
    ("misaligned lse", dict(lse=P + 2), 9),
    ("misaligned full bias", dict(bias_kind=2, bias=P + 4), 9),
    ("huge q", dict(B=1 << 16, Sq=1 << 16, Hq=1 << 8, Hkv=1 << 8, D=128), 2),
]


@pytest.mark.parametrize("entry", ["sdpa_fwd", "sdpa_fwd_bf16_f32out", "sdpa_fwd_f32"])
@pytest.mark.parametrize("name,kw,code", BAD_CASES, ids=[c[0] for c in BAD_CASES])
def test_invalid_arguments_return_status(lib, entry, name, kw, code):
    assert call(entry, **kw) == code


def test_first_failing_check_wins(lib):
    # null pointer is checked before shapes, shapes before heads, heads before head dim
    assert call(q=None, B=0) == 1
    assert call(B=0, Hq=6, Hkv=4) == 2
    assert call(Hq=6, Hkv=4, D=96) == 3
    assert call(D=96, mask_kind=9) == 4


def _grid(lib, **kw):
    a = dict(GOOD)
    a.update(kw)
    wg = ctypes.c_longlong(-1)
    st = lib.sdpa_fwd_launch_grid(a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["D"],
                                  a["mask_kind"], a["window"], a["bias_kind"], ctypes.byref(wg))
    return st, wg.value


# the query takes no buffers: the cases about shapes, mask, window and an unknown bias kind
_SHAPE_KEYS = {"B", "Hq", "Hkv", "Sq", "Sk", "D", "mask_kind", "window"}
GRID_BAD = [c for c in BAD_CASES
            if set(c[1]) <= _SHAPE_KEYS or c[1].get("bias_kind", 0) not in range(5)]


@pytest.mark.parametrize("name,kw,code", GRID_BAD, ids=[c[0] for c in GRID_BAD])
def test_launch_grid_query_rejects_what_the_forward_rejects(lib, name, kw, code):
    assert call(**kw) == code
    assert _grid(lib, **kw) == (code, -1)


def test_launch_grid_query_null_out_pointer(lib):
    assert lib.sdpa_fwd_launch_grid(1, 4, 2, 8, 8, 64, 1, 0, 0, None) == 1


@pytest.mark.parametrize("kw,tiles", [
    # shapes that never take the persistent grid, so no device is asked for its CU count
    (dict(B=2, Hq=8, Hkv=8, Sq=1000, D=256), 2 * 8 * 8),             # 128 query rows a tile
    (dict(B=3, Hq=4, Hkv=4, Sq=129, D=32), 3 * 4 * 2),
    (dict(B=1, Hq=4, Hkv=2, Sq=8, D=64), 4),                          # 256 rows a tile
    (dict(B=1, Hq=6, Hkv=2, Sq=4097, D=128, bias_kind=1, bias=P), 6 * 17),   # T5 at D = 128
    (dict(B=8, Hq=8, Hkv=8, Sq=4096, D=64, bias_kind=2, bias=P), 8 * 8 * 32),  # full bias: 128 rows
])
def test_launch_grid_query_one_workgroup_per_tile(lib, kw, tiles):
    assert _grid(lib, **kw) == (0, tiles)
    assert sdpa.fwd_launch_grid(kw["B"], kw["Hq"], kw["Hkv"], kw["Sq"], 8, kw["D"],
                                bias_kind=kw.get("bias_kind", 0)) == tiles


def test_binding_rejects_before_launch(lib):
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sdpa.fwd(q, q, q)            # cpu tensors are refused by the binding


# backward: same validation as the forward, plus its own pointers
GOOD_BWD = dict(GOOD, dout=P, dq=P, dk=P, dv=P, ws=P)


def call_bwd(entry="sdpa_bwd", **kw):
    a = dict(GOOD_BWD)
    a.update(kw)
    return sdpa.call_raw_bwd(entry, a["q"], a["k"], a["v"], a["out"], a["lse"], a["dout"],
                             a["dq"], a["dk"], a["dv"], a["ws"], a["B"], a["Hq"], a["Hkv"],
                             a["Sq"], a["Sk"], a["D"], a["scale"], a["mask_kind"], a["window"],
                             a["bias_kind"], a["bias"], a["stream"])


BWD_CASES = BAD_CASES + [
    ("null dout", dict(dout=None), 1),
    ("null dq", dict(dq=None), 1),
    ("null dk", dict(dk=None), 1),
    ("null dv", dict(dv=None), 1),
    ("null ws", dict(ws=None), 1),
    ("misaligned dout", dict(dout=P + 2), 9),
    ("misaligned dq", dict(dq=P + 8), 9),
    ("misaligned dk", dict(dk=P + 4), 9),
    ("misaligned dv", dict(dv=P + 2), 9),
    ("misaligned ws", dict(ws=P + 2), 9),
]


@pytest.mark.parametrize("entry", ["sdpa_bwd", "sdpa_bwd_f32out"])
@pytest.mark.parametrize("name,kw,code", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_backward_invalid_arguments_return_status(lib, entry, name, kw, code):
    assert call_bwd(entry, **kw) == code


def test_backward_binding_rejects_before_launch(lib):
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        sdpa.bwd(q, q, q, q, lse, q)  # cpu tensors are refused by the binding


# decode: the forward's validation, plus the workspace
def call_dec(entry="sdpa_decode", **kw):
    a = dict(GOOD, ws=P, ws_bytes=1 << 40)
    a.update(kw)
    return sdpa.call_raw_decode(entry, a["q"], a["k"], a["v"], a["out"], a["lse"], a["ws"],
                                a["ws_bytes"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"],
                                a["D"], a["scale"], a["mask_kind"], a["window"],
                                a["bias_kind"], a["bias"], a["stream"])


DEC_CASES = BAD_CASES + [
    ("null ws", dict(ws=None), 11),
    ("misaligned ws", dict(ws=P + 8), 11),
    ("small ws", dict(ws_bytes=16), 11),
]


@pytest.mark.parametrize("entry", ["sdpa_decode", "sdpa_decode_f32out"])
@pytest.mark.parametrize("name,kw,code", DEC_CASES, ids=[c[0] for c in DEC_CASES])
def test_decode_invalid_arguments_return_status(lib, entry, name, kw, code):
    assert call_dec(entry, **kw) == code


def test_decode_workspace_size(lib):
    # 32 fp32 rows of (D + 2) per (batch, KV head, 32-row block, split); 0 for invalid shapes
    n = sdpa.decode_ws_bytes(16, 32, 8, 1, 16384, 128)
    assert n > 0 and n % (32 * 130 * 4) == 0
    units = n // (32 * 130 * 4)
    assert units % (16 * 8) == 0
    assert sdpa.decode_ws_bytes(1, 6, 4, 1, 100, 128) == 0
    assert sdpa.decode_ws_bytes(1, 8, 8, 1, 100, 96) == 0
    assert sdpa.decode_ws_bytes(1, 8, 8, 1, 100, 32) > 0
    assert sdpa.decode_ws_bytes(1, 8, 8, 1, 100, 256) > 0
    # the exact requirement is accepted, one byte less is not (validation only, no launch)
    need = sdpa.decode_ws_bytes(1, 4, 2, 8, 8, 64)
    assert call_dec(ws_bytes=need - 1) == 11



# packed variable-length sequences
def call_vl(entry="sdpa_fwd_varlen", **kw):
    a = dict(q=P, k=P, v=P, out=P, lse=P, cu_q=P, cu_k=P, n=3, tq=100, tk=100, mq=50, mk=50,
             Hq=4, Hkv=2, D=64, scale=0.125, mask_kind=1, window=0, bias_kind=0, bias=None,
             stream=None)
    a.update(kw)
    return sdpa.call_raw_varlen(entry, a["q"], a["k"], a["v"], a["out"], a["lse"], a["cu_q"],
                                a["cu_k"], a["n"], a["tq"], a["tk"], a["mq"], a["mk"], a["Hq"],
                                a["Hkv"], a["D"], a["scale"], a["mask_kind"], a["window"],
                                a["bias_kind"], a["bias"], a["stream"])


VL_CASES = [
    ("null cu_q", dict(cu_q=None), 1), ("null cu_k", dict(cu_k=None), 1),
    ("null q", dict(q=None), 1),
    ("no sequences", dict(n=0), 2), ("no query tokens", dict(tq=0), 2),
    ("no key tokens", dict(tk=0), 2), ("max len 0", dict(mq=0), 2),
    ("heads", dict(Hq=6, Hkv=4), 3), ("head dim", dict(D=96), 4),
    ("mask", dict(mask_kind=7), 5), ("window", dict(mask_kind=2, window=0), 6),
    ("full bias", dict(bias_kind=2, bias=P), 7), ("t5 without table", dict(bias_kind=1), 7),
    ("scale", dict(scale=math.inf), 8),
    ("misaligned cu", dict(cu_q=P + 2), 9), ("misaligned q", dict(q=P + 4), 9),
]


@pytest.mark.parametrize("entry", ["sdpa_fwd_varlen", "sdpa_fwd_varlen_f32out"])
@pytest.mark.parametrize("name,kw,code", VL_CASES, ids=[c[0] for c in VL_CASES])
def test_varlen_invalid_arguments_return_status(lib, entry, name, kw, code):
    assert call_vl(entry, **kw) == code


def test_library_binds_to_torch_hip_runtime():
    """Loading the library before torch is imported must not bring a second HIP runtime into
    the process: the binding imports torch first, so the library binds to torch's runtime."""
    import subprocess
    import sys
    code = ("import scaled_dot_product_03_amd as sdpa; sdpa.load(); import torch; "
            "maps = open('/proc/self/maps').read(); "
            "print(sorted({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    libs = eval(r.stdout.strip().splitlines()[-1])
    assert len(libs) == 1, libs
