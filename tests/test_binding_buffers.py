"""The binding checks every caller-supplied output and workspace buffer before the C call.

The C ABI sees raw pointers only: a buffer of the wrong dtype, shape, device or size would be
written past its end by the kernels. The binding must raise ValueError first. The CPU tests
call the checks directly; the GPU tests hand wrong buffers to every entry point and expect the
ValueError (nothing is launched: the check precedes the library call).
"""
import pytest
import torch

import scaled_dot_product_03_amd as sdpa

CPU = torch.device("cpu")


def test_check_buf_accepts_exact_buffer():
    t = torch.empty(2, 3, 4, 8, dtype=torch.bfloat16)
    assert sdpa._check_buf(t, "out", (2, 3, 4, 8), torch.bfloat16, CPU) is t


@pytest.mark.parametrize("what", ["dtype", "shape", "numel_same_shape_other", "noncontig",
                                  "device"])
def test_check_buf_rejects(what):
    shape = (2, 3, 4, 8)
    t = torch.empty(shape, dtype=torch.bfloat16)
    dev = CPU
    if what == "dtype":
        t = torch.empty(shape, dtype=torch.float32)   # 4-byte elements for a 2-byte output
    elif what == "shape":
        t = torch.empty(2, 3, 4, 7, dtype=torch.bfloat16)
    elif what == "numel_same_shape_other":
        t = torch.empty(2, 4, 3, 8, dtype=torch.bfloat16)
    elif what == "noncontig":
        t = torch.empty(2, 3, 8, 4, dtype=torch.bfloat16).transpose(2, 3)
    elif what == "device":
        dev = torch.device("meta")
    with pytest.raises(ValueError):
        sdpa._check_buf(t, "out", shape, torch.bfloat16, dev)


def test_check_ws_size():
    ws = torch.empty(100, dtype=torch.float32)
    assert sdpa._check_ws(ws, "ws", 400, CPU) is ws
    with pytest.raises(ValueError):
        sdpa._check_ws(ws, "ws", 401, CPU)
    with pytest.raises(ValueError):
        sdpa._check_ws(torch.empty(200, dtype=torch.float32)[::2], "ws", 4, CPU)


# ------------------------------------------------------------------------------------------
# through the entry points (needs cuda tensors; nothing is launched)
# ------------------------------------------------------------------------------------------
def _qkv(B=1, S=64, Hq=4, Hkv=2, D=64):
    q = torch.zeros(B, S, Hq, D, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(B, S, Hkv, D, dtype=torch.bfloat16, device="cuda")
    return q, k, k.clone()


@pytest.mark.gpu
def test_fwd_rejects_wrong_out_and_lse(gpu_lib):
    q, k, v = _qkv()
    bad_out = [
        dict(out=torch.empty(q.shape, dtype=torch.bfloat16, device="cuda"),
             out_dtype=torch.float32),                                  # fp32 epilogue, 2-byte out
        dict(out=torch.empty(1, 64, 4, 32, dtype=torch.bfloat16, device="cuda")),
        dict(out=torch.empty(q.shape, dtype=torch.bfloat16)),           # host memory
        dict(lse=torch.empty(1, 4, 63, device="cuda")),
        dict(lse=torch.empty(1, 4, 64, dtype=torch.float16, device="cuda")),
        dict(lse=torch.empty(1, 64, 4, device="cuda").transpose(1, 2)),
    ]
    for kw in bad_out:
        with pytest.raises(ValueError):
            gpu_lib.fwd(q, k, v, **kw)


@pytest.mark.gpu
def test_bwd_rejects_wrong_gradient_buffers_and_short_workspace(gpu_lib):
    q, k, v = _qkv()
    out = torch.zeros_like(q)
    lse = torch.zeros(1, 4, 64, device="cuda")
    cases = [
        dict(dq=torch.empty(q.shape, dtype=torch.bfloat16, device="cuda"),
             grad_dtype=torch.float32),
        dict(dk=torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")),   # Hq heads, not Hkv
        dict(dv=torch.empty(k.shape, dtype=torch.float32, device="cuda")),
        dict(ws=torch.empty(4 * 64 - 1, device="cuda")),                      # B*Hq*Sq - 1
        dict(ws=torch.empty(4 * 64, dtype=torch.bfloat16, device="cuda")),
    ]
    for kw in cases:
        with pytest.raises(ValueError):
            gpu_lib.bwd(q, k, v, out, lse, out, **kw)
    with pytest.raises(ValueError):
        gpu_lib.bwd(q, k, v, out, torch.zeros(1, 4, 32, device="cuda"), out)


@pytest.mark.gpu
def test_decode_rejects_short_workspace_and_wrong_out(gpu_lib):
    q = torch.zeros(2, 1, 8, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(2, 4096, 2, 128, dtype=torch.bfloat16, device="cuda")
    need = gpu_lib.decode_ws_bytes(2, 8, 2, 1, 4096, 128)
    assert need > 16
    with pytest.raises(ValueError):
        gpu_lib.decode(q, k, k, ws=torch.empty(need - 1, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        gpu_lib.decode(q, k, k, out=torch.empty(2, 1, 8, 128, device="cuda"))
    with pytest.raises(ValueError):
        gpu_lib.decode(q, k, k, lse=torch.empty(2, 1, 8, device="cuda"))


@pytest.mark.gpu
def test_varlen_rejects_wrong_out_and_lse(gpu_lib):
    q = torch.zeros(100, 4, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(100, 2, 64, dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, 40, 100], dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        gpu_lib.fwd_varlen(q, k, k, cu, cu, 60, 60, out=torch.empty(100, 4, 64, device="cuda"))
    with pytest.raises(ValueError):
        gpu_lib.fwd_varlen(q, k, k, cu, cu, 60, 60, lse=torch.empty(100, 4, device="cuda"))
