"""The C ABI library loads, exports every function declared in include/attn.h,
and rejects invalid arguments on the host before any HIP call (CPU only).

Every call below carries at least one invalid argument, so no kernel is ever
launched and no pointer is dereferenced; the fake pointers are never read.
"""
import ctypes
import os
import re
import subprocess

import pytest

import io_aware_exact_attn_amd as ia

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

P = 0x10000          # 16-byte aligned fake device address (never dereferenced)
MIS = 0x10004        # misaligned


def declared_functions():
    src = open(HEADER, encoding="utf-8").read()
    return re.findall(r"ATTN_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)


def test_header_declares_the_entry_points():
    assert set(declared_functions()) == {"attn_fwd", "attn_fwd_fp8", "attn_quantize_fp8", "attn_quantize_fp8_rotated", "attn_quantize_mxfp8", "attn_fwd_mxfp8", "attn_bwd",
                                         "attn_bwd_noalloc", "attn_status_str", "attn_kernel_name"}


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", ia.library_path], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(ia.lib, name)


def bf16(**kw):
    args = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=16, d=128, scale=0.1, causal=0,
                cu_seqlens=None, dtype=ia.ATTN_BF16, stream=0)
    args.update(kw)
    return ia.attn_fwd(**args, check=False)


def fp8(**kw):
    args = dict(q=P, k=P, v=P, q_scale=P, k_scale=P, v_scale=P, o=P, lse=P, B=1, H=1, N=128,
                d=128, scale=0.1, causal=1, cu_seqlens=None, stream=0)
    args.update(kw)
    return ia.attn_fwd_fp8(**args, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ia.ATTN_ERR_NULL), (dict(k=None), ia.ATTN_ERR_NULL),
    (dict(v=None), ia.ATTN_ERR_NULL), (dict(o=None), ia.ATTN_ERR_NULL),
    (dict(lse=None), ia.ATTN_ERR_NULL),
    (dict(B=0), ia.ATTN_ERR_SHAPE), (dict(H=-1), ia.ATTN_ERR_SHAPE), (dict(N=0), ia.ATTN_ERR_SHAPE),
    (dict(B=1 << 16, H=1 << 8, N=1 << 8), ia.ATTN_ERR_SHAPE),
    (dict(d=96, N=1), ia.ATTN_ERR_UNSUPPORTED), (dict(d=256), ia.ATTN_ERR_UNSUPPORTED),
    (dict(causal=2), ia.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=ia.ATTN_FP8_E4M3), ia.ATTN_ERR_UNSUPPORTED), (dict(dtype=7), ia.ATTN_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), ia.ATTN_ERR_SCALE), (dict(scale=float("inf")), ia.ATTN_ERR_SCALE),
    (dict(q=MIS), ia.ATTN_ERR_ALIGN), (dict(o=MIS), ia.ATTN_ERR_ALIGN), (dict(lse=MIS), ia.ATTN_ERR_ALIGN),
    (dict(cu_seqlens=MIS), ia.ATTN_ERR_ALIGN),
    (dict(cu_seqlens=P, B=1 << 30, H=4, N=1 << 0), ia.ATTN_ERR_SHAPE),
    (dict(H=(1 << 17) + 1, N=1), ia.ATTN_ERR_SHAPE),     # H * d > 2^24
])
def test_attn_fwd_rejects(kw, status):
    assert bf16(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q_scale=None), ia.ATTN_ERR_NULL), (dict(v_scale=None), ia.ATTN_ERR_NULL),
    (dict(o=None), ia.ATTN_ERR_NULL),
    (dict(d=64), ia.ATTN_ERR_UNSUPPORTED), (dict(cu_seqlens=MIS), ia.ATTN_ERR_ALIGN),
    (dict(cu_seqlens=P, B=1 << 30, H=4, N=1), ia.ATTN_ERR_SHAPE),
    (dict(causal=-1), ia.ATTN_ERR_UNSUPPORTED),
    (dict(scale=float("-inf")), ia.ATTN_ERR_SCALE),
    (dict(k_scale=MIS), ia.ATTN_ERR_ALIGN), (dict(v=MIS), ia.ATTN_ERR_ALIGN),
    (dict(N=0), ia.ATTN_ERR_SHAPE),
    (dict(H=(1 << 17) + 1, N=1), ia.ATTN_ERR_SHAPE),     # H * d > 2^24
])
def test_attn_fwd_fp8_rejects(kw, status):
    assert fp8(**kw) == status


def mxfp8(**kw):
    args = dict(q=P, k=P, v=P, q_scale=P, k_scale=P, v_scale=P, o=P, lse=P, B=1, H=1, N=128,
                d=128, scale=0.1, causal=1, cu_seqlens=None, stream=0)
    args.update(kw)
    return ia.attn_fwd_mxfp8(**args, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ia.ATTN_ERR_NULL), (dict(k_scale=None), ia.ATTN_ERR_NULL), (dict(v_scale=None), ia.ATTN_ERR_NULL),
    (dict(lse=None), ia.ATTN_ERR_NULL),
    (dict(d=64), ia.ATTN_ERR_UNSUPPORTED), (dict(causal=3), ia.ATTN_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), ia.ATTN_ERR_SCALE),
    (dict(q_scale=MIS), ia.ATTN_ERR_ALIGN), (dict(v_scale=MIS), ia.ATTN_ERR_ALIGN), (dict(o=MIS), ia.ATTN_ERR_ALIGN),
    (dict(cu_seqlens=MIS), ia.ATTN_ERR_ALIGN),
    (dict(N=0), ia.ATTN_ERR_SHAPE), (dict(B=1 << 16, H=1 << 8, N=1 << 8), ia.ATTN_ERR_SHAPE),
    (dict(cu_seqlens=P, B=1 << 30, H=4, N=1), ia.ATTN_ERR_SHAPE),
    (dict(H=(1 << 17) + 1, N=1), ia.ATTN_ERR_SHAPE),     # H * d > 2^24
])
def test_attn_fwd_mxfp8_rejects(kw, status):
    assert mxfp8(**kw) == status


def quant(**kw):
    args = dict(x=P, y=P, scales=P, B=1, H=2, N=300, d=128, cu_seqlens=None, stream=0)
    args.update(kw)
    return ia.attn_quantize_fp8(**args, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), ia.ATTN_ERR_NULL), (dict(y=None), ia.ATTN_ERR_NULL), (dict(scales=None), ia.ATTN_ERR_NULL),
    (dict(B=0), ia.ATTN_ERR_SHAPE), (dict(H=0), ia.ATTN_ERR_SHAPE), (dict(N=-5), ia.ATTN_ERR_SHAPE),
    (dict(B=1 << 16, H=1 << 8, N=1 << 8), ia.ATTN_ERR_SHAPE),
    (dict(d=96), ia.ATTN_ERR_UNSUPPORTED), (dict(d=256), ia.ATTN_ERR_UNSUPPORTED),
    (dict(x=MIS), ia.ATTN_ERR_ALIGN), (dict(y=MIS), ia.ATTN_ERR_ALIGN), (dict(scales=MIS), ia.ATTN_ERR_ALIGN),
    (dict(cu_seqlens=MIS), ia.ATTN_ERR_ALIGN),
    (dict(cu_seqlens=P, B=1 << 30, H=4, N=1), ia.ATTN_ERR_SHAPE),
])
def test_attn_quantize_fp8_rejects(kw, status):
    assert quant(**kw) == status


def quant_rot(**kw):
    args = dict(x=P, y=P, scales=P, signs=P, B=1, H=2, N=300, d=128, cu_seqlens=None, stream=0)
    args.update(kw)
    return ia.attn_quantize_fp8_rotated(**args, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), ia.ATTN_ERR_NULL), (dict(signs=None), ia.ATTN_ERR_NULL), (dict(scales=None), ia.ATTN_ERR_NULL),
    (dict(B=0), ia.ATTN_ERR_SHAPE), (dict(N=0), ia.ATTN_ERR_SHAPE),
    (dict(B=1 << 16, H=1 << 8, N=1 << 8), ia.ATTN_ERR_SHAPE),
    (dict(d=32), ia.ATTN_ERR_UNSUPPORTED), (dict(d=256), ia.ATTN_ERR_UNSUPPORTED),
    (dict(signs=MIS), ia.ATTN_ERR_ALIGN), (dict(y=MIS), ia.ATTN_ERR_ALIGN), (dict(cu_seqlens=MIS), ia.ATTN_ERR_ALIGN),
    (dict(cu_seqlens=P, B=1 << 30, H=4, N=1), ia.ATTN_ERR_SHAPE),
])
def test_attn_quantize_fp8_rotated_rejects(kw, status):
    assert quant_rot(**kw) == status


def quant_mx(**kw):
    args = dict(x=P, y=P, scales=P, B=1, H=2, N=300, d=128, cu_seqlens=None, along_tokens=0, stream=0)
    args.update(kw)
    return ia.attn_quantize_mxfp8(**args, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), ia.ATTN_ERR_NULL), (dict(scales=None), ia.ATTN_ERR_NULL),
    (dict(B=0), ia.ATTN_ERR_SHAPE), (dict(N=0), ia.ATTN_ERR_SHAPE),
    (dict(B=1 << 16, H=1 << 8, N=1 << 8), ia.ATTN_ERR_SHAPE),
    (dict(d=96), ia.ATTN_ERR_UNSUPPORTED), (dict(along_tokens=2), ia.ATTN_ERR_UNSUPPORTED),
    (dict(y=MIS), ia.ATTN_ERR_ALIGN), (dict(scales=MIS), ia.ATTN_ERR_ALIGN), (dict(cu_seqlens=MIS), ia.ATTN_ERR_ALIGN),
])
def test_attn_quantize_mxfp8_rejects(kw, status):
    assert quant_mx(**kw) == status


def bwd(**kw):
    args = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, delta=P, dq=P, dk=P, dv=P, B=1, H=2, N=300, d=128,
                scale=0.1, causal=1, cu_seqlens=None, stream=0)
    args.update(kw)
    return ia.attn_bwd(**args, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ia.ATTN_ERR_NULL), (dict(dout=None), ia.ATTN_ERR_NULL), (dict(lse=None), ia.ATTN_ERR_NULL),
    (dict(delta=None), ia.ATTN_ERR_NULL), (dict(dq=None), ia.ATTN_ERR_NULL), (dict(dv=None), ia.ATTN_ERR_NULL),
    (dict(B=0), ia.ATTN_ERR_SHAPE), (dict(H=0), ia.ATTN_ERR_SHAPE), (dict(N=-1), ia.ATTN_ERR_SHAPE),
    (dict(B=1 << 16, H=1 << 8, N=1 << 8), ia.ATTN_ERR_SHAPE),
    (dict(d=96), ia.ATTN_ERR_UNSUPPORTED), (dict(d=256), ia.ATTN_ERR_UNSUPPORTED),
    (dict(causal=2), ia.ATTN_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), ia.ATTN_ERR_SCALE),
    (dict(o=MIS), ia.ATTN_ERR_ALIGN), (dict(delta=MIS), ia.ATTN_ERR_ALIGN), (dict(dk=MIS), ia.ATTN_ERR_ALIGN),
    (dict(cu_seqlens=MIS), ia.ATTN_ERR_ALIGN),
    (dict(cu_seqlens=P, B=1 << 30, H=4, N=1), ia.ATTN_ERR_SHAPE),
    (dict(H=(1 << 17) + 1, N=1), ia.ATTN_ERR_SHAPE),     # H * d > 2^24
])
def test_attn_bwd_rejects(kw, status):
    assert bwd(**kw) == status


def bwd_noalloc(**kw):
    args = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, B=1, H=2, N=300, d=128,
                scale=0.1, causal=1, cu_seqlens=None, stream=0)
    args.update(kw)
    return ia.attn_bwd_noalloc(**args, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ia.ATTN_ERR_NULL), (dict(lse=None), ia.ATTN_ERR_NULL), (dict(dk=None), ia.ATTN_ERR_NULL),
    (dict(B=0), ia.ATTN_ERR_SHAPE), (dict(d=96), ia.ATTN_ERR_UNSUPPORTED), (dict(causal=5), ia.ATTN_ERR_UNSUPPORTED),
    (dict(scale=float("inf")), ia.ATTN_ERR_SCALE), (dict(dv=MIS), ia.ATTN_ERR_ALIGN),
    (dict(cu_seqlens=MIS), ia.ATTN_ERR_ALIGN),
    # D rows beyond the fixed 2^21-row scratch: fixed length B * H * N, packed H * N
    (dict(B=2, H=16, N=(1 << 16) + 1), ia.ATTN_ERR_SCRATCH),
    (dict(cu_seqlens=P, B=3, H=32, N=(1 << 16) + 1), ia.ATTN_ERR_SCRATCH),
])
def test_attn_bwd_noalloc_rejects(kw, status):
    assert bwd_noalloc(**kw) == status


def test_status_strings():
    for s in range(8):
        assert ia.attn_status_str(s) and ia.attn_status_str(s) != "unknown status"
    assert ia.attn_status_str(99) == "unknown status"
    assert ia.attn_status_str(-1) == "unknown status"


def test_kernel_names():
    assert ia.attn_kernel_name(128, 1, 0, ia.ATTN_BF16) == "attn_fwd_bf16_kernel<d128,causal,fixed,bf16>"
    assert ia.attn_kernel_name(64, 0, 1, ia.ATTN_BF16_OUT_F32) == "attn_fwd_bf16_kernel<d64,full,packed,f32>"
    assert ia.attn_kernel_name(128, 1, 0, 0, fp8=1) == "attn_fwd_fp8_kernel<causal,fixed>"
    assert ia.attn_kernel_name(128, 0, 1, 0, fp8=1) == "attn_fwd_fp8_kernel<full,packed>"
    assert ia.attn_kernel_name(96, 1, 0, 0) == ""
    assert ia.attn_kernel_name(64, 1, 1, 0, fp8=1) == ""
    assert ia.attn_kernel_name(128, 3, 0, 0) == ""


def test_python_binding_refuses_host_tensors():
    import torch
    t = torch.zeros(4)
    with pytest.raises(ValueError):
        ia.attn_fwd(t, t, t, t, t, 1, 1, 1, 128, 0.1, 0, None, 0, stream=0)


def test_status_raises():
    with pytest.raises(ia.AttnError) as e:
        ia.attn_fwd(None, P, P, P, P, 1, 1, 1, 128, 0.1, 0, None, 0, stream=0)
    assert e.value.status == ia.ATTN_ERR_NULL


def test_single_hip_runtime_whatever_the_import_order():
    """The library must share torch's HIP runtime (torch owns the memory and
    streams); importing the binding before torch must not map a second one."""
    code = ("import io_aware_exact_attn_amd, torch\n"
            "libs = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(libs))\n")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=ROOT, check=True)
    assert out.stdout.strip() == "1", out.stdout + out.stderr
