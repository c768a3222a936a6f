"""The C ABI: every symbol include/splash.h declares is exported, and
argument errors come back as status codes before anything runs (CPU; no
GPU compute is called here)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from block_sparse_attention_make_amd import splash

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "splash.h")).read()
    return sorted(set(re.findall(r"SPLASH_API\s+[\w\s\*]+?\b(splash_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_symbols() == sorted([
        "splash_bwd", "splash_decode", "splash_decode_static", "splash_decode_workspace_size", "splash_fwd",
        "splash_fwd_heads_per_workgroup", "splash_fwd_plan", "splash_fwd_sinks", "splash_fwd_split",
        "splash_fwd_tiled", "splash_fwd_workspace_size",
        "splash_last_error", "splash_lse_merge",
        "splash_make_mask_info", "splash_make_mask_info_kv_slice", "splash_mask_info_destroy",
        "splash_mask_info_read_device", "splash_mask_info_upload", "splash_mask_info_view"])


def test_library_exports_every_declared_symbol():
    lib = splash.load_library()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    # nothing else with C linkage leaks out under the splash_ prefix
    out = os.popen(f"nm -D --defined-only {splash.LIB_PATH}").read()
    exported = sorted(set(re.findall(r"\b(splash_\w+)\b", out)))
    assert exported == declared_symbols()


def test_struct_layouts_match_header():
    assert ctypes.sizeof(splash._MaskDesc) == 56
    assert ctypes.sizeof(splash._ArrayView) == 48


def _fwd_args(info, **over):
    mi = info
    a = dict(mi=mi.handle, q=16, k=16, v=16, out=16, lse=None, B=1, Hq=2, Hkv=2, Sq=mi.q_len,
             Skv=mi.kv_len, D=128, Dv=128, dtype=splash.BF16, scale=math.nan, cap=0.0, stream=None)
    a.update(over)
    return list(a.values())


@pytest.mark.parametrize("over,status", [
    (dict(Sq=256), splash.EINVAL),                 # does not match the MaskInfo
    (dict(Hq=3, Hkv=2), splash.EINVAL),            # head ratio
    (dict(D=72, Dv=72), splash.EUNSUPPORTED),      # padding takes multiples of 16 only
    (dict(D=72, Dv=72, dtype=splash.F32), splash.EUNSUPPORTED),
    (dict(D=128, Dv=120), splash.EUNSUPPORTED),
    (dict(D=144, Dv=144), splash.EUNSUPPORTED),    # above the 128-column kernel
    (dict(D=64, Dv=256), splash.EUNSUPPORTED),
    (dict(D=8, Dv=8), splash.EUNSUPPORTED),
    (dict(dtype=7), splash.EINVAL),
    (dict(scale=-1.0), splash.EINVAL),
    (dict(scale=math.inf), splash.EINVAL),
    (dict(q=0), splash.EINVAL),                    # NULL tensor
    (dict(q=8), splash.EINVAL),                    # misaligned
    (dict(mi=None), splash.EINVAL),
])
def test_fwd_validation_errors_before_launch(over, status):
    lib = splash.load_library()
    mi = splash.make_mask_info("causal", 512, 512)
    st = lib.splash_fwd(*_fwd_args(mi, **over))
    assert st == status, lib.splash_last_error()
    assert lib.splash_last_error()


def test_fwd_rejects_non_128_blocks():
    lib = splash.load_library()
    mi = splash.make_mask_info("causal", 512, 512, block_q=64, block_kv=64)
    assert lib.splash_fwd(*_fwd_args(mi)) == splash.EUNSUPPORTED


def test_fwd_rejects_mask_head_mismatch():
    lib = splash.load_library()
    m = np.ones((3, 128, 128), dtype=bool)
    mi = splash.make_mask_info("dense", 128, 128, dense=m)
    assert lib.splash_fwd(*_fwd_args(mi, Hq=2, Hkv=2)) == splash.EINVAL


def test_fwd_empty_batch_is_noop():
    lib = splash.load_library()
    mi = splash.make_mask_info("causal", 512, 512)
    assert lib.splash_fwd(*_fwd_args(mi, B=0, q=0, k=0, v=0, out=0)) == splash.OK


def test_null_arguments():
    lib = splash.load_library()
    assert lib.splash_make_mask_info(None, 128, 128, 3, None) == splash.EINVAL
    assert lib.splash_mask_info_view(None, 0, None) == splash.EINVAL
    assert lib.splash_mask_info_upload(None) == splash.EINVAL
    lib.splash_mask_info_destroy(None)
    mi = splash.make_mask_info("causal", 256, 256)
    v = splash._ArrayView()
    assert lib.splash_mask_info_view(mi.handle, 9, ctypes.byref(v)) == splash.EINVAL
    # not uploaded -> read_device refuses
    buf = np.zeros(4, dtype=np.int8)
    assert lib.splash_mask_info_read_device(mi.handle, 0, buf.ctypes.data, 4) == splash.EINVAL


@pytest.mark.parametrize("aux,rows,ns,status", [
    (None, 1, 2, splash.EINVAL),     # NULL logits with sinks
    (16, 3, 1, splash.EINVAL),       # rows neither 1, Hkv nor Hq
    (16, 1, -1, splash.EINVAL),      # negative count
    (18, 1, 1, splash.EINVAL),       # misaligned
])
def test_fwd_sinks_validation_errors_before_launch(aux, rows, ns, status):
    lib = splash.load_library()
    mi = splash.make_mask_info("causal", 512, 512)
    a = _fwd_args(mi, Hq=4, Hkv=2)
    st = lib.splash_fwd_sinks(*a[:-1], aux, rows, ns, None)
    assert st == status, lib.splash_last_error()
    assert lib.splash_last_error()


def test_fwd_sinks_empty_batch_is_noop():
    lib = splash.load_library()
    mi = splash.make_mask_info("causal", 512, 512)
    a = _fwd_args(mi, B=0, q=0, k=0, v=0, out=0)
    assert lib.splash_fwd_sinks(*a[:-1], 16, 1, 1, None) == splash.OK
    assert lib.splash_fwd_sinks(*a[:-1], None, 0, 0, None) == splash.OK


@pytest.mark.parametrize("over,status", [
    (dict(dta=5), splash.EINVAL),
    (dict(rows=-1), splash.EINVAL),
    (dict(dv=100), splash.EUNSUPPORTED),           # not a multiple of 8
    (dict(dv=520), splash.EUNSUPPORTED),
    (dict(dv=1024), splash.EUNSUPPORTED),
    (dict(oa=0), splash.EINVAL),
    (dict(oa=8), splash.EINVAL),
    (dict(oo=16, dto=splash.F32), splash.EINVAL),   # in place with another dtype
])
def test_lse_merge_validation_errors_before_launch(over, status):
    lib = splash.load_library()
    a = dict(oa=16, la=16, dta=splash.BF16, ob=32, lb=32, dtb=splash.BF16, oo=16, lo=16,
             dto=splash.BF16, rows=4, dv=128, stream=None)
    a.update(over)
    assert lib.splash_lse_merge(*a.values()) == status, lib.splash_last_error()
    assert lib.splash_last_error()


def test_lse_merge_zero_rows_is_noop():
    lib = splash.load_library()
    assert lib.splash_lse_merge(None, None, 0, None, None, 0, None, None, 0, 0, 128, None) == splash.OK


@pytest.mark.parametrize("over,status", [
    (dict(dtype=splash.F32), splash.EUNSUPPORTED),
    (dict(Hq=3), splash.EINVAL),                     # head ratio
    (dict(Hq=64, Hkv=2), splash.EUNSUPPORTED),       # group of 32
    (dict(D=96, Dv=80), splash.EUNSUPPORTED),        # decode pads D == Dv only
    (dict(D=72, Dv=72), splash.EUNSUPPORTED),        # not a multiple of 16
    (dict(D=256, Dv=256), splash.EUNSUPPORTED),
    (dict(Skv=0), splash.EUNSUPPORTED),
    (dict(ws=0), splash.EINVAL),
    (dict(ws_bytes=16), splash.EINVAL),              # too small
    (dict(q=8), splash.EINVAL),
    (dict(Skv=1 << 23), splash.EUNSUPPORTED),        # one head's K cache of 2 GiB
])
def test_decode_validation_errors_before_launch(over, status):
    lib = splash.load_library()
    a = dict(q=16, k=16, v=16, out=16, lse=None, ws=16, ws_bytes=1 << 30, B=1, Hq=4, Hkv=2, Skv=1000, D=128,
             Dv=128, dtype=splash.BF16, scale=math.nan, cap=0.0, stream=None)
    a.update(over)
    assert lib.splash_decode(*a.values()) == status, lib.splash_last_error()


def test_decode_workspace_size():
    lib = splash.load_library()
    n = ctypes.c_size_t()
    assert lib.splash_decode_workspace_size(2, 8, 2, 1000, 128, ctypes.byref(n)) == splash.OK
    # groups of 4 at D = 128 stream 32-key stages: 4 (b, kv head) units x 32 stages -> 8 key
    # ranges of 4 stages (128 keys) each (at least 4 stages per range), (D + 2) floats per range
    # and query head
    assert n.value == 2 * 2 * 8 * 4 * (128 + 2) * 4
    # the bench's decode shape: 64 units x 1024 stages -> 8 ranges of 4096 keys (512 workgroups)
    assert lib.splash_decode_workspace_size(8, 32, 8, 32768, 128, ctypes.byref(n)) == splash.OK
    assert n.value == 8 * 8 * 8 * 4 * (128 + 2) * 4
    # groups of 16 at D = 128 (16 lanes per key): 1 unit x 32 stages -> 8 ranges of 4 stages
    assert lib.splash_decode_workspace_size(1, 16, 1, 1000, 128, ctypes.byref(n)) == splash.OK
    assert n.value == 1 * 1 * 8 * 16 * (128 + 2) * 4
    assert lib.splash_decode_workspace_size(1, 3, 2, 10, 64, ctypes.byref(n)) == splash.EINVAL


@pytest.mark.parametrize("dtype,skv", [(splash.BF16, 8 * 1024 * 1024 + 128), (splash.F32, 4 * 1024 * 1024 + 128)])
def test_fwd_and_bwd_reject_heads_beyond_32bit_buffers(dtype, skv):
    """One head of k / v larger than 2^31 - 1 bytes cannot be addressed by the
    kernels' 32-bit buffer resources: refused before anything runs."""
    lib = splash.load_library()
    mi = splash.make_mask_info("causal", 128, skv)
    st = lib.splash_fwd(*_fwd_args(mi, Hq=1, Hkv=1, dtype=dtype))
    assert st == splash.EUNSUPPORTED and "2^31" in lib.splash_last_error().decode()
    a = _fwd_args(mi, Hq=1, Hkv=1, dtype=dtype)
    assert lib.splash_fwd_sinks(*a[:-1], None, 0, 0, None) == splash.EUNSUPPORTED
    if dtype == splash.BF16:
        st = lib.splash_bwd(mi.handle, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 1, 1, 1, 128, skv, 128, 128,
                            splash.BF16, math.nan, 0.0, None)
        assert st == splash.EUNSUPPORTED and "2^31" in lib.splash_last_error().decode()
    # one block short of the limit passes validation (and then stops at the NULL lse-free no-op: B = 0)
    mi_ok = splash.make_mask_info("causal", 128, skv - 256)
    assert lib.splash_fwd(*_fwd_args(mi_ok, Hq=1, Hkv=1, dtype=dtype, B=0)) == splash.OK


@pytest.mark.parametrize("D,Dv,dtype,status", [
    (96, 96, splash.BF16, splash.OK),              # padded head dims pass validation (B = 0: no-op)
    (128, 64, splash.BF16, splash.OK),
    (96, 96, splash.F32, splash.EUNSUPPORTED),     # float32 runs D == Dv in {64, 128}
    (72, 72, splash.BF16, splash.EUNSUPPORTED),    # not a multiple of 16
    (160, 160, splash.BF16, splash.EUNSUPPORTED),  # above the 128-column kernels
])
def test_bwd_head_dims_validation(D, Dv, dtype, status):
    lib = splash.load_library()
    mi = splash.make_mask_info("causal", 256, 256)
    st = lib.splash_bwd(mi.handle, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 2, 2, 256, 256, D, Dv, dtype, math.nan, 0.0,
                        None)
    assert st == status, lib.splash_last_error()


def test_decode_workspace_size_padded_dims():
    """A padded head dim keeps its partials at the kernel's width: D = 96 and
    D = 112 take the 128-column workspace, D = 48 the 64-column one."""
    lib = splash.load_library()
    n = {}
    for d in (48, 64, 96, 112, 128):
        v = ctypes.c_size_t()
        assert lib.splash_decode_workspace_size(8, 32, 8, 32768, d, ctypes.byref(v)) == splash.OK
        n[d] = v.value
    assert n[96] == n[112] == n[128] and n[48] == n[64] and n[64] < n[128]


def test_binding_checks_caller_buffers():
    """Outputs the caller passes must have the shape and dtype the kernel
    writes; the check runs before any GPU work (CPU tensors are refused too)."""
    import torch
    x = torch.zeros((1, 2, 128, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        splash._check_buffer("out", x, (1, 2, 128, 128), torch.bfloat16, torch.device("cuda:0"))
    with pytest.raises(ValueError):
        splash._check_buffer("lse", torch.zeros(4), (1, 2, 128), torch.float32, torch.device("cpu"))
    with pytest.raises(ValueError):
        splash._check_buffer("out", x[:, :, :, :64], (1, 2, 128, 64), torch.bfloat16, torch.device("cpu"))
    splash._check_buffer("out", None, (1,), torch.float32, torch.device("cpu"))


def test_static_decode_rejects_more_than_its_scratch_before_running():
    """splash_decode_static keeps its partials in a 16 MiB static array: a
    decode whose partials need more is refused before any GPU call, and the
    other argument errors match splash_decode's."""
    lib = splash.load_library()
    n = ctypes.c_size_t()
    # 4096 x 16 query heads of D = 128, one range each: 4096 * 16 * 130 * 4 bytes = 34 MB of partials
    assert lib.splash_decode_workspace_size(4096, 16, 1, 1000, 128, ctypes.byref(n)) == splash.OK
    assert n.value > 16 << 20
    a = dict(q=16, k=16, v=16, out=16, lse=None, B=4096, Hq=16, Hkv=1, Skv=1000, D=128, Dv=128,
             dtype=splash.BF16, scale=math.nan, cap=0.0, stream=None)
    st = lib.splash_decode_static(*a.values())
    assert st == splash.EUNSUPPORTED and "scratch" in lib.splash_last_error().decode()
    for over, status in ((dict(dtype=splash.F32), splash.EUNSUPPORTED), (dict(Hq=3, Hkv=2), splash.EINVAL),
                         (dict(q=0), splash.EINVAL), (dict(q=8), splash.EINVAL), (dict(D=72, Dv=72), splash.EUNSUPPORTED)):
        b = dict(a, B=1, **over)
        assert lib.splash_decode_static(*b.values()) == status, (over, lib.splash_last_error())
    assert lib.splash_decode_static(*dict(a, B=0, q=0, k=0, v=0, out=0).values()) == splash.OK


@pytest.mark.parametrize("over,status", [
    (dict(splits=0), splash.EINVAL),
    (dict(splits=9), splash.EINVAL),
    (dict(splits=2, dtype=splash.F32), splash.EUNSUPPORTED),
    (dict(splits=2, ws=None), splash.EINVAL),                 # no workspace
    (dict(splits=2, ws_bytes=1024), splash.EINVAL),           # too small
    (dict(splits=2, ws=24), splash.EINVAL),                   # misaligned
    (dict(splits=2, Sq=256), splash.EINVAL),                  # MaskInfo mismatch, as splash_fwd
    (dict(splits=2, D=96, Dv=96, dtype=splash.F32), splash.EUNSUPPORTED),
])
def test_fwd_split_validation_errors_before_launch(over, status):
    lib = splash.load_library()
    mi = splash.make_mask_info("causal", 512, 512)
    a = dict(mi=mi.handle, q=16, k=16, v=16, out=16, lse=None, B=1, Hq=2, Hkv=2, Sq=512, Skv=512, D=128, Dv=128,
             dtype=splash.BF16, scale=math.nan, cap=0.0, aux=None, aux_rows=0, ns=0, splits=1, ws=16,
             ws_bytes=1 << 30, stream=None)
    a.update(over)
    assert lib.splash_fwd_split(*a.values()) == status, lib.splash_last_error()
    assert lib.splash_last_error()


def test_fwd_workspace_size_and_plan_on_host():
    lib = splash.load_library()
    n = ctypes.c_size_t()
    assert lib.splash_fwd_workspace_size(1, 8, 2048, 128, 4, ctypes.byref(n)) == splash.OK
    assert n.value == 4 * 8 * 2048 * (2 * 128 + 4)
    assert lib.splash_fwd_workspace_size(1, 8, 2048, 128, 1, ctypes.byref(n)) == splash.OK and n.value == 0
    assert lib.splash_fwd_workspace_size(1, 8, 2048, 128, 9, ctypes.byref(n)) == splash.EINVAL
    mi = splash.make_mask_info("causal", 512, 512)
    s = ctypes.c_int32(7)
    # float32 never splits; no device query is needed for it
    assert lib.splash_fwd_plan(mi.handle, 1, 2, splash.F32, ctypes.byref(s)) == splash.OK and s.value == 1
    assert lib.splash_fwd_plan(mi.handle, 0, 2, splash.BF16, ctypes.byref(s)) == splash.OK and s.value == 1
    assert lib.splash_fwd_plan(None, 1, 2, splash.BF16, ctypes.byref(s)) == splash.EINVAL


@pytest.mark.parametrize("mask, over, status", [
    ("causal", dict(heads=3), splash.EINVAL),                        # not 0, 1 or 2
    ("causal", dict(heads=-1), splash.EINVAL),
    ("causal", dict(heads=2, Hkv=4), splash.EUNSUPPORTED),           # group of one head
    ("causal", dict(heads=2, Hq=6, Hkv=2), splash.EUNSUPPORTED),     # odd group
    ("causal", dict(heads=2, D=64, Dv=64), splash.EUNSUPPORTED),     # D = 64
    ("causal", dict(heads=2, dtype=splash.F32), splash.EUNSUPPORTED),
    ("causal", dict(heads=2, D=64, Dv=48), splash.EUNSUPPORTED),     # padded dims in the 64-column kernel
    ("causal", dict(heads=2, D=32, Dv=32), splash.EUNSUPPORTED),
    ("dense", dict(heads=2), splash.EUNSUPPORTED),                   # dense mask
])
def test_fwd_tiled_validation_errors_before_launch(mask, over, status):
    """splash_fwd_tiled refuses shapes two heads cannot share a workgroup for
    (on the host, before anything is launched)."""
    lib = splash.load_library()
    if mask == "dense":
        mi = splash.make_mask_info("dense", 256, 256, dense=np.ones((1, 256, 256), dtype=bool))
    else:
        mi = splash.make_mask_info("causal", 256, 256)
    a = dict(mi=mi.handle, q=16, k=16, v=16, out=16, lse=None, B=1, Hq=4, Hkv=2, Sq=256, Skv=256, D=128, Dv=128,
             dtype=splash.BF16, scale=math.nan, cap=0.0, aux=None, aux_rows=0, ns=0, splits=1, heads=0, ws=None,
             ws_bytes=0, stream=None)
    a.update(over)
    assert lib.splash_fwd_tiled(*a.values()) == status, lib.splash_last_error()
    assert lib.splash_last_error()


def test_heads_per_workgroup_choice_on_host():
    lib = splash.load_library()
    h = ctypes.c_int32(7)
    causal = splash.make_mask_info("causal", 8192, 8192)
    # local_gqa_8k's shape: 16 pairs x 64 block rows fill 256 compute units
    assert lib.splash_fwd_heads_per_workgroup(causal.handle, 1, 32, 8, 128, splash.BF16, 1, ctypes.byref(h)) == 0
    assert h.value == 2
    # one head per kv head, float32, D = 64: no pairs
    for args in ((1, 16, 16, 128, splash.BF16), (1, 32, 8, 128, splash.F32), (1, 32, 8, 64, splash.BF16)):
        assert lib.splash_fwd_heads_per_workgroup(causal.handle, *args, 1, ctypes.byref(h)) == 0 and h.value == 1
    # too few pairs to give every compute unit one, unless split
    small = splash.make_mask_info("causal", 1024, 1024)
    assert lib.splash_fwd_heads_per_workgroup(small.handle, 1, 8, 2, 128, splash.BF16, 1, ctypes.byref(h)) == 0
    assert h.value == 1
    assert lib.splash_fwd_heads_per_workgroup(small.handle, 1, 8, 2, 128, splash.BF16, 8, ctypes.byref(h)) == 0
    assert h.value == 2
    dense = splash.make_mask_info("dense", 8192, 8192, dense=np.ones((1, 8192, 8192), dtype=bool))
    assert lib.splash_fwd_heads_per_workgroup(dense.handle, 1, 32, 8, 128, splash.BF16, 1, ctypes.byref(h)) == 0
    assert h.value == 1
    assert lib.splash_fwd_heads_per_workgroup(causal.handle, 1, 32, 0, 128, splash.BF16, 1, ctypes.byref(h)) == \
        splash.EINVAL
