"""Python binding of libsplash (ctypes).  Argument marshalling only: every
step of the path -- mask compilation and the attention kernel -- runs in the
native library.  torch is used for device memory and streams.

The library must have been built (block_sparse_attention_make_amd.build);
there is no fallback: a missing library raises.
"""
import ctypes
import math
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libsplash.so")

OK, EINVAL, ENOMEM, EHIP, EUNSUPPORTED = 0, 1, 2, 3, 4
MASK_KINDS = {"causal": 0, "local": 1, "chunked": 2, "dense": 3}
BF16, F32 = 0, 1
BLOCK_MASK, DATA_NEXT, MASK_NEXT, PARTIAL_BLOCKS, Q_SEQUENCE = range(5)
ARRAY_NAMES = ("block_mask", "data_next", "mask_next", "partial_mask_blocks", "q_sequence")
FLAG_SHRINK, FLAG_DOWNCAST = 1, 2


class SplashError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"splash status {status}: {msg}")
        self.status = status


class _MaskDesc(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("q_len", ctypes.c_int64), ("kv_len", ctypes.c_int64),
                ("left", ctypes.c_int64), ("right", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("dense", ctypes.c_void_p)]


class _ArrayView(ctypes.Structure):
    _fields_ = [("elem_bits", ctypes.c_int32), ("is_signed", ctypes.c_int32),
                ("ndim", ctypes.c_int32), ("_pad", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 3), ("data", ctypes.c_void_p)]


_lib = None


def load_library(path=None):
    """Load libsplash.so once; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m block_sparse_attention_make_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.splash_make_mask_info.argtypes = [ctypes.POINTER(_MaskDesc), i32, i32, ctypes.c_uint32, ctypes.POINTER(vp)]
    lib.splash_make_mask_info.restype = ctypes.c_int
    lib.splash_mask_info_view.argtypes = [vp, i32, ctypes.POINTER(_ArrayView)]
    lib.splash_mask_info_view.restype = ctypes.c_int
    lib.splash_mask_info_upload.argtypes = [vp]
    lib.splash_mask_info_upload.restype = ctypes.c_int
    lib.splash_mask_info_read_device.argtypes = [vp, i32, vp, ctypes.c_size_t]
    lib.splash_mask_info_read_device.restype = ctypes.c_int
    lib.splash_mask_info_destroy.argtypes = [vp]
    lib.splash_mask_info_destroy.restype = None
    lib.splash_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i32,
                               ctypes.c_float, ctypes.c_float, vp]
    lib.splash_fwd.restype = ctypes.c_int
    lib.splash_fwd_sinks.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i32,
                                     ctypes.c_float, ctypes.c_float, vp, i32, i32, vp]
    lib.splash_fwd_sinks.restype = ctypes.c_int
    lib.splash_fwd_split.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i32,
                                     ctypes.c_float, ctypes.c_float, vp, i32, i32, i32, vp, ctypes.c_size_t, vp]
    lib.splash_fwd_split.restype = ctypes.c_int
    lib.splash_fwd_tiled.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i32,
                                     ctypes.c_float, ctypes.c_float, vp, i32, i32, i32, i32, vp, ctypes.c_size_t, vp]
    lib.splash_fwd_tiled.restype = ctypes.c_int
    lib.splash_fwd_heads_per_workgroup.argtypes = [vp, i64, i64, i64, i64, i32, i32, ctypes.POINTER(ctypes.c_int32)]
    lib.splash_fwd_heads_per_workgroup.restype = ctypes.c_int
    lib.splash_fwd_workspace_size.argtypes = [i64, i64, i64, i64, i32, ctypes.POINTER(ctypes.c_size_t)]
    lib.splash_fwd_workspace_size.restype = ctypes.c_int
    lib.splash_fwd_plan.argtypes = [vp, i64, i64, i32, ctypes.POINTER(ctypes.c_int32)]
    lib.splash_fwd_plan.restype = ctypes.c_int
    lib.splash_make_mask_info_kv_slice.argtypes = [ctypes.POINTER(_MaskDesc), i64, i64, i32, i32,
                                                   ctypes.c_uint32, ctypes.POINTER(vp)]
    lib.splash_make_mask_info_kv_slice.restype = ctypes.c_int
    lib.splash_lse_merge.argtypes = [vp, vp, i32, vp, vp, i32, vp, vp, i32, i64, i64, vp]
    lib.splash_lse_merge.restype = ctypes.c_int
    lib.splash_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                               i32, ctypes.c_float, ctypes.c_float, vp]
    lib.splash_bwd.restype = ctypes.c_int
    lib.splash_decode_workspace_size.argtypes = [i64, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.splash_decode_workspace_size.restype = ctypes.c_int
    lib.splash_decode.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, i64, i64, i64, i64, i64, i64, i32,
                                  ctypes.c_float, ctypes.c_float, vp]
    lib.splash_decode.restype = ctypes.c_int
    lib.splash_decode_static.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, ctypes.c_float,
                                         ctypes.c_float, vp]
    lib.splash_decode_static.restype = ctypes.c_int
    lib.splash_last_error.argtypes = []
    lib.splash_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(lib, status):
    if status != OK:
        raise SplashError(status, lib.splash_last_error().decode())


_NP_INT = {(8, 1): np.int8, (16, 1): np.int16, (32, 1): np.int32, (8, 0): np.uint8}


class MaskInfo:
    """A compiled mask owned by the native library."""

    def __init__(self, handle, lib, kind, q_len, kv_len, block_q, block_kv, num_heads):
        self._h = handle
        self._lib = lib
        self.kind, self.q_len, self.kv_len = kind, q_len, kv_len
        self.block_q, self.block_kv, self.num_heads = block_q, block_kv, num_heads

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._lib.splash_mask_info_destroy(h)

    @property
    def handle(self):
        return self._h

    def _view(self, which):
        v = _ArrayView()
        _check(self._lib, self._lib.splash_mask_info_view(self._h, which, ctypes.byref(v)))
        return v

    def array(self, which):
        """Host copy of one MaskInfo array as numpy, or None."""
        v = self._view(which)
        if not v.data:
            return None
        dt = _NP_INT[(v.elem_bits, v.is_signed)]
        shape = tuple(v.shape[i] for i in range(v.ndim))
        n = int(np.prod(shape)) if shape else 0
        buf = (ctypes.c_char * (n * np.dtype(dt).itemsize)).from_address(v.data) if n else b""
        return np.frombuffer(bytes(buf), dtype=dt).reshape(shape).copy()

    def array_nbytes(self, which):
        v = self._view(which)
        if not v.data:
            return 0
        return int(np.prod([v.shape[i] for i in range(v.ndim)])) * v.elem_bits // 8

    @property
    def block_mask(self):
        return self.array(BLOCK_MASK)

    @property
    def data_next(self):
        return self.array(DATA_NEXT)

    @property
    def mask_next(self):
        return self.array(MASK_NEXT)

    @property
    def partial_mask_blocks(self):
        return self.array(PARTIAL_BLOCKS)

    @property
    def q_sequence(self):
        return self.array(Q_SEQUENCE)

    def upload(self):
        _check(self._lib, self._lib.splash_mask_info_upload(self._h))

    def read_device(self, which):
        """The device copy (current device) of one array, copied back to host."""
        host = self.array(which)
        if host is None:
            return None
        out = np.empty_like(host)
        _check(self._lib, self._lib.splash_mask_info_read_device(
            self._h, which, out.ctypes.data_as(ctypes.c_void_p), out.nbytes))
        return out


def make_mask_info(kind, q_len, kv_len, left=None, right=None, chunk=None, dense=None,
                   block_q=128, block_kv=128, shrink=True, downcast=True, kv_slice=None):
    """Compile a mask.  kind: "causal" | "local" | "chunked" | "dense".
    dense: host array [Hm, q_len, kv_len] (or [q_len, kv_len]), nonzero = allowed.
    kv_slice: optional (kv_start, kv_count) -- the MaskInfo of that key-axis
    slice of the mask (for a key/value shard); its kv_len is kv_count."""
    lib = load_library()
    if kind not in MASK_KINDS:
        raise ValueError(f"unknown mask kind {kind!r}")
    d = _MaskDesc()
    d.kind = MASK_KINDS[kind]
    d.num_heads = 1
    d.q_len, d.kv_len = int(q_len), int(kv_len)
    d.left = -1 if left is None else int(left)
    d.right = -1 if right is None else int(right)
    d.chunk = 0 if chunk is None else int(chunk)
    keep = None
    if kind == "dense":
        arr = dense.detach().cpu().numpy() if hasattr(dense, "detach") else np.asarray(dense)
        if arr.ndim == 2:
            arr = arr[None]
        keep = np.ascontiguousarray(arr.astype(np.uint8, copy=False))
        if keep.shape[1:] != (q_len, kv_len):
            raise ValueError("dense mask shape does not match (q_len, kv_len)")
        d.num_heads = keep.shape[0]
        d.dense = keep.ctypes.data
    flags = (FLAG_SHRINK if shrink else 0) | (FLAG_DOWNCAST if downcast else 0)
    h = ctypes.c_void_p()
    if kv_slice is None:
        _check(lib, lib.splash_make_mask_info(ctypes.byref(d), int(block_q), int(block_kv), flags,
                                              ctypes.byref(h)))
        local_kv = int(kv_len)
    else:
        k0, kn = int(kv_slice[0]), int(kv_slice[1])
        _check(lib, lib.splash_make_mask_info_kv_slice(ctypes.byref(d), k0, kn, int(block_q), int(block_kv),
                                                       flags, ctypes.byref(h)))
        local_kv = kn
    del keep
    return MaskInfo(h.value, lib, kind, int(q_len), local_kv, int(block_q), int(block_kv), d.num_heads)


def _check_buffer(name, t, shape, dtype, device):
    """A caller-supplied output or workspace tensor: the kernels write
    exactly `shape` elements of `dtype` at its data pointer, so anything else
    would be written out of bounds or misread."""
    if t is None:
        return
    if not (t.is_cuda and t.device == device):
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")


def plan_kv_splits(mask_info, B, Hq, dtype_code=BF16):
    """The library's recommended key-split count for this grid on the
    current device (splash_fwd_plan)."""
    lib = load_library()
    n = ctypes.c_int32()
    _check(lib, lib.splash_fwd_plan(mask_info.handle, int(B), int(Hq), int(dtype_code), ctypes.byref(n)))
    return int(n.value)


def plan_heads_per_workgroup(mask_info, B, Hq, Hkv, D, dtype_code=BF16, kv_splits=1):
    """The library's choice of query heads per workgroup (1, or 2 for two
    heads of a GQA group sharing each K/V stage) for this launch
    (splash_fwd_heads_per_workgroup)."""
    lib = load_library()
    n = ctypes.c_int32()
    _check(lib, lib.splash_fwd_heads_per_workgroup(mask_info.handle, int(B), int(Hq), int(Hkv), int(D),
                                                   int(dtype_code), int(kv_splits), ctypes.byref(n)))
    return int(n.value)


def splash_fwd(q, k, v, mask_info, softmax_scale=None, logits_soft_cap=None,
               out=None, lse=None, return_lse=True, stream=None, softmax_aux=None, kv_splits="auto",
               workspace=None, heads_per_workgroup=0):
    """Splash-attention forward on GPU torch tensors (contiguous BHSD).

    softmax_aux: optional attention-sink logits, a float32 GPU tensor [ns]
    (shared), [Hkv, ns] (query head h uses row h // (Hq // Hkv)) or [Hq, ns].
    Head dims: D == Dv in {64, 128}, or any D and Dv that are multiples of 16
    up to 128, which run zero-padded inside the 64- or 128-column kernel.
    kv_splits: "auto" (the library's plan: splits only when the grid has
    fewer block rows than the GPU has workgroup slots) or 1..8 -- each block
    row's non-empty blocks divided into that many workgroups, merged by lse;
    with more than one split a float32 workspace is allocated unless given.
    heads_per_workgroup: 0 (the library's choice), 1, or 2 (two heads of a
    GQA group per workgroup, sharing each K/V stage; see splash_fwd_tiled).
    Returns (out, lse); lse is float32 [B, Hq, Sq] or None if return_lse is False.
    Launches asynchronously on `stream` (default: torch's current stream).
    """
    import torch
    lib = load_library()
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if q.dtype not in (torch.bfloat16, torch.float32) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-d tensor [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Hkv, Skv, Dv = k.shape[1], k.shape[2], v.shape[3]
    if k.shape[0] != B or v.shape[:3] != k.shape[:3] or k.shape[3] != D:
        raise ValueError("k / v shapes do not match q")
    _check_buffer("out", out, (B, Hq, Sq, Dv), q.dtype, q.device)
    _check_buffer("lse", lse, (B, Hq, Sq), torch.float32, q.device)
    if out is None:
        out = torch.empty((B, Hq, Sq, Dv), dtype=q.dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    scale = math.nan if softmax_scale is None else float(softmax_scale)
    cap = 0.0 if logits_soft_cap is None else float(logits_soft_cap)
    dt = BF16 if q.dtype == torch.bfloat16 else F32
    lse_p = lse.data_ptr() if lse is not None else None
    aux_p, rows, ns = None, 0, 0
    if softmax_aux is not None:
        aux = softmax_aux
        if not (aux.is_cuda and aux.dtype == torch.float32 and aux.is_contiguous() and aux.dim() in (1, 2)):
            raise ValueError("softmax_aux must be a contiguous float32 GPU tensor [ns] or [rows, ns]")
        rows, ns = (1, aux.shape[0]) if aux.dim() == 1 else (aux.shape[0], aux.shape[1])
        aux_p = aux.data_ptr() if ns else None
    with torch.cuda.device(q.device):
        splits = plan_kv_splits(mask_info, B, Hq, dt) if kv_splits == "auto" else int(kv_splits)
        ws_p, ws_bytes = None, 0
        if splits > 1:
            nbytes = ctypes.c_size_t()
            _check(lib, lib.splash_fwd_workspace_size(B, Hq, Sq, Dv, splits, ctypes.byref(nbytes)))
            if workspace is None:
                workspace = torch.empty(max(1, nbytes.value // 4), dtype=torch.float32, device=q.device)
            elif not (workspace.is_cuda and workspace.device == q.device and workspace.is_contiguous()
                      and workspace.numel() * workspace.element_size() >= nbytes.value):
                raise ValueError(f"workspace must be a contiguous GPU tensor of at least {nbytes.value} bytes")
            ws_p, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        st = lib.splash_fwd_tiled(mask_info.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse_p, B, Hq, Hkv, Sq, Skv, D, Dv, dt, scale, cap, aux_p, rows, ns, splits,
                                  int(heads_per_workgroup), ws_p, ws_bytes, ctypes.c_void_p(stream.cuda_stream))
    _check(lib, st)
    return out, lse


def lse_merge(out_a, lse_a, out_b, lse_b, out=None, lse=None, out_dtype=None, stream=None):
    """Merge two attention results over disjoint key sets (GPU tensors
    [..., Dv] and float32 [...]) into the result over their union.  out / lse
    may be out_a / lse_a for an in-place accumulation.  Returns (out, lse)."""
    import torch
    lib = load_library()
    dts = {torch.bfloat16: BF16, torch.float32: F32}
    if out_a.shape != out_b.shape or lse_a.shape != lse_b.shape or out_a.shape[:-1] != lse_a.shape:
        raise ValueError("shapes of the two parts do not match")
    for t in (out_a, lse_a, out_b, lse_b):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("merge operands must be contiguous GPU tensors")
    if lse_a.dtype != torch.float32 or lse_b.dtype != torch.float32:
        raise ValueError("lse must be float32")
    if out is None:
        out = torch.empty(out_a.shape, dtype=out_dtype or out_a.dtype, device=out_a.device)
    _check_buffer("out", out, out_a.shape, out.dtype if out is not None else None, out_a.device)
    if out is not None and out.dtype not in dts:
        raise ValueError("out must be bfloat16 or float32")
    _check_buffer("lse", lse, lse_a.shape, torch.float32, out_a.device)
    if lse is None:
        lse = torch.empty(lse_a.shape, dtype=torch.float32, device=out_a.device)
    if stream is None:
        stream = torch.cuda.current_stream(out_a.device)
    rows, dv = lse_a.numel(), out_a.shape[-1]
    with torch.cuda.device(out_a.device):
        st = lib.splash_lse_merge(out_a.data_ptr(), lse_a.data_ptr(), dts[out_a.dtype],
                                  out_b.data_ptr(), lse_b.data_ptr(), dts[out_b.dtype],
                                  out.data_ptr(), lse.data_ptr(), dts[out.dtype], rows, dv,
                                  ctypes.c_void_p(stream.cuda_stream))
    _check(lib, st)
    return out, lse


def splash_fwd_kv_sharded(q, k_shards, v_shards, mask_infos, softmax_scale=None, logits_soft_cap=None,
                          stream=None):
    """Attention over key/value shards on one GPU -- the per-device part of
    ring attention: splash_fwd on each shard with its key-sliced MaskInfo,
    then an lse merge of each shard's result into a float32 accumulator.
    k_shards[s], v_shards[s]: [B, Hkv, n_s, D]; mask_infos[s] the MaskInfo of
    keys [sum of earlier n, + n_s) (make_mask_info(..., kv_slice=...)).
    Attention sinks are not accepted here (the tokamax ring variant refuses
    them too): a sink would be counted once per shard.  Returns (out, lse)."""
    import torch
    if not (len(k_shards) == len(v_shards) == len(mask_infos)) or not k_shards:
        raise ValueError("need one k, v and MaskInfo per shard")
    kw = dict(softmax_scale=softmax_scale, logits_soft_cap=logits_soft_cap, stream=stream)
    if len(k_shards) == 1:
        return splash_fwd(q, k_shards[0], v_shards[0], mask_infos[0], **kw)
    acc = lse = None
    for s, (k, v, mi) in enumerate(zip(k_shards, v_shards, mask_infos)):
        o_s, l_s = splash_fwd(q, k, v, mi, **kw)
        last = s == len(k_shards) - 1
        if acc is None:
            acc, lse = o_s, l_s
            continue
        dst = torch.empty(acc.shape, dtype=q.dtype if last else torch.float32, device=q.device) \
            if (last or acc.dtype != torch.float32) else acc
        acc, lse = lse_merge(acc, lse, o_s, l_s, out=dst, lse=lse, stream=stream)
    return acc, lse


def splash_bwd(q, k, v, out, lse, dout, mask_info, softmax_scale=None, logits_soft_cap=None,
               dq=None, dk=None, dv=None, delta=None, stream=None):
    """Gradients (dq, dk, dv) of splash_fwd's output for the output gradient
    dout (bf16 GPU tensors, contiguous BHSD; lse is splash_fwd's).  delta is
    an optional float32 [B, Hq, Sq] workspace.  Head dims as splash_fwd's
    bf16 forward."""
    import torch
    lib = load_library()
    if q.dtype != torch.bfloat16:
        raise ValueError("the backward runs bf16 only")
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if not (t.is_cuda and t.is_contiguous() and t.dim() == 4 and t.dtype == torch.bfloat16):
            raise ValueError(f"{name} must be a contiguous bf16 GPU tensor [B, H, S, D]")
    if lse is None or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be splash_fwd's float32 [B, Hq, Sq]")
    B, Hq, Sq, D = q.shape
    Hkv, Skv, Dv = k.shape[1], k.shape[2], v.shape[3]
    if out.shape != (B, Hq, Sq, Dv) or dout.shape != out.shape or lse.shape != (B, Hq, Sq):
        raise ValueError("out / dout / lse shapes do not match q")
    _check_buffer("dq", dq, q.shape, q.dtype, q.device)
    _check_buffer("dk", dk, k.shape, k.dtype, q.device)
    _check_buffer("dv", dv, v.shape, v.dtype, q.device)
    _check_buffer("delta", delta, (B, Hq, Sq), torch.float32, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if delta is None:
        delta = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    scale = math.nan if softmax_scale is None else float(softmax_scale)
    cap = 0.0 if logits_soft_cap is None else float(logits_soft_cap)
    with torch.cuda.device(q.device):
        st = lib.splash_bwd(mask_info.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                            delta.data_ptr(), B, Hq, Hkv, Sq, Skv, D, Dv, BF16, scale, cap,
                            ctypes.c_void_p(stream.cuda_stream))
    _check(lib, st)
    return dq, dk, dv


def splash_attention(q, k, v, mask_info, softmax_scale=None, logits_soft_cap=None):
    """Differentiable splash attention (bf16): forward through splash_fwd,
    backward through splash_bwd, as a torch.autograd.Function."""
    return _SplashFn.apply(q, k, v, mask_info, softmax_scale, logits_soft_cap)


def _make_fn():
    import torch

    class SplashFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, mask_info, softmax_scale, logits_soft_cap):
            out, lse = splash_fwd(q.contiguous(), k.contiguous(), v.contiguous(), mask_info,
                                  softmax_scale=softmax_scale, logits_soft_cap=logits_soft_cap)
            ctx.save_for_backward(q, k, v, out, lse)
            ctx.mask_info, ctx.scale, ctx.cap = mask_info, softmax_scale, logits_soft_cap
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, out, lse = ctx.saved_tensors
            dq, dk, dv = splash_bwd(q.contiguous(), k.contiguous(), v.contiguous(), out, lse,
                                    dout.contiguous(), ctx.mask_info, softmax_scale=ctx.scale,
                                    logits_soft_cap=ctx.cap)
            return dq, dk, dv, None, None, None

    return SplashFn


class _LazyFn:
    _fn = None

    def apply(self, *a):
        if _LazyFn._fn is None:
            _LazyFn._fn = _make_fn()
        return _LazyFn._fn.apply(*a)


_SplashFn = _LazyFn()


def splash_decode(q, k, v, softmax_scale=None, logits_soft_cap=None, out=None, lse=None, workspace=None,
                  stream=None):
    """Decode attention: q [B, Hq, 1, D] against every key of k, v [B, Hkv, Skv, D]
    (bf16 GPU tensors).  Returns (out [B, Hq, 1, D], lse float32 [B, Hq])."""
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not (t.is_cuda and t.is_contiguous() and t.dim() == 4 and t.dtype == torch.bfloat16):
            raise ValueError(f"{name} must be a contiguous bf16 GPU tensor [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Hkv, Skv, Dv = k.shape[1], k.shape[2], v.shape[3]
    if Sq != 1:
        raise ValueError("decode takes one query per head (q_len == 1)")
    nbytes = ctypes.c_size_t()
    _check(lib, lib.splash_decode_workspace_size(B, Hq, Hkv, Skv, D, ctypes.byref(nbytes)))
    _check_buffer("out", out, (B, Hq, 1, Dv), q.dtype, q.device)
    _check_buffer("lse", lse, (B, Hq), torch.float32, q.device)
    if workspace is not None and not (workspace.is_cuda and workspace.device == q.device
                                      and workspace.is_contiguous()
                                      and workspace.numel() * workspace.element_size() >= nbytes.value):
        raise ValueError(f"workspace must be a contiguous GPU tensor of at least {nbytes.value} bytes on {q.device}")
    if workspace is None:
        workspace = torch.empty(max(1, nbytes.value // 4), dtype=torch.float32, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, 1, Dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    scale = math.nan if softmax_scale is None else float(softmax_scale)
    cap = 0.0 if logits_soft_cap is None else float(logits_soft_cap)
    with torch.cuda.device(q.device):
        st = lib.splash_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               B, Hq, Hkv, Skv, D, Dv, BF16, scale, cap, ctypes.c_void_p(stream.cuda_stream))
    _check(lib, st)
    return out, lse


def splash_decode_static(q, k, v, softmax_scale=None, logits_soft_cap=None, out=None, lse=None, stream=None):
    """splash_decode without a workspace: the library keeps the partials in
    its own per-GPU static scratch (16 MiB), so the call itself allocates
    nothing beyond out / lse when those are not given.  Calls that overlap
    on one GPU race; calls ordered on one stream are safe."""
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not (t.is_cuda and t.is_contiguous() and t.dim() == 4 and t.dtype == torch.bfloat16):
            raise ValueError(f"{name} must be a contiguous bf16 GPU tensor [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Hkv, Skv, Dv = k.shape[1], k.shape[2], v.shape[3]
    if Sq != 1:
        raise ValueError("decode takes one query per head (q_len == 1)")
    _check_buffer("out", out, (B, Hq, 1, Dv), q.dtype, q.device)
    _check_buffer("lse", lse, (B, Hq), torch.float32, q.device)
    if out is None:
        out = torch.empty((B, Hq, 1, Dv), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    scale = math.nan if softmax_scale is None else float(softmax_scale)
    cap = 0.0 if logits_soft_cap is None else float(logits_soft_cap)
    with torch.cuda.device(q.device):
        st = lib.splash_decode_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                      B, Hq, Hkv, Skv, D, Dv, BF16, scale, cap, ctypes.c_void_p(stream.cuda_stream))
    _check(lib, st)
    return out, lse
