"""Shared helpers for the GPU parity tests: run the HIP path and the oracle
on the same seeded inputs."""
import numpy as np
import torch

from block_sparse_attention_make_amd import make_mask_info, splash_fwd
from oracle import attention as oatt
from oracle import masks as omasks

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-5}


def mask_rows_fn(kind, skv, left=None, right=None, chunk=None, dense=None):
    if kind == "dense":
        return lambda h, rows: dense[0 if dense.shape[0] == 1 else h][rows]
    cols = np.arange(skv)
    return lambda h, rows: omasks.allowed_block(kind, rows, cols, left=left, right=right, chunk=chunk)


def run_gpu(q, k, v, kind, left=None, right=None, chunk=None, dense=None, cap=None, scale=None,
            nan_fill=True, aux=None, kv_splits="auto", **mi_kw):
    """splash_fwd on cuda:0 with a MaskInfo compiled for the mask (mi_kw:
    further make_mask_info options, e.g. shrink / downcast) and the given key
    splits ("auto": the library's plan); returns out and lse as numpy arrays
    and the MaskInfo."""
    dev = torch.device("cuda:0")
    Sq, Skv = q.shape[2], k.shape[2]
    mi = make_mask_info(kind, Sq, Skv, left=left, right=right, chunk=chunk, dense=dense, **mi_kw)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = lse = None
    if nan_fill:   # rows the kernel fails to write stay NaN and fail the comparison
        out = torch.full((q.shape[0], q.shape[1], Sq, v.shape[3]), float("nan"), dtype=q.dtype, device=dev)
        lse = torch.full((q.shape[0], q.shape[1], Sq), float("nan"), dtype=torch.float32, device=dev)
    auxd = None if aux is None else torch.as_tensor(np.asarray(aux, dtype=np.float32)).to(dev)
    out, lse = splash_fwd(qd, kd, vd, mi, softmax_scale=scale, logits_soft_cap=cap, out=out, lse=lse,
                          softmax_aux=auxd, kv_splits=kv_splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), mi


def oracle_full(q, k, v, kind, left=None, right=None, chunk=None, dense=None, cap=None, scale=None,
                aux=None):
    fn = mask_rows_fn(kind, k.shape[2], left, right, chunk, dense)
    return oatt.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), fn,
                          scale=scale, soft_cap=cap,
                          softmax_aux=None if aux is None else np.asarray(aux, dtype=np.float32))


def compare(o, l, o_ref, l_ref, tol, what=""):
    """Max-abs error on out and lse; -inf lse rows must match exactly."""
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    inf_ref = ~np.isfinite(l_ref)
    assert np.array_equal(inf_ref, ~np.isfinite(l)), f"{what}: -inf lse rows differ"
    assert (l[inf_ref] == -np.inf).all() and (l_ref[inf_ref] == -np.inf).all()
    err_o = float(np.abs(o - o_ref).max()) if o.size else 0.0
    err_l = float(np.abs(l[~inf_ref] - l_ref[~inf_ref]).max()) if (~inf_ref).any() else 0.0
    print(f"{what}: max|dO|={err_o:.3e} max|dlse|={err_l:.3e} tol={tol}", flush=True)
    assert err_o <= tol and err_l <= tol, (what, err_o, err_l)
    return err_o, err_l


def oracle_by_block_rows(q, k, v, kind, left=None, right=None, chunk=None, dense=None, cap=None,
                         scale=None, rows_per_call=256, workers=None):
    """The fp64 oracle over every output row, called per (b, h, group of query
    rows) on only the key columns from the first to the last key any of
    those rows may see.  Keys outside that span are masked for all of the
    rows, and a masked key adds nothing to the definition's sums, so this is
    the oracle's own result at a fraction of its cost; it makes whole-output
    parity affordable at the full workload sizes.  The calls run on a thread
    pool with one BLAS thread each: numpy releases the GIL inside its kernels."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    B, Hq, Sq, _ = q.shape
    Hkv, Skv, Dv = k.shape[1], k.shape[2], v.shape[3]
    group = Hq // Hkv
    fn = mask_rows_fn(kind, Skv, left, right, chunk, dense)
    q64 = q.double().numpy()
    k64 = k.double().numpy()
    v64 = v.double().numpy()
    o = np.zeros((B, Hq, Sq, Dv), dtype=np.float64)
    lse = np.zeros((B, Hq, Sq), dtype=np.float64)

    def one(task):
        b, h, i0 = task
        kk, vv = k64[b, h // group], v64[b, h // group]
        rows = np.arange(i0, min(Sq, i0 + rows_per_call))
        allowed = fn(h, rows)
        seen = np.flatnonzero(allowed.any(axis=0))
        if seen.size == 0:
            o[b, h, rows] = 0.0
            lse[b, h, rows] = -np.inf
            return
        c0, c1 = int(seen[0]), int(seen[-1]) + 1
        ob, lb = oatt.attention_rows(q64[b, h, rows], kk[c0:c1], vv[c0:c1], allowed[:, c0:c1], scale, cap)
        o[b, h, rows] = ob
        lse[b, h, rows] = lb

    tasks = [(b, h, i0) for b in range(B) for h in range(Hq) for i0 in range(0, Sq, rows_per_call)]
    n = workers or min(16, os.cpu_count() or 1)
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(one, tasks))
    return o, lse
