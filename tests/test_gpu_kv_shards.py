"""GPU parity of the key/value-sharded path (the per-device part of ring
attention): key-axis MaskInfo slices run by splash_fwd, and the lse merge
kernel, against the fp64 oracle (its merge is pinned to full attention by
the shard-split identity)."""
import numpy as np
import pytest
import torch

from block_sparse_attention_make_amd import (lse_merge, make_mask_info, splash_fwd, splash_fwd_kv_sharded,
                                             synthetic)
from oracle import attention as oatt
from tests.gpu_cases import TOL, compare, mask_rows_fn, oracle_full

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


DEV = torch.device("cuda:0")


def _oracle_slice(q, k, v, kind, k0, kn, cap=None, **mk):
    """Oracle attention over keys [k0, k0 + kn) only, with the full mask's columns."""
    full = mask_rows_fn(kind, k.shape[2], **mk)
    fn = lambda h, rows: full(h, rows)[:, k0:k0 + kn]
    return oatt.attention(q.double().numpy(), k[:, :, k0:k0 + kn].double().numpy(),
                          v[:, :, k0:k0 + kn].double().numpy(), fn, soft_cap=cap)


@pytest.mark.parametrize("kind,mk,dt,D,cap", [
    ("causal", {}, torch.bfloat16, 128, None),
    ("local", dict(left=150, right=60), torch.bfloat16, 128, 4.0),
    ("local", dict(left=None, right=20), torch.bfloat16, 64, None),
    ("chunked", dict(chunk=200), torch.bfloat16, 128, None),
    ("causal", {}, torch.float32, 128, None),
    ("local", dict(left=100, right=100), torch.float32, 64, None),
])
def test_single_slice_at_offset(kind, mk, dt, D, cap):
    """One middle slice alone: the kernel must apply the computable mask at the
    slice's key offset (rows with no allowed key in the slice give 0 / -inf)."""
    q, k, v = synthetic.make_qkv(91, 1, 2, 2, 768, 768, D, D, dtype=dt)
    k0, kn = 256, 384
    mi = make_mask_info(kind, 768, 768, kv_slice=(k0, kn), **mk)
    kd = k[:, :, k0:k0 + kn].contiguous().to(DEV)
    vd = v[:, :, k0:k0 + kn].contiguous().to(DEV)
    o, l = splash_fwd(q.to(DEV), kd, vd, mi, logits_soft_cap=cap)
    torch.cuda.synchronize()
    o_ref, l_ref = _oracle_slice(q, k, v, kind, k0, kn, cap=cap, **mk)
    compare(o.float().cpu().numpy(), l.cpu().numpy(), o_ref, l_ref, TOL[dt], f"slice_{kind}")


def _shards(S, sizes):
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    assert sum(sizes) == S
    return list(zip(starts.tolist(), sizes))


@pytest.mark.parametrize("kind,mk,sizes,cap", [
    ("causal", {}, [256, 256, 256, 256], None),
    ("causal", {}, [128, 640, 256], None),
    ("local", dict(left=200, right=30), [384, 640], 5.0),
    ("chunked", dict(chunk=300), [512, 128, 384], None),
    ("dense", {}, [256, 384, 384], None),
])
def test_sharded_forward_equals_full_attention(kind, mk, sizes, cap):
    S = sum(sizes)
    q, k, v = synthetic.make_qkv(92, 1, 4, 2, S, S, 128, 128)
    dense = None
    if kind == "dense":
        rng = np.random.default_rng(93)
        dense = synthetic.random_dense_mask(rng, 1, S, S, 0.1, force_diagonal=True)
        mk = dict(dense=dense)
    mis, ks, vs = [], [], []
    for k0, kn in _shards(S, sizes):
        mis.append(make_mask_info(kind, S, S, kv_slice=(k0, kn), **mk))
        ks.append(k[:, :, k0:k0 + kn].contiguous().to(DEV))
        vs.append(v[:, :, k0:k0 + kn].contiguous().to(DEV))
    o, l = splash_fwd_kv_sharded(q.to(DEV), ks, vs, mis, logits_soft_cap=cap)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    o_ref, l_ref = oracle_full(q, k, v, kind, cap=cap, **mk)
    compare(o.float().cpu().numpy(), l.cpu().numpy(), o_ref, l_ref, TOL[torch.bfloat16], f"sharded_{kind}")


@pytest.mark.parametrize("dta,dtb,dto,dv", [
    (torch.float32, torch.float32, torch.float32, 128),
    (torch.bfloat16, torch.bfloat16, torch.float32, 128),
    (torch.float32, torch.bfloat16, torch.bfloat16, 64),
    (torch.bfloat16, torch.float32, torch.bfloat16, 256),
    (torch.float32, torch.float32, torch.float32, 8),
    (torch.bfloat16, torch.bfloat16, torch.float32, 96),     # 12 chunks a row: 16 threads, 4 idle
    (torch.float32, torch.bfloat16, torch.bfloat16, 40),
    (torch.float32, torch.float32, torch.float32, 512),
])
def test_merge_kernel_parity(dta, dtb, dto, dv):
    """Random parts with rows empty in one part, in the other, in both; the
    empty parts' outputs hold NaN garbage, which must not leak."""
    rng = np.random.default_rng(94)
    rows = 3000
    oa = rng.standard_normal((rows, dv)).astype(np.float32)
    ob = rng.standard_normal((rows, dv)).astype(np.float32)
    la = (3 * rng.standard_normal(rows)).astype(np.float32)
    lb = (3 * rng.standard_normal(rows)).astype(np.float32)
    la[::7] = -np.inf
    lb[::5] = -np.inf
    lb[:40] = la[:40] + 30          # far apart
    oa[la == -np.inf] = np.nan
    ob[lb == -np.inf] = np.nan
    ta = torch.from_numpy(oa).to(dta).to(DEV)
    tb = torch.from_numpy(ob).to(dtb).to(DEV)
    o, l = lse_merge(ta, torch.from_numpy(la).to(DEV), tb, torch.from_numpy(lb).to(DEV), out_dtype=dto)
    torch.cuda.synchronize()
    ref_o, ref_l = oatt.merge(ta.float().cpu().numpy(), la, tb.float().cpu().numpy(), lb)
    tol = 2e-2 if dto == torch.bfloat16 else 1e-5
    compare(o.float().cpu().numpy(), l.cpu().numpy(), ref_o, ref_l, tol, "merge")


@pytest.mark.parametrize("dv", [128, 96, 24])
def test_merge_in_place(dv):
    """Out and lse written over part a; a row's threads must all read its
    lse before any writes it (also where Dv / 8 is not a power of two)."""
    rng = np.random.default_rng(95)
    rows = 1000
    a = torch.from_numpy(rng.standard_normal((rows, dv)).astype(np.float32)).to(DEV)
    b = torch.from_numpy(rng.standard_normal((rows, dv)).astype(np.float32)).to(DEV)
    la = torch.from_numpy(rng.standard_normal(rows).astype(np.float32)).to(DEV)
    lb = torch.from_numpy(rng.standard_normal(rows).astype(np.float32)).to(DEV)
    ref_o, ref_l = oatt.merge(a.cpu().numpy(), la.cpu().numpy(), b.cpu().numpy(), lb.cpu().numpy())
    o, l = lse_merge(a, la, b, lb, out=a, lse=la)
    torch.cuda.synchronize()
    assert o.data_ptr() == a.data_ptr() and l.data_ptr() == la.data_ptr()
    compare(a.cpu().numpy(), la.cpu().numpy(), ref_o, ref_l, 1e-5, f"merge_in_place dv={dv}")


@pytest.mark.parametrize("D,Dv", [(96, 80), (32, 48)])
def test_sharded_forward_padded_head_dims(D, Dv):
    """The key/value-sharded path at head dims run zero-padded: each shard's
    forward, then the merge over rows of Dv elements."""
    sizes = [384, 256, 384]
    S = sum(sizes)
    q, k, v = synthetic.make_qkv(96 + D, 1, 4, 2, S, S, D, Dv)
    mis, ks, vs = [], [], []
    for k0, kn in _shards(S, sizes):
        mis.append(make_mask_info("causal", S, S, kv_slice=(k0, kn)))
        ks.append(k[:, :, k0:k0 + kn].contiguous().to(DEV))
        vs.append(v[:, :, k0:k0 + kn].contiguous().to(DEV))
    o, l = splash_fwd_kv_sharded(q.to(DEV), ks, vs, mis)
    torch.cuda.synchronize()
    assert o.shape == (1, 4, S, Dv)
    o_ref, l_ref = oracle_full(q, k, v, "causal")
    compare(o.float().cpu().numpy(), l.cpu().numpy(), o_ref, l_ref, TOL[torch.bfloat16], f"sharded D={D} Dv={Dv}")
