"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: every element of out and lse against the fp64 oracle, and
the device copy of each MaskInfo read back and compared bit for bit with the
oracle's MaskInfo."""
import numpy as np
import pytest
import torch

from block_sparse_attention_make_amd import synthetic
from oracle import attention as oatt
from oracle import mask_info as omi
from oracle import masks as omasks
from tests.gpu_cases import TOL, compare, mask_rows_fn, oracle_by_block_rows, run_gpu

pytestmark = pytest.mark.gpu

FULL = ["causal_mha_8k", "local_gqa_8k", "chunked_gqa_16k_cap", "random_dense_2k", "causal_d96_8k"]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _mask_kw(w, dense):
    m = w.mask
    return dict(kind=m.kind, left=m.left, right=m.right, chunk=m.chunk, dense=dense)


@pytest.mark.parametrize("name", FULL)
def test_full_size_whole_output(name):
    """Every row of every head of the workload, as bench.py launches it."""
    w = synthetic.WORKLOADS[name]
    q, k, v, dense = synthetic.make_inputs(w)
    kw = _mask_kw(w, dense)
    o, l, mi = run_gpu(q, k, v, cap=w.soft_cap, **kw)
    assert np.isfinite(l).all(), "every row of these masks has an allowed key"
    o_ref, l_ref = oracle_by_block_rows(q, k, v, cap=w.soft_cap, **kw)
    compare(o, l, o_ref, l_ref, TOL[w.torch_dtype], f"{name} (all {o.shape[0] * o.shape[1] * o.shape[2]} rows)")


def test_dense_empty_rows_whole_output():
    """dense_empty_rows_2k as bench.py launches it (split keys): every 16th
    row allows no key and must come out as 0 with lse -inf, the rest as the
    oracle's."""
    w = synthetic.WORKLOADS["dense_empty_rows_2k"]
    q, k, v, dense = synthetic.make_inputs(w)
    kw = _mask_kw(w, dense)
    o, l, mi = run_gpu(q, k, v, cap=w.soft_cap, **kw)
    assert np.isneginf(l[:, :, ::16]).all() and np.isfinite(l[:, :, 1::16]).all()
    assert (o[:, :, ::16] == 0).all()
    o_ref, l_ref = oracle_by_block_rows(q, k, v, cap=w.soft_cap, **kw)
    compare(o, l, o_ref, l_ref, TOL[w.torch_dtype], f"{w.name} (all rows)")


@pytest.mark.parametrize("name", synthetic.WORKLOAD_ORDER)
def test_device_mask_info_bit_exact(name):
    w = synthetic.WORKLOADS[name]
    from block_sparse_attention_make_amd import make_mask_info
    from block_sparse_attention_make_amd.splash import ARRAY_NAMES
    dense = synthetic.make_inputs(w)[3] if w.mask.kind == "dense" else None
    m = w.mask
    mi = make_mask_info(m.kind, w.Sq, w.Skv, left=m.left, right=m.right, chunk=m.chunk, dense=dense)
    mi.upload()
    if m.kind == "dense":
        ref = omi.build(dense, 128, 128, computable=False)
    else:
        ref = omi.build(omasks.materialize(m.kind, w.Sq, w.Skv, left=m.left, right=m.right, chunk=m.chunk),
                        128, 128, computable=True)
    for which, nm in enumerate(ARRAY_NAMES):
        r = getattr(ref, nm)
        d = mi.read_device(which)
        if r is None:
            assert d is None, nm
            continue
        assert d.dtype == r.dtype and d.shape == r.shape and d.tobytes() == r.tobytes(), nm


@pytest.mark.parametrize("name", sorted(synthetic.DECODE_WORKLOADS))
def test_decode_full_size_whole_output(name):
    """decode_gqa_32k (B = 8, Hq = 32, Hkv = 8, 32,768 cached keys, D = 128, and the same at
    D = 96), called as the decode benchmark calls it: every (b, query head) row against the
    fp64 oracle with every key allowed."""
    from block_sparse_attention_make_amd import splash_decode
    w = synthetic.DECODE_WORKLOADS[name]
    q, k, v = synthetic.make_qkv(w.seed, w.B, w.Hq, w.Hkv, 1, w.Skv, w.D, w.Dv)
    dev = torch.device("cuda:0")
    out, lse = splash_decode(q.to(dev), k.to(dev), v.to(dev))
    torch.cuda.synchronize()
    o, l = out.float().cpu().numpy(), lse.cpu().numpy()
    o_ref, l_ref = oracle_by_block_rows(q, k, v, "local")   # no window: every key allowed
    compare(o, l[:, :, None], o_ref, l_ref, TOL[torch.bfloat16], f"{w.name} (all {w.B * w.Hq} rows)")


def test_bwd_full_size_sampled():
    """causal_mha_8k backward (B = 1, 16 heads, S = 8192, D = 128), with the output gradient
    the backward benchmark draws (torch generator seed 11): every gradient finite; dq, dk and
    dv of two whole heads, and dq of sampled rows of the other heads, against the fp64 oracle.
    Tolerance: 1e-2 of the larger of 1 and the reference's max-abs, as for the small cases."""
    from block_sparse_attention_make_amd import make_mask_info, splash_bwd, splash_fwd
    w = synthetic.WORKLOADS["causal_mha_8k"]
    q, k, v, _ = synthetic.make_inputs(w)
    dev = torch.device("cuda:0")
    mi = make_mask_info("causal", w.Sq, w.Skv)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out, lse = splash_fwd(qd, kd, vd, mi)
    g = torch.Generator().manual_seed(11)
    do = torch.randn(out.shape, generator=g).to(q.dtype)
    dq, dk, dv = splash_bwd(qd, kd, vd, out, lse, do.to(dev), mi)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy() for t in (dq, dk, dv)]
    for name, t in zip(("dq", "dk", "dv"), got):
        assert np.isfinite(t).all(), name
    q64, k64, v64, do64 = (t.double().numpy() for t in (q, k, v, do))
    fn = mask_rows_fn("causal", w.Skv)

    def check(name, a, ref):
        scale = max(1.0, float(np.abs(ref).max()))
        err = float(np.abs(a - ref).max())
        print(f"{w.name} {name}: max|d|={err:.3e} ref max={scale:.3e}", flush=True)
        assert err <= 1e-2 * scale, (name, err, scale)

    rng = np.random.default_rng(3000 + w.seed)
    heads = [0, int(rng.integers(1, w.Hq))]
    for h in heads:
        sl = slice(h, h + 1)   # MHA: query head h reads kv head h
        rq, rk, rv = oatt.attention_bwd(q64[:, sl], k64[:, sl], v64[:, sl], do64[:, sl], fn)
        check(f"head {h} dq", got[0][:, sl], rq)
        check(f"head {h} dk", got[1][:, sl], rk)
        check(f"head {h} dv", got[2][:, sl], rv)
    rows = [(int(rng.integers(w.Hq)), int(rng.integers(w.Sq))) for _ in range(24)] + [(w.Hq - 1, w.Sq - 1)]
    for h, i in rows:
        rq, _, _ = oatt.attention_bwd_rows(q64[0, h, [i]], k64[0, h], v64[0, h], do64[0, h, [i]],
                                           fn(h, np.array([i])))
        check(f"dq row ({h}, {i})", got[0][0, h, [i]], rq)
