"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: the whole output is checked for finiteness and for the
properties that hold at any size, and a seeded sample of rows is compared
with the fp64 oracle row by row.  The device copy of each MaskInfo is read
back and compared bit for bit with the oracle's MaskInfo."""
import numpy as np
import pytest
import torch

from block_sparse_attention_make_amd import synthetic
from oracle import attention as oatt
from oracle import mask_info as omi
from oracle import masks as omasks
from tests.gpu_cases import TOL, mask_rows_fn, run_gpu

pytestmark = pytest.mark.gpu

FULL = ["causal_mha_8k", "local_gqa_8k", "chunked_gqa_16k_cap", "random_dense_2k"]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _mask_kw(w, dense):
    m = w.mask
    return dict(kind=m.kind, left=m.left, right=m.right, chunk=m.chunk, dense=dense)


def _samples(w, n, seed):
    rng = np.random.default_rng(seed)
    picks = []
    for _ in range(n):
        picks.append((int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(w.Sq))))
    # block edges and the last rows, where masks change
    picks += [(0, 0, 0), (w.B - 1, w.Hq - 1, w.Sq - 1), (0, w.Hq - 1, 127), (0, 0, 128), (w.B - 1, 0, w.Sq - 128)]
    return picks


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(name):
    w = synthetic.WORKLOADS[name]
    q, k, v, dense = synthetic.make_inputs(w)
    kw = _mask_kw(w, dense)
    o, l, mi = run_gpu(q, k, v, cap=w.soft_cap, **kw)
    assert np.isfinite(o).all() and np.isfinite(l).all(), "every row of these masks has an allowed key"
    # lse >= the row's own (diagonal) logit is not assumed; lse >= -|max logit| - 0 holds trivially.
    picks = _samples(w, 96, 1000 + w.seed)
    fn = mask_rows_fn(w.mask.kind, w.Skv, w.mask.left, w.mask.right, w.mask.chunk, dense)
    o_ref, l_ref = oatt.attention_sampled(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                          fn, picks, soft_cap=w.soft_cap)
    got_o = np.stack([o[b, h, i] for b, h, i in picks])
    got_l = np.array([l[b, h, i] for b, h, i in picks])
    err_o = float(np.abs(got_o - o_ref).max())
    err_l = float(np.abs(got_l - l_ref).max())
    print(f"{name}: {len(picks)} sampled rows max|dO|={err_o:.3e} max|dlse|={err_l:.3e}", flush=True)
    tol = TOL[w.torch_dtype]
    assert err_o <= tol and err_l <= tol


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
