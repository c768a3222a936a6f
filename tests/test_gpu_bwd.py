"""GPU parity of the backward (splash_bwd) against the fp64 oracle's
attention_bwd (itself pinned against torch autograd and central differences).

Tolerance: max-abs error of each gradient at most 1e-2 of the larger of 1 and
the reference's max-abs (GRAD_TOL).  The gradients are written in bf16 (a
relative rounding of up to 2^-9, 0.2 %) and p and ds enter the matrix
products rounded to bf16 (another 0.2 % per term, fp32 accumulation), so a
correct kernel sits near 0.4 % of the scale; measured maxima are 0.375 % in
these cases and 0.54 % in the smoke case's dq.  A dropped term, a wrong
scale or a missed block moves a gradient by far more."""
import numpy as np
import pytest
import torch

from block_sparse_attention_make_amd import make_mask_info, splash_attention, splash_bwd, splash_fwd, synthetic
from oracle import attention as oatt
from tests.gpu_cases import mask_rows_fn

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
GRAD_TOL = 1e-2


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(name, got, ref):
    got = got.float().cpu().numpy()
    assert np.isfinite(got).all(), f"{name}: non-finite"
    scale = max(1.0, float(np.abs(ref).max()))
    err = float(np.abs(got - ref).max())
    print(f"{name}: max|d|={err:.3e} ref max={scale:.3e}", flush=True)
    assert err <= GRAD_TOL * scale, (name, err, scale)


def _run(seed, B, Hq, Hkv, Sq, Skv, D, kind, cap=None, dense=None, **mk):
    q, k, v = synthetic.make_qkv(seed, B, Hq, Hkv, Sq, Skv, D, D)
    g = torch.Generator().manual_seed(seed + 1000)
    do = torch.randn((B, Hq, Sq, D), generator=g).to(torch.bfloat16)
    # compile-only options (block shape, shrink, downcast) do not change the mask
    compile_kw = {key: mk.pop(key) for key in ("block_q", "block_kv", "shrink", "downcast") if key in mk}
    mi = make_mask_info(kind, Sq, Skv, dense=dense, **mk, **compile_kw)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    out, lse = splash_fwd(qd, kd, vd, mi, logits_soft_cap=cap)
    nan = float("nan")
    dq = torch.full_like(qd, nan)
    dk = torch.full_like(kd, nan)
    dv = torch.full_like(vd, nan)
    splash_bwd(qd, kd, vd, out, lse, dod, mi, logits_soft_cap=cap, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    fn = mask_rows_fn(kind, Skv, dense=dense, **mk)
    rq, rk, rv = oatt.attention_bwd(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                    do.double().numpy(), fn, soft_cap=cap)
    return (dq, dk, dv), (rq, rk, rv)


CASES = [
    # name, seed, B, Hq, Hkv, Sq, Skv, D, mask kwargs, cap
    ("causal_gqa", 101, 1, 4, 2, 640, 640, 128, dict(kind="causal"), None),
    ("causal_mqa_b2", 102, 2, 2, 1, 384, 384, 128, dict(kind="causal"), None),
    ("local_cap", 103, 1, 2, 2, 768, 768, 128, dict(kind="local", left=200, right=50), 5.0),
    ("chunked", 104, 1, 4, 2, 1024, 1024, 128, dict(kind="chunked", chunk=300), None),
    ("causal_d64", 105, 1, 4, 2, 512, 512, 64, dict(kind="causal"), None),
    ("local_d64_cap", 106, 1, 2, 1, 512, 512, 64, dict(kind="local", left=None, right=100), 3.0),
    ("rect_sq_lt_skv", 107, 1, 2, 2, 256, 640, 128, dict(kind="causal"), None),
    ("rect_sq_gt_skv", 108, 1, 2, 2, 640, 256, 128, dict(kind="causal"), None),
    # 258 key blocks per row (more than one 256-slot metadata chunk; int16 data_next)
    ("rows_258_blocks", 109, 1, 2, 1, 256, 33024, 128, dict(kind="local", left=None, right=None), None),
    # more dQ workgroups (2 x 32 x 5 = 320) than compute units: the dQ kernel
    # streams 64-key half tiles, two workgroups per CU
    ("causal_half_tiles", 112, 2, 32, 8, 640, 640, 128, dict(kind="causal"), None),
    ("chunked_cap_half_tiles", 113, 2, 32, 4, 640, 640, 128, dict(kind="chunked", chunk=200), 5.0),
    # MaskInfo variants the walks must follow: 256 x 512 blocks (walked as
    # 128 x 128 sub-blocks), interior empty slots kept (shrink off), int32
    # index arrays (downcast off), and shrink off with half tiles
    ("causal_coarse_256x512", 114, 1, 4, 2, 1024, 1024, 128, dict(kind="causal", block_q=256, block_kv=512), None),
    ("local_no_shrink", 115, 1, 2, 2, 768, 768, 128, dict(kind="local", left=130, right=0, shrink=False), None),
    ("chunked_no_downcast_d64", 116, 1, 2, 1, 640, 640, 64, dict(kind="chunked", chunk=256, downcast=False), None),
    ("local_no_shrink_half_tiles", 117, 2, 32, 8, 640, 640, 128,
     dict(kind="local", left=150, right=20, shrink=False), None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_parity(case):
    name, seed, B, Hq, Hkv, Sq, Skv, D, mk, cap = case
    got, ref = _run(seed, B, Hq, Hkv, Sq, Skv, D, cap=cap, **mk)
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
        _check(f"{name}.{nm}", g_, r_)


@pytest.mark.parametrize("hm", [1, 2])
def test_bwd_dense_with_empty_rows_and_blocks(hm):
    rng = np.random.default_rng(110 + hm)
    dense = synthetic.random_dense_mask(rng, hm, 512, 640, 0.2, force_diagonal=True)
    dense[:, 0:128, 128:256] = True          # a full block
    dense[:, 128:256, 0:128] = False         # an empty block
    dense[:, 7, :] = False                   # a row with no allowed key
    dense[:, :, 600:] = False                # keys no query sees: their dk, dv are 0
    got, ref = _run(111, 1, 2, 1, 512, 640, 128, "dense", dense=dense)
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
        _check(f"dense_hm{hm}.{nm}", g_, r_)
    assert (got[0][:, :, 7] == 0).all()
    assert (got[1][:, :, 600:] == 0).all() and (got[2][:, :, 600:] == 0).all()


def test_bwd_dense_half_tiles():
    """A dense mask over more dQ workgroups than compute units (half tiles;
    mask words shared by a block's two halves)."""
    rng = np.random.default_rng(114)
    dense = synthetic.random_dense_mask(rng, 1, 640, 640, 0.2, force_diagonal=True)
    dense[:, 0:128, 128:256] = True          # a full block
    dense[:, 128:256, 0:128] = False         # an empty block
    got, ref = _run(115, 2, 32, 8, 640, 640, 128, "dense", dense=dense)
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
        _check(f"dense_half_tiles.{nm}", g_, r_)


def test_autograd_function_matches_splash_bwd():
    q, k, v = synthetic.make_qkv(120, 1, 2, 2, 384, 384, 128, 128)
    mi = make_mask_info("causal", 384, 384)
    qd, kd, vd = (t.to(DEV).requires_grad_() for t in (q, k, v))
    out = splash_attention(qd, kd, vd, mi)
    g = torch.Generator().manual_seed(121)
    do = torch.randn(out.shape, generator=g).to(torch.bfloat16).to(DEV)
    out.backward(do)
    torch.cuda.synchronize()
    o2, lse = splash_fwd(q.to(DEV), k.to(DEV), v.to(DEV), mi)
    dq, dk, dv = splash_bwd(q.to(DEV), k.to(DEV), v.to(DEV), o2, lse, do, mi)
    torch.cuda.synchronize()
    assert torch.equal(qd.grad, dq) and torch.equal(kd.grad, dk) and torch.equal(vd.grad, dv)
