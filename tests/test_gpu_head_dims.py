"""GPU parity for head dims other than D == Dv in {64, 128}: the forward
(bf16 and float32) runs any D and Dv that are multiples of 16 up to 128
zero-padded inside its 64- or 128-column kernel (the EasyDeL BlockSparseAttn
signature types the query/key head dim and the value head dim apart).

Each case is compared element by element with the fp64 oracle (whose
attention is pinned with Dv != D and the default scale of the true D) at the
bf16 tolerance, 2e-2 max-abs on out and lse.  The cases cover both padded
kernels, with and without the soft cap, computable and dense masks, GQA /
MQA, Sq != Skv, attention sinks, and the default softmax scale (D ** -0.5 of
the caller's D, not of the padded one).  The backward runs the same
padding; its gradients are compared with the oracle's attention_bwd (pinned
with Dv != D against torch autograd and central differences).
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_make_amd import make_mask_info, splash_bwd, splash_fwd, synthetic
from oracle import attention as oatt
from tests.gpu_cases import TOL, compare, mask_rows_fn, oracle_full, run_gpu

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    # name, seed, B, Hq, Hkv, Sq, Skv, D, Dv, mask kwargs, cap
    # 64-column kernel (D, Dv <= 64)
    ("d32_causal_mqa_b2", 201, 2, 2, 1, 384, 384, 32, 32, dict(kind="causal"), None),
    ("d48_local_cap", 202, 1, 4, 2, 640, 640, 48, 48, dict(kind="local", left=200, right=50), 5.0),
    ("d16_dv48_chunked", 203, 1, 2, 2, 768, 768, 16, 48, dict(kind="chunked", chunk=300), None),
    ("d64_dv32_causal_rect", 204, 1, 2, 2, 256, 640, 64, 32, dict(kind="causal"), None),
    # 128-column kernel
    ("d96_causal_gqa", 205, 1, 4, 2, 640, 640, 96, 96, dict(kind="causal"), None),
    ("d128_dv64_local", 206, 1, 2, 2, 768, 768, 128, 64, dict(kind="local", left=None, right=100), None),
    ("d64_dv128_chunked_cap", 207, 1, 4, 2, 1024, 1024, 64, 128, dict(kind="chunked", chunk=300), 5.0),
    ("d80_dv112_causal_rect", 208, 1, 2, 1, 640, 256, 80, 112, dict(kind="causal"), None),
    ("d112_dv16_full_cap", 209, 1, 2, 2, 384, 384, 112, 16, dict(kind="local", left=None, right=None), 2.0),
    ("d96_long_causal", 210, 1, 2, 2, 2048, 2048, 96, 96, dict(kind="causal"), None),
    ("d96_one_block", 211, 1, 1, 1, 128, 128, 96, 96, dict(kind="causal"), None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_padded_head_dims_parity(case):
    """kv_splits="auto": the library's split plan (these small grids split)."""
    name, seed, B, Hq, Hkv, Sq, Skv, D, Dv, mk, cap = case
    q, k, v = synthetic.make_qkv(seed, B, Hq, Hkv, Sq, Skv, D, Dv)
    o, l, _ = run_gpu(q, k, v, cap=cap, **mk)
    assert o.shape == (B, Hq, Sq, Dv)
    o_ref, l_ref = oracle_full(q, k, v, cap=cap, **mk)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], name)


F32_CASES = [
    # name, seed, B, Hq, Hkv, Sq, Skv, D, Dv, mask kwargs, cap
    ("f32_d96_causal_gqa", 290, 1, 4, 2, 384, 384, 96, 96, dict(kind="causal"), None),
    ("f32_d32_dv48_local_cap", 291, 1, 2, 1, 512, 512, 32, 48, dict(kind="local", left=130, right=3), 4.0),
    ("f32_d112_dv80_rect", 292, 1, 2, 2, 256, 640, 112, 80, dict(kind="causal"), None),
]


@pytest.mark.parametrize("case", F32_CASES, ids=[c[0] for c in F32_CASES])
def test_padded_head_dims_f32(case):
    """The float32 forward at padded dims, at its own bar (1e-5)."""
    name, seed, B, Hq, Hkv, Sq, Skv, D, Dv, mk, cap = case
    q, k, v = synthetic.make_qkv(seed, B, Hq, Hkv, Sq, Skv, D, Dv, dtype=torch.float32)
    o, l, _ = run_gpu(q, k, v, cap=cap, **mk)
    o_ref, l_ref = oracle_full(q, k, v, cap=cap, **mk)
    compare(o, l, o_ref, l_ref, TOL[torch.float32], name)


@pytest.mark.parametrize("D,Dv,cap", [(48, 64, None), (96, 80, 3.0)], ids=["kernel64", "kernel128_cap"])
@pytest.mark.parametrize("hm", [1, 2])
def test_padded_head_dims_dense(D, Dv, cap, hm):
    """Dense masks (partial blocks read from the mask bits) in both padded
    kernels, shared and per-head masks, with an empty and a full block."""
    rng = np.random.default_rng(220 + hm + D)
    q, k, v = synthetic.make_qkv(221 + D, 1, 2, 2, 512, 640, D, Dv)
    dense = synthetic.random_dense_mask(rng, hm, 512, 640, 0.2, force_diagonal=True)
    dense[:, 0:128, 128:256] = True
    dense[:, 128:256, 0:128] = False
    o, l, _ = run_gpu(q, k, v, "dense", dense=dense, cap=cap)
    o_ref, l_ref = oracle_full(q, k, v, "dense", dense=dense, cap=cap)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], f"dense D={D} Dv={Dv} hm={hm}")


@pytest.mark.parametrize("D,Dv", [(32, 48), (96, 112)])
def test_padded_head_dims_sinks(D, Dv):
    """Attention sinks per key/value head, with a fully masked block row (its
    rows then hold only the sinks: out 0, lse = log sum exp of the sinks)."""
    q, k, v = synthetic.make_qkv(230 + D, 1, 4, 2, 384, 512, D, Dv)
    dense = np.ones((1, 384, 512), dtype=bool)
    dense[0, 128:256, :] = False
    aux = np.array([[0.5, -1.0], [1.5, -np.inf]], dtype=np.float32)
    o, l, _ = run_gpu(q, k, v, "dense", dense=dense, aux=aux)
    o_ref, l_ref = oracle_full(q, k, v, "dense", dense=dense, aux=aux)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], f"sinks D={D} Dv={Dv}")
    assert (o[:, :, 128:256] == 0).all()


def test_padded_head_dims_explicit_scale_and_neighbours_untouched():
    """An explicit softmax_scale, and an output buffer carved from a larger
    one: the kernel writes exactly [B, Hq, Sq, Dv] elements, nothing past
    them (the 128-column kernel must not store its padding columns)."""
    B, Hq, Hkv, S, D, Dv = 1, 2, 2, 384, 96, 80
    q, k, v = synthetic.make_qkv(240, B, Hq, Hkv, S, S, D, Dv)
    mi = make_mask_info("causal", S, S)
    n = B * Hq * S * Dv
    buf = torch.full((n + 4096,), 7.0, dtype=torch.bfloat16, device=DEV)
    out = buf[:n].view(B, Hq, S, Dv)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=DEV)
    splash_fwd(q.to(DEV), k.to(DEV), v.to(DEV), mi, softmax_scale=0.05, out=out, lse=lse)
    torch.cuda.synchronize()
    assert (buf[n:] == 7.0).all()
    o_ref, l_ref = oracle_full(q, k, v, "causal", scale=0.05)
    compare(out.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, TOL[torch.bfloat16], "scale 0.05")


SHAPE_CASES = [
    # name, seed, B, Hq, Hkv, Sq, Skv, D, Dv, mask kwargs, cap, splits
    ("d96_causal_g2_splits4", 250, 1, 4, 2, 640, 640, 96, 96, dict(kind="causal"), None, 4),
    ("d64_dv112_local_g4", 251, 1, 8, 2, 1024, 1024, 64, 112, dict(kind="local", left=300, right=40), None, 1),
    ("d80_chunked_cap_g2_splits3", 252, 1, 4, 2, 1536, 1536, 80, 80, dict(kind="chunked", chunk=640), 30.0, 3),
    ("d128_dv96_rect_g2_splits2", 253, 1, 4, 2, 512, 1664, 128, 96, dict(kind="causal"), None, 2),
]


def _run_shape(q, k, v, mk, cap, splits, heads, aux=None):
    Sq, Skv = q.shape[2], k.shape[2]
    mi = make_mask_info(mk["kind"], Sq, Skv, left=mk.get("left"), right=mk.get("right"), chunk=mk.get("chunk"))
    out = torch.full(q.shape[:3] + (v.shape[3],), float("nan"), dtype=q.dtype, device=DEV)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    auxd = None if aux is None else torch.as_tensor(aux).to(DEV)
    splash_fwd(q.to(DEV), k.to(DEV), v.to(DEV), mi, logits_soft_cap=cap, out=out, lse=lse, kv_splits=splits,
               heads_per_workgroup=heads, softmax_aux=auxd)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("case", SHAPE_CASES, ids=[c[0] for c in SHAPE_CASES])
def test_padded_head_dims_launch_shapes(case):
    """Key splits and two heads per workgroup at padded dims (128-column
    kernel): against the oracle, and one head per workgroup against two bit
    for bit (each row's arithmetic is the same in both shapes)."""
    name, seed, B, Hq, Hkv, Sq, Skv, D, Dv, mk, cap, splits = case
    q, k, v = synthetic.make_qkv(seed, B, Hq, Hkv, Sq, Skv, D, Dv)
    o2, l2 = _run_shape(q, k, v, mk, cap, splits, heads=2)
    o_ref, l_ref = oracle_full(q, k, v, cap=cap, **mk)
    compare(o2.float().numpy(), l2.numpy(), o_ref, l_ref, TOL[torch.bfloat16], f"{name} two heads per workgroup")
    o1, l1 = _run_shape(q, k, v, mk, cap, splits, heads=1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{name}: one and two heads per workgroup differ"


@pytest.mark.parametrize("D,Dv", [(32, 48), (112, 80)])
def test_padded_head_dims_splits_dense_sinks(D, Dv):
    """Key splits (1, 2, 5) at padded dims with a dense mask, an empty block
    row and sinks (the merge adds them once); every split count against the
    oracle."""
    q, k, v = synthetic.make_qkv(255 + D, 1, 4, 2, 512, 768, D, Dv)
    rng = np.random.default_rng(256 + D)
    dense = synthetic.random_dense_mask(rng, 1, 512, 768, 0.3, force_diagonal=True)
    dense[0, 128:256, :] = False
    aux = np.array([[0.25, -0.5], [1.0, -np.inf]], dtype=np.float32)
    o_ref, l_ref = oracle_full(q, k, v, "dense", dense=dense, aux=aux)
    for splits in (1, 2, 5):
        o, l, _ = run_gpu(q, k, v, "dense", dense=dense, aux=aux, kv_splits=splits)
        compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], f"dense sinks D={D} Dv={Dv} splits={splits}")
        assert (o[:, :, 128:256] == 0).all()


# ---- backward at padded head dims --------------------------------------------
# Tolerance as in the backward's own parity tests: max-abs error of each
# gradient at most 1e-2 of the larger of 1 and the oracle's max-abs (bf16
# gradients and bf16 p and ds in the products sit near 0.4 % of the scale).
GRAD_TOL = 1e-2


def _grad_check(name, got, ref):
    got = got.float().cpu().numpy()
    assert np.isfinite(got).all(), f"{name}: non-finite"
    scale = max(1.0, float(np.abs(ref).max()))
    err = float(np.abs(got - ref).max())
    print(f"{name}: max|d|={err:.3e} ref max={scale:.3e}", flush=True)
    assert err <= GRAD_TOL * scale, (name, err, scale)


def _run_bwd(seed, B, Hq, Hkv, Sq, Skv, D, Dv, kind, cap=None, dense=None, **mk):
    q, k, v = synthetic.make_qkv(seed, B, Hq, Hkv, Sq, Skv, D, Dv)
    g = torch.Generator().manual_seed(seed + 1000)
    do = torch.randn((B, Hq, Sq, Dv), generator=g).to(torch.bfloat16)
    mi = make_mask_info(kind, Sq, Skv, dense=dense, **mk)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    out, lse = splash_fwd(qd, kd, vd, mi, logits_soft_cap=cap)
    nan = float("nan")
    dq, dk, dv = torch.full_like(qd, nan), torch.full_like(kd, nan), torch.full_like(vd, nan)
    splash_bwd(qd, kd, vd, out, lse, dod, mi, logits_soft_cap=cap, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    fn = mask_rows_fn(kind, Skv, dense=dense, **mk)
    ref = oatt.attention_bwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy(), fn,
                             soft_cap=cap)
    return (dq, dk, dv), ref


BWD_CASES = [
    # name, seed, B, Hq, Hkv, Sq, Skv, D, Dv, mask kwargs, cap
    ("d96_causal_gqa", 260, 1, 4, 2, 640, 640, 96, 96, dict(kind="causal"), None),
    ("d32_local_cap", 261, 1, 2, 1, 512, 512, 32, 32, dict(kind="local", left=200, right=50), 3.0),
    ("d128_dv64_chunked", 262, 1, 2, 2, 768, 768, 128, 64, dict(kind="chunked", chunk=300), None),
    ("d48_dv112_rect", 263, 1, 2, 2, 256, 640, 48, 112, dict(kind="causal"), None),
    ("d64_dv16_rect", 264, 1, 2, 1, 640, 256, 64, 16, dict(kind="causal"), 4.0),
    # more dQ workgroups (2 x 32 x 5 = 320) than compute units: the
    # 128-column dQ kernel streams 64-key half tiles
    ("d80_half_tiles_cap", 265, 2, 32, 8, 640, 640, 80, 80, dict(kind="causal"), 5.0),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_padded_head_dims_bwd(case):
    name, seed, B, Hq, Hkv, Sq, Skv, D, Dv, mk, cap = case
    got, ref = _run_bwd(seed, B, Hq, Hkv, Sq, Skv, D, Dv, cap=cap, **mk)
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
        _grad_check(f"{name}.{nm}", g_, r_)


@pytest.mark.parametrize("D,Dv", [(48, 32), (112, 96)])
def test_padded_head_dims_bwd_dense(D, Dv):
    """Dense masks in both padded backward kernels: a full block, an empty
    block, a row with no allowed key (zero dq) and keys no query sees (zero
    dk, dv)."""
    rng = np.random.default_rng(270 + D)
    dense = synthetic.random_dense_mask(rng, 1, 512, 640, 0.2, force_diagonal=True)
    dense[:, 0:128, 128:256] = True
    dense[:, 128:256, 0:128] = False
    dense[:, 7, :] = False
    dense[:, :, 600:] = False
    got, ref = _run_bwd(271 + D, 1, 2, 1, 512, 640, D, Dv, "dense", dense=dense)
    for nm, g_, r_ in zip(("dq", "dk", "dv"), got, ref):
        _grad_check(f"dense D={D} Dv={Dv}.{nm}", g_, r_)
    assert (got[0][:, :, 7] == 0).all()
    assert (got[1][:, :, 600:] == 0).all() and (got[2][:, :, 600:] == 0).all()


def test_padded_head_dims_autograd():
    """splash_attention (the autograd wrapper) at D = 96, Dv = 64 against the
    oracle's gradients."""
    from block_sparse_attention_make_amd import splash_attention
    q, k, v = synthetic.make_qkv(280, 1, 2, 2, 384, 384, 96, 64)
    mi = make_mask_info("causal", 384, 384)
    g = torch.Generator().manual_seed(281)
    do = torch.randn((1, 2, 384, 64), generator=g).to(torch.bfloat16)
    qd, kd, vd = (t.to(DEV).requires_grad_() for t in (q, k, v))
    o = splash_attention(qd, kd, vd, mi)
    o.backward(do.to(DEV))
    torch.cuda.synchronize()
    fn = mask_rows_fn("causal", 384)
    ref = oatt.attention_bwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy(), fn)
    for nm, g_, r_ in zip(("dq", "dk", "dv"), (qd.grad, kd.grad, vd.grad), ref):
        _grad_check(f"autograd.{nm}", g_, r_)
