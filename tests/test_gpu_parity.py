"""GPU parity: the HIP path against the fp64 oracle, element by element.

Small cases span several 128-blocks with odd block counts, every mask kind,
GQA / MQA, the soft cap, both dtypes and head dims, Sq != Skv, per-head dense
masks and fully masked rows.  Tolerances: max-abs 2e-2 (bf16) and 1e-5
(float32) on out and lse.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_make_amd import synthetic
from tests.gpu_cases import TOL, compare, oracle_full, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


SMALL = [
    # name, seed, B, Hq, Hkv, Sq, Skv, D, dtype, mask kwargs, cap
    ("causal_5blk_gqa", 11, 2, 4, 2, 640, 640, 128, torch.bfloat16, dict(kind="causal"), None),
    ("causal_mqa", 12, 1, 3, 1, 384, 384, 128, torch.bfloat16, dict(kind="causal"), None),
    ("local_200_50", 13, 1, 4, 4, 768, 768, 128, torch.bfloat16, dict(kind="local", left=200, right=50), None),
    ("local_right_only", 14, 1, 2, 2, 512, 512, 128, torch.bfloat16, dict(kind="local", left=None, right=100), None),
    ("chunked_300_cap", 15, 1, 4, 2, 1024, 1024, 128, torch.bfloat16, dict(kind="chunked", chunk=300), 5.0),
    ("chunked_256", 16, 2, 2, 2, 896, 896, 128, torch.bfloat16, dict(kind="chunked", chunk=256), None),
    ("causal_rect_sq_lt_skv", 17, 1, 2, 2, 256, 640, 128, torch.bfloat16, dict(kind="causal"), None),
    ("causal_rect_sq_gt_skv", 18, 1, 2, 2, 640, 256, 128, torch.bfloat16, dict(kind="causal"), None),
    ("causal_d64_bf16", 19, 1, 4, 2, 512, 512, 64, torch.bfloat16, dict(kind="causal"), None),
    ("causal_d128_f32", 20, 1, 2, 1, 384, 384, 128, torch.float32, dict(kind="causal"), None),
    ("local_d64_f32_cap", 21, 1, 2, 2, 512, 512, 64, torch.float32, dict(kind="local", left=130, right=3), 4.0),
    ("one_block", 22, 1, 1, 1, 128, 128, 128, torch.bfloat16, dict(kind="causal"), None),
    ("cap_only_full", 23, 1, 2, 2, 256, 256, 128, torch.bfloat16, dict(kind="local", left=None, right=None), 2.0),
]


@pytest.mark.parametrize("splits", [1, "auto"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_parity(case, splits):
    """Each case with one workgroup per block row, and with the library's
    key-split plan (these small grids split up to 8 ways; float32 never)."""
    name, seed, B, Hq, Hkv, Sq, Skv, D, dt, mk, cap = case
    q, k, v = synthetic.make_qkv(seed, B, Hq, Hkv, Sq, Skv, D, D, dtype=dt)
    o, l, _ = run_gpu(q, k, v, cap=cap, kv_splits=splits, **mk)
    o_ref, l_ref = oracle_full(q, k, v, cap=cap, **mk)
    compare(o, l, o_ref, l_ref, TOL[dt], f"{name} splits={splits}")


@pytest.mark.parametrize("hm", [1, 4])
def test_dense_random_small(hm):
    rng = np.random.default_rng(30 + hm)
    q, k, v = synthetic.make_qkv(31, 1, 4, 2, 512, 640, 128, 128)
    dense = synthetic.random_dense_mask(rng, hm, 512, 640, 0.2, force_diagonal=True)
    # plant an all-ones block, an all-zeros block and a repeated block
    dense[:, 0:128, 128:256] = True
    dense[:, 128:256, 0:128] = False
    dense[:, 384:512, 512:640] = dense[:, 256:384, 384:512]
    o, l, mi = run_gpu(q, k, v, "dense", dense=dense)
    o_ref, l_ref = oracle_full(q, k, v, "dense", dense=dense)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], f"dense_hm{hm}")


def test_fully_masked_rows_give_zero_and_neg_inf():
    q, k, v = synthetic.make_qkv(40, 1, 2, 2, 256, 384, 128, 128)
    dense = np.ones((1, 256, 384), dtype=bool)
    dense[0, 5] = False                    # one empty row inside a partial block
    dense[0, 128:256, :] = False           # a whole empty block row (label 0 everywhere)
    o, l, _ = run_gpu(q, k, v, "dense", dense=dense)
    o_ref, l_ref = oracle_full(q, k, v, "dense", dense=dense)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], "masked_rows")
    assert (o[:, :, 128:256] == 0).all() and (l[:, :, 128:256] == -np.inf).all()
    assert (o[:, :, 5] == 0).all() and (l[:, :, 5] == -np.inf).all()


def test_tiny_causal_f32_workload_full():
    w = synthetic.WORKLOADS["tiny_causal_f32"]
    q, k, v, _ = synthetic.make_inputs(w)
    o, l, mi = run_gpu(q, k, v, "causal")
    o_ref, l_ref = oracle_full(q, k, v, "causal")
    compare(o, l, o_ref, l_ref, TOL[torch.float32], w.name)
    assert int((mi.block_mask == 0).sum()) == 6


def test_random_dense_workload_full():
    w = synthetic.WORKLOADS["random_dense_2k"]
    q, k, v, dense = synthetic.make_inputs(w)
    o, l, _ = run_gpu(q, k, v, "dense", dense=dense)
    o_ref, l_ref = oracle_full(q, k, v, "dense", dense=dense)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], w.name)


def test_explicit_scale_and_no_lse():
    from block_sparse_attention_make_amd import make_mask_info, splash_fwd
    q, k, v = synthetic.make_qkv(50, 1, 2, 2, 256, 256, 128, 128)
    dev = torch.device("cuda:0")
    mi = make_mask_info("causal", 256, 256)
    out, lse = splash_fwd(q.to(dev), k.to(dev), v.to(dev), mi, softmax_scale=0.05, return_lse=False)
    torch.cuda.synchronize()
    assert lse is None
    o_ref, _ = oracle_full(q, k, v, "causal", scale=0.05)
    assert float(np.abs(out.float().cpu().numpy() - o_ref).max()) <= 2e-2


def test_repeat_calls_are_bitwise_identical():
    q, k, v = synthetic.make_qkv(60, 1, 4, 4, 512, 512, 128, 128)
    a = run_gpu(q, k, v, "local", left=300, right=0)
    b = run_gpu(q, k, v, "local", left=300, right=0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _growing_scores(seed, B, H, S, D, a=31.0, b=31.0):
    """q_i = a e0 (+ small noise), k_j = b (j / S) e0 (+ small noise): every
    row's scores grow along the keys, so late rows end up more than 2^64 above
    the max of their first allowed keys -- the kernel must fall back to its
    exact-max recompute for them, while early rows stay on the fast path with
    exponentials far above 1."""
    q, k, v = synthetic.make_qkv(seed, B, H, H, S, S, D, D)
    t = torch.arange(S, dtype=torch.float32) / S
    q = (0.05 * q.float()).clone()
    k = (0.05 * k.float()).clone()
    q[..., 0] += a
    k[..., 0] += b * t
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v


@pytest.mark.parametrize("kind,kw,cap", [
    ("causal", {}, None),
    ("local", dict(left=300, right=40), None),
    ("chunked", dict(chunk=384), 30.0),
])
def test_scores_outgrowing_first_block_base(kind, kw, cap):
    q, k, v = _growing_scores(70, 1, 2, 768, 128)
    o, l, _ = run_gpu(q, k, v, kind, cap=cap, **kw)
    o_ref, l_ref = oracle_full(q, k, v, kind, cap=cap, **kw)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], f"growing_{kind}")


def test_large_logits_along_one_direction():
    """Logits up to about 74 along one dominant query/key direction: the scale
    must be applied to the float scores.  Rounding q * scale to bf16 first (an
    error of up to 2^-8 of each logit, which one dominant direction does not
    average away; here 29 * scale rounds 0.14% off) would put the lse about 0.1
    off."""
    q, k, v = _growing_scores(72, 1, 2, 512, 128, a=29.0, b=29.0)
    o, l, _ = run_gpu(q, k, v, "causal")
    o_ref, l_ref = oracle_full(q, k, v, "causal")
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], "large_logits_causal")


def test_scores_outgrowing_base_dense_mask():
    q, k, v = _growing_scores(71, 1, 2, 512, 128)
    rng = np.random.default_rng(72)
    dense = synthetic.random_dense_mask(rng, 1, 512, 512, 0.3, force_diagonal=True)
    o, l, _ = run_gpu(q, k, v, "dense", dense=dense)
    o_ref, l_ref = oracle_full(q, k, v, "dense", dense=dense)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], "growing_dense")


@pytest.mark.parametrize("kind,kw,cap,a", [
    ("causal", {}, None, 31.0),
    ("local", dict(left=None, right=None), None, 36.0),
    ("chunked", dict(chunk=640), 30.0, 31.0),
])
def test_scores_growing_far_past_the_base_over_many_blocks(kind, kw, cap, a):
    """Logits that grow along 2,048 keys to about a^2 / sqrt(D) (74 to 102
    nats): the kernel's exponent base has to move up several times inside
    each long row (the in-loop rescale), whole output against the oracle."""
    q, k, v = _growing_scores(73, 1, 2, 2048, 128, a=a, b=a)
    o, l, _ = run_gpu(q, k, v, kind, cap=cap, kv_splits=1, **kw)
    o_ref, l_ref = oracle_full(q, k, v, kind, cap=cap, **kw)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], f"growing_{kind}_{a}")
