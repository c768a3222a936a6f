"""GPU parity of the split-key forward (splash_fwd_split): each block row's
non-empty blocks divided over kv_splits workgroups whose results are merged
by their log-sum-exp.  Every case compares the whole output with the fp64
oracle (max-abs 2e-2 on out and lse, bf16), including splits that receive no
block, rows with no allowed key, attention sinks (added once, by the merge),
rows wider than one 256-slot metadata chunk, grids without shrinking and
mask blocks coarser than 128 x 128."""
import numpy as np
import pytest
import torch

from block_sparse_attention_make_amd import make_mask_info, splash_fwd, synthetic
from block_sparse_attention_make_amd.splash import plan_kv_splits
from tests.gpu_cases import TOL, compare, oracle_by_block_rows, oracle_full

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(q, k, v, mk, splits, cap=None, aux=None, mi_kw=None):
    mi = make_mask_info(mk["kind"], q.shape[2], k.shape[2], left=mk.get("left"), right=mk.get("right"),
                        chunk=mk.get("chunk"), dense=mk.get("dense"), **(mi_kw or {}))
    out = torch.full((q.shape[0], q.shape[1], q.shape[2], v.shape[3]), float("nan"), dtype=q.dtype, device=DEV)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    auxd = None if aux is None else torch.as_tensor(np.asarray(aux, dtype=np.float32)).to(DEV)
    out, lse = splash_fwd(q.to(DEV), k.to(DEV), v.to(DEV), mi, logits_soft_cap=cap, out=out, lse=lse,
                          softmax_aux=auxd, kv_splits=splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


CASES = [
    # name, seed, B, Hq, Hkv, Sq, Skv, mask kwargs, cap
    ("causal_gqa", 401, 2, 4, 2, 1024, 1024, dict(kind="causal"), None),
    ("local_window", 402, 1, 4, 4, 1536, 1536, dict(kind="local", left=300, right=40), None),
    ("chunked_cap", 403, 1, 4, 1, 2048, 2048, dict(kind="chunked", chunk=640), 30.0),
    ("rect_causal", 404, 1, 2, 2, 512, 1664, dict(kind="causal"), None),
]


@pytest.mark.parametrize("splits", [2, 3, 4, 8])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_parity(case, splits):
    name, seed, B, Hq, Hkv, Sq, Skv, mk, cap = case
    q, k, v = synthetic.make_qkv(seed, B, Hq, Hkv, Sq, Skv, 128, 128)
    o, l = _run(q, k, v, mk, splits, cap)
    o_ref, l_ref = oracle_by_block_rows(q, k, v, cap=cap, **mk)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], f"{name} splits={splits}")


@pytest.mark.parametrize("splits", [1, 3])
def test_split_head_dim_64(splits):
    """D = 64: half-width rows through the output staging and the merge."""
    q, k, v = synthetic.make_qkv(405, 1, 4, 2, 768, 768, 64, 64)
    mk = dict(kind="local", left=200, right=0)
    o, l = _run(q, k, v, mk, splits)
    o_ref, l_ref = oracle_by_block_rows(q, k, v, **mk)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], f"d64 splits={splits}")


@pytest.mark.parametrize("hm", [1, 4])
@pytest.mark.parametrize("splits", [2, 5])
def test_split_dense_with_empty_rows(hm, splits):
    rng = np.random.default_rng(410 + hm)
    Sq, Skv = 640, 1024
    dense = synthetic.random_dense_mask(rng, hm, Sq, Skv, 0.15, force_diagonal=True)
    dense[:, 9] = False                  # a row with no allowed key
    dense[:, 256:384] = False            # a whole empty block row: every split is empty
    dense[:, 0:128, 0:640] = False       # block row 0 keeps only its last three blocks
    q, k, v = synthetic.make_qkv(411, 1, 4, 2, Sq, Skv, 128, 128)
    mk = dict(kind="dense", dense=dense)
    o, l = _run(q, k, v, mk, splits)
    o_ref, l_ref = oracle_by_block_rows(q, k, v, **mk)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], f"dense hm={hm} splits={splits}")
    assert (o[:, :, 9] == 0).all() and (l[:, :, 9] == -np.inf).all()


@pytest.mark.parametrize("splits", [3, 8])
def test_split_more_splits_than_blocks(splits):
    """A 200-key window touches two or three key blocks per row: most splits
    get no block and must add nothing."""
    q, k, v = synthetic.make_qkv(420, 1, 2, 2, 1024, 1024, 128, 128)
    mk = dict(kind="local", left=100, right=100)
    o, l = _run(q, k, v, mk, splits)
    o_ref, l_ref = oracle_by_block_rows(q, k, v, **mk)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], f"few blocks splits={splits}")


@pytest.mark.parametrize("aux_rows", [1, 2, 4])
def test_split_with_sinks(aux_rows):
    q, k, v = synthetic.make_qkv(430, 1, 4, 2, 768, 768, 128, 128)
    rng = np.random.default_rng(431)
    aux = rng.standard_normal((aux_rows, 2)).astype(np.float32) * 2.0
    aux_arg = aux[0] if aux_rows == 1 else aux
    mk = dict(kind="causal")
    o, l = _run(q, k, v, mk, 4, aux=aux_arg)
    o_ref, l_ref = oracle_full(q, k, v, aux=aux_arg, **mk)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], f"sinks rows={aux_rows}")


def test_split_rows_wider_than_one_chunk_and_no_shrink():
    """300 key blocks per row divided in 3: every split range crosses a
    256-slot metadata chunk boundary or ends inside one; without shrinking,
    empty slots sit inside the ranges."""
    q, k, v = synthetic.make_qkv(440, 1, 2, 1, 256, 38400, 128, 128)
    mk = dict(kind="local", left=None, right=None)
    o, l = _run(q, k, v, mk, 3)
    o_ref, l_ref = oracle_by_block_rows(q, k, v, **mk)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], "300 blocks splits=3")
    q, k, v = synthetic.make_qkv(441, 1, 2, 2, 1536, 1536, 128, 128)
    mk = dict(kind="local", left=300, right=0)
    o, l = _run(q, k, v, mk, 2, mi_kw=dict(shrink=False))
    o_ref, l_ref = oracle_by_block_rows(q, k, v, **mk)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], "no shrink splits=2")


def test_split_coarse_blocks():
    q, k, v = synthetic.make_qkv(450, 1, 2, 2, 1024, 2048, 128, 128)
    mk = dict(kind="causal")
    o, l = _run(q, k, v, mk, 4, mi_kw=dict(block_q=256, block_kv=512))
    o_ref, l_ref = oracle_by_block_rows(q, k, v, **mk)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], "256x512 blocks splits=4")


def test_plan_fills_the_gpu():
    """The library's plan: one split when the grid already holds two
    workgroups per CU, enough splits to reach that otherwise."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    w = synthetic.WORKLOADS["random_dense_2k"]
    dense = synthetic.make_inputs(w)[3]
    mi = make_mask_info("dense", w.Sq, w.Skv, dense=dense)
    n_wg = w.B * w.Hq * (w.Sq // 128)
    assert plan_kv_splits(mi, w.B, w.Hq) == min(8, -(-2 * cus // n_wg))
    mi = make_mask_info("causal", 8192, 8192)
    assert plan_kv_splits(mi, 1, 16) == 1          # 1,024 workgroups
    assert plan_kv_splits(mi, 1, 1) == min(8, -(-2 * cus // 64))
