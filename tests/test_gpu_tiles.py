"""GPU parity of the workgroup shapes of splash_fwd_tiled: two query heads of
a GQA group per workgroup (four waves sharing every K/V stage) against the
fp64 oracle, and bit for bit against one head per workgroup (each row's
arithmetic is the same in both shapes).  Covers causal, local and chunked
masks with a soft cap, group sizes 2 and 4, a rectangular grid, key splits
and attention sinks."""
import numpy as np
import pytest
import torch

from block_sparse_attention_make_amd import make_mask_info, splash_fwd, synthetic
from tests.gpu_cases import TOL, compare, oracle_by_block_rows, oracle_full

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    # name, seed, B, Hq, Hkv, Sq, Skv, mask kwargs, cap, splits
    ("causal_g2", 501, 2, 4, 2, 640, 640, dict(kind="causal"), None, 1),
    ("local_g4", 502, 1, 8, 2, 1024, 1024, dict(kind="local", left=300, right=40), None, 1),
    ("chunked_cap_g4", 503, 1, 4, 1, 1536, 1536, dict(kind="chunked", chunk=640), 30.0, 1),
    ("rect_causal_g2", 504, 1, 4, 2, 512, 1664, dict(kind="causal"), None, 1),
    ("local_g2_splits", 505, 1, 4, 2, 768, 768, dict(kind="local", left=200, right=0), None, 3),
]


def _run(q, k, v, mk, cap, splits, heads, aux=None):
    Sq, Skv = q.shape[2], k.shape[2]
    mi = make_mask_info(mk["kind"], Sq, Skv, left=mk.get("left"), right=mk.get("right"), chunk=mk.get("chunk"))
    out = torch.full(q.shape[:3] + (v.shape[3],), float("nan"), dtype=q.dtype, device=DEV)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    auxd = None if aux is None else torch.as_tensor(aux).to(DEV)
    splash_fwd(q.to(DEV), k.to(DEV), v.to(DEV), mi, logits_soft_cap=cap, out=out, lse=lse, kv_splits=splits,
               heads_per_workgroup=heads, softmax_aux=auxd)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_head_pairs_parity(case):
    name, seed, B, Hq, Hkv, Sq, Skv, mk, cap, splits = case
    q, k, v = synthetic.make_qkv(seed, B, Hq, Hkv, Sq, Skv, 128, 128)
    o2, l2 = _run(q, k, v, mk, cap, splits, heads=2)
    o_ref, l_ref = oracle_by_block_rows(q, k, v, cap=cap, **mk)
    compare(o2.float().numpy(), l2.numpy(), o_ref, l_ref, TOL[torch.bfloat16], f"{name} two heads per workgroup")
    o1, l1 = _run(q, k, v, mk, cap, splits, heads=1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{name}: one and two heads per workgroup differ"


def test_head_pairs_with_sinks():
    """Sinks per kv head: each wave adds its own head's row (the pair shares
    the kv head, so both read the same row)."""
    q, k, v = synthetic.make_qkv(506, 1, 4, 2, 512, 512, 128, 128)
    aux = (np.random.default_rng(507).standard_normal((2, 2)) * 2.0).astype(np.float32)
    mk = dict(kind="causal")
    o2, l2 = _run(q, k, v, mk, None, 1, heads=2, aux=aux)
    o_ref, l_ref = oracle_full(q, k, v, aux=aux, **mk)
    compare(o2.float().numpy(), l2.numpy(), o_ref, l_ref, TOL[torch.bfloat16], "sinks, two heads per workgroup")
    o1, l1 = _run(q, k, v, mk, None, 1, heads=1, aux=aux)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
