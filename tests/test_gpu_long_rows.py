"""GPU parity of the paths the standard workloads do not reach, each on its
whole output against the fp64 oracle:

  * block rows wider than one metadata chunk (more than 256 non-empty key
    blocks: causal beyond 32,768 keys, long key ranges with short query
    ranges), which also gives int16 data_next and, for dense masks, int16
    mask_next -- the long-context case splash attention is for (splash
    explainer, FAQ "What is MaskInfo in splash attention?": the integer
    arrays are downcast when their values fit);
  * MaskInfos compiled without grid shrinking (interior and whole-chunk
    label-0 slots stay in the grid; FAQ "What does grid shrinking do in splash
    attention?") or without downcasting (int32 arrays);
  * the exact-max recompute of the bf16 kernel on rows wider than one chunk.

Tolerances as everywhere: max-abs 2e-2 (bf16), 1e-5 (float32).
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_make_amd import synthetic
from tests.gpu_cases import TOL, compare, oracle_by_block_rows, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(name, q, k, v, mk, cap=None, expect=None, **mi_kw):
    o, l, mi = run_gpu(q, k, v, cap=cap, **mk, **mi_kw)
    if expect is not None:
        expect(mi)
    o_ref, l_ref = oracle_by_block_rows(q, k, v, cap=cap, **mk)
    compare(o, l, o_ref, l_ref, TOL[q.dtype], name)


def _wide(mi, width, dn=None, mn=None):
    bm = mi.block_mask
    assert bm.shape[-1] == width, bm.shape
    if dn is not None:
        assert mi.data_next.dtype == dn, mi.data_next.dtype
    if mn is not None:
        assert mi.mask_next.dtype == mn, mi.mask_next.dtype


LONG = [
    # name, seed, B, Hq, Hkv, Sq, Skv, D, dtype, mask kwargs, cap, grid width, data_next dtype
    ("causal_40k_bf16", 201, 1, 1, 1, 40960, 40960, 128, torch.bfloat16, dict(kind="causal"), None, 320,
     np.int16),
    ("causal_33k_f32_d64", 202, 1, 1, 1, 33024, 33024, 64, torch.float32, dict(kind="causal"), None, 258,
     np.int16),
    ("full_rows_40k_gqa", 203, 1, 4, 2, 256, 40960, 128, torch.bfloat16,
     dict(kind="local", left=None, right=None), None, 320, np.int16),
    ("local_33k_cap", 204, 1, 2, 1, 384, 33152, 128, torch.bfloat16,
     dict(kind="local", left=None, right=33000), 20.0, 259, np.int16),
]


@pytest.mark.parametrize("case", LONG, ids=[c[0] for c in LONG])
def test_rows_wider_than_one_metadata_chunk(case):
    name, seed, B, Hq, Hkv, Sq, Skv, D, dt, mk, cap, width, dn = case
    q, k, v = synthetic.make_qkv(seed, B, Hq, Hkv, Sq, Skv, D, D, dtype=dt)
    _check(name, q, k, v, mk, cap, expect=lambda mi: _wide(mi, width, dn))


@pytest.mark.parametrize("dt,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_dense_mask_wider_than_one_metadata_chunk(dt, D):
    """258 key blocks, all partial: two metadata chunks, int16 data_next and
    int16 mask_next (516 distinct partial blocks), one mask per head."""
    rng = np.random.default_rng(210)
    Sq, Skv = 256, 33024
    dense = synthetic.random_dense_mask(rng, 2, Sq, Skv, 0.3, force_diagonal=True)
    q, k, v = synthetic.make_qkv(211, 1, 2, 1, Sq, Skv, D, D, dtype=dt)
    _check(f"dense_258_blocks_{dt}", q, k, v, dict(kind="dense", dense=dense),
           expect=lambda mi: _wide(mi, 258, np.int16, np.int16))


@pytest.mark.parametrize("dt,D", [(torch.bfloat16, 128), (torch.float32, 128)])
def test_no_shrink_whole_empty_chunk(dt, D):
    """shrink off: every row keeps all 320 slots, so each row's few non-empty
    blocks sit between label-0 slots; rows whose window lies in the first 256
    slots see a second metadata chunk with nothing to run, and rows past
    block 256 a first chunk with nothing to run."""
    q, k, v = synthetic.make_qkv(220, 1, 2, 1, 40960, 40960, D, D, dtype=dt)
    mk = dict(kind="local", left=700, right=200)
    _check(f"local_no_shrink_{dt}", q, k, v, mk, expect=lambda mi: _wide(mi, 320), shrink=False)


@pytest.mark.parametrize("mk,cap", [
    (dict(kind="local", left=300, right=0), None),
    (dict(kind="chunked", chunk=384), 30.0),
    (dict(kind="causal"), None),
])
def test_no_shrink_interior_empty_slots(mk, cap):
    """shrink off at ordinary sizes: the grid keeps every key block, label 0
    included, and the kernel must still skip them."""
    q, k, v = synthetic.make_qkv(230, 1, 4, 2, 1536, 1536, 128, 128)
    _check(f"no_shrink_{mk['kind']}", q, k, v, mk, cap, expect=lambda mi: _wide(mi, 12), shrink=False)


@pytest.mark.parametrize("kind", ["local", "dense"])
def test_no_downcast(kind):
    """downcast off: every index array is int32."""
    q, k, v = synthetic.make_qkv(240, 1, 2, 2, 1024, 1024, 128, 128)
    if kind == "dense":
        rng = np.random.default_rng(241)
        dense = synthetic.random_dense_mask(rng, 1, 1024, 1024, 0.2, force_diagonal=True)
        mk = dict(kind="dense", dense=dense)
    else:
        mk = dict(kind="local", left=200, right=100)

    def expect(mi):
        assert mi.block_mask.dtype == np.int32 and mi.data_next.dtype == np.int32
        if kind == "dense":
            assert mi.mask_next.dtype == np.int32

    _check(f"no_downcast_{kind}", q, k, v, mk, expect=expect, downcast=False)
    _check(f"no_downcast_no_shrink_{kind}", q, k, v, mk, expect=expect, downcast=False, shrink=False)


def test_growing_scores_recompute_across_chunks():
    """Scores that grow along 33,024 keys by far more than 2^64 of exponent
    range: rows that fix an exponent base early must rescale or recompute,
    across both metadata chunks."""
    Sq, Skv = 256, 33024
    q, k, v = synthetic.make_qkv(250, 1, 2, 2, Sq, Skv, 128, 128)
    t = torch.arange(Skv, dtype=torch.float32) / Skv
    q = (0.05 * q.float()).clone()
    k = (0.05 * k.float()).clone()
    q[..., 0] += 31.0
    k[..., 0] += 31.0 * t
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    _check("growing_33k", q, k, v, dict(kind="local", left=None, right=None))
    _check("growing_33k_causal_window", q, k, v, dict(kind="local", left=20000, right=None))
