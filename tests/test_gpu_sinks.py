"""GPU parity of attention sinks (splash_fwd_sinks) against the fp64 oracle.

Sink logits are drawn in float32 and the same values go to both sides.
Covers both kernels (bf16 wide rows, float32), the three sink-row layouts
([ns], [Hkv, ns], [Hq, ns]), sinks far above and far below the scores, rows
with no allowed key, the exact-max recompute path, and the -inf identity.
"""
import numpy as np
import pytest
import torch

from block_sparse_attention_make_amd import synthetic
from tests.gpu_cases import TOL, compare, oracle_full, run_gpu
from tests.test_gpu_parity import _growing_scores

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    # name, seed, B, Hq, Hkv, S, D, dtype, mask kwargs, cap, aux shape, aux scale, aux offset
    ("causal_gqa_kvrows", 81, 1, 4, 2, 640, 128, torch.bfloat16, dict(kind="causal"), None, (2, 2), 2.0, 0.0),
    ("local_shared_high", 82, 1, 2, 2, 512, 128, torch.bfloat16, dict(kind="local", left=200, right=0), None,
     (1,), 1.0, 8.0),
    ("chunked_cap_qrows", 83, 1, 4, 2, 768, 128, torch.bfloat16, dict(kind="chunked", chunk=256), 5.0,
     (4, 3), 1.0, 0.0),
    ("causal_d64_low", 84, 1, 2, 1, 384, 64, torch.bfloat16, dict(kind="causal"), None, (1, 2), 1.0, -20.0),
    ("causal_f32_qrows", 85, 1, 2, 2, 384, 128, torch.float32, dict(kind="causal"), None, (2, 3), 1.0, 0.0),
    ("local_f32_d64_kvrows", 86, 1, 4, 2, 512, 64, torch.float32, dict(kind="local", left=100, right=30), 3.0,
     (2, 1), 1.0, 2.0),
]


def _aux(seed, shape, scale, offset):
    rng = np.random.default_rng(seed)
    return (offset + scale * rng.standard_normal(shape)).astype(np.float32)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sinks_parity(case):
    name, seed, B, Hq, Hkv, S, D, dt, mk, cap, shape, sc, off = case
    q, k, v = synthetic.make_qkv(seed, B, Hq, Hkv, S, S, D, D, dtype=dt)
    aux = _aux(seed, shape, sc, off)
    o, l, _ = run_gpu(q, k, v, cap=cap, aux=aux, **mk)
    o_ref, l_ref = oracle_full(q, k, v, cap=cap, aux=aux, **mk)
    compare(o, l, o_ref, l_ref, TOL[dt], name)


def test_sinks_minus_inf_equal_plain_forward():
    q, k, v = synthetic.make_qkv(87, 1, 2, 2, 512, 512, 128, 128)
    a = run_gpu(q, k, v, "causal")
    b = run_gpu(q, k, v, "causal", aux=np.full((2, 2), -np.inf, dtype=np.float32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_sinks_rows_without_allowed_keys():
    q, k, v = synthetic.make_qkv(88, 1, 2, 2, 256, 384, 128, 128)
    dense = np.ones((1, 256, 384), dtype=bool)
    dense[0, 5] = False
    dense[0, 128:256, :] = False
    aux = np.array([0.5, -1.0], dtype=np.float32)
    o, l, _ = run_gpu(q, k, v, "dense", dense=dense, aux=aux)
    o_ref, l_ref = oracle_full(q, k, v, "dense", dense=dense, aux=aux)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], "sinks_empty_rows")
    want = float(np.logaddexp(0.5, -1.0))
    assert (o[:, :, 128:256] == 0).all() and np.allclose(l[:, :, 128:256], want, atol=1e-6)
    assert (o[:, :, 5] == 0).all() and np.allclose(l[:, :, 5], want, atol=1e-6)


def test_sinks_with_exact_max_recompute():
    q, k, v = _growing_scores(89, 1, 2, 768, 128)
    aux = np.array([[3.0], [-2.0]], dtype=np.float32)
    o, l, _ = run_gpu(q, k, v, "causal", aux=aux)
    o_ref, l_ref = oracle_full(q, k, v, "causal", aux=aux)
    compare(o, l, o_ref, l_ref, TOL[torch.bfloat16], "sinks_growing")
