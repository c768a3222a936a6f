"""GPU parity of MaskInfos with mask blocks larger than 128 x 128 (the
EasyDeL example uses 256 x 512): the kernels walk such a MaskInfo as 128 x 128
sub-blocks with the parent block's label, so the result is the same masked
attention, forward and backward."""
import numpy as np
import pytest
import torch

from block_sparse_attention_make_amd import make_mask_info, splash_bwd, splash_fwd, synthetic
from oracle import attention as oatt
from tests.gpu_cases import TOL, compare, mask_rows_fn

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    # name, seed, Hq, Hkv, S, D, dtype, mask kwargs, cap, bq, bk
    ("causal_256x512", 141, 4, 2, 1024, 128, torch.bfloat16, dict(kind="causal"), None, 256, 512),
    ("local_512x128_cap", 142, 2, 2, 1024, 128, torch.bfloat16, dict(kind="local", left=300, right=20), 5.0, 512, 128),
    ("chunked_128x256", 143, 4, 1, 1024, 64, torch.bfloat16, dict(kind="chunked", chunk=300), None, 128, 256),
    ("causal_f32_256x256", 144, 2, 2, 512, 64, torch.float32, dict(kind="causal"), None, 256, 256),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_coarse_block_forward(case):
    name, seed, Hq, Hkv, S, D, dt, mk, cap, bq, bk = case
    q, k, v = synthetic.make_qkv(seed, 1, Hq, Hkv, S, S, D, D, dtype=dt)
    mi = make_mask_info(mk["kind"], S, S, block_q=bq, block_kv=bk, **{a: b for a, b in mk.items() if a != "kind"})
    o, l = splash_fwd(q.to(DEV), k.to(DEV), v.to(DEV), mi, logits_soft_cap=cap)
    torch.cuda.synchronize()
    fn = mask_rows_fn(mk["kind"], S, **{a: b for a, b in mk.items() if a != "kind"})
    o_ref, l_ref = oatt.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), fn, soft_cap=cap)
    compare(o.float().cpu().numpy(), l.cpu().numpy(), o_ref, l_ref, TOL[dt], name)


def test_coarse_block_dense_forward_and_backward():
    rng = np.random.default_rng(145)
    S = 1024
    dense = synthetic.random_dense_mask(rng, 1, S, S, 0.15, force_diagonal=True)
    dense[:, 0:256, 512:1024] = False          # an empty 256 x 512 block
    dense[:, 512:768, 0:512] = True            # a full one
    q, k, v = synthetic.make_qkv(146, 1, 2, 1, S, S, 128, 128)
    mi = make_mask_info("dense", S, S, dense=dense, block_q=256, block_kv=512)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, l = splash_fwd(qd, kd, vd, mi)
    g = torch.Generator().manual_seed(147)
    do = torch.randn(o.shape, generator=g).to(torch.bfloat16)
    dq, dk, dv = splash_bwd(qd, kd, vd, o, l, do.to(DEV), mi)
    torch.cuda.synchronize()
    fn = mask_rows_fn("dense", S, dense=dense)
    o_ref, l_ref = oatt.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), fn)
    compare(o.float().cpu().numpy(), l.cpu().numpy(), o_ref, l_ref, TOL[torch.bfloat16], "dense_256x512")
    refs = oatt.attention_bwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), do.double().numpy(), fn)
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        err = float(np.abs(got.float().cpu().numpy() - ref).max())
        scale = max(1.0, float(np.abs(ref).max()))
        print(f"dense_256x512.{name}: max|d|={err:.3e} scale={scale:.3e}", flush=True)
        assert err <= 2e-2 * scale, (name, err, scale)
