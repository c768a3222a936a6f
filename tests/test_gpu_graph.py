"""The forward captured into a HIP graph: every replay, with the program's own
eager launches and synchronisations between replays, gives the eager result
bit for bit.  Covers a causal GQA forward (two heads per workgroup), a
dense forward with split keys (forward kernel plus merge in one graph) and
padded head dims with both launch shapes."""
import pytest
import torch

from block_sparse_attention_make_amd import make_mask_info, splash_fwd, synthetic

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(name):
    if name == "causal_pairs":
        q, k, v = synthetic.make_qkv(601, 1, 8, 2, 1024, 1024, 128, 128)
        mi = make_mask_info("causal", 1024, 1024)
        return q, k, v, mi, dict(heads_per_workgroup=2, kv_splits=1)
    if name == "padded_pairs_splits":   # head dims run zero-padded: D = 96, Dv = 80
        q, k, v = synthetic.make_qkv(604, 1, 8, 2, 1024, 1024, 96, 80)
        mi = make_mask_info("causal", 1024, 1024)
        return q, k, v, mi, dict(heads_per_workgroup=2, kv_splits=2)
    rng = __import__("numpy").random.default_rng(602)
    q, k, v = synthetic.make_qkv(603, 1, 4, 4, 768, 768, 128, 128)
    dense = synthetic.random_dense_mask(rng, 1, 768, 768, 0.2)
    mi = make_mask_info("dense", 768, 768, dense=dense)
    return q, k, v, mi, dict(kv_splits=3)


@pytest.mark.parametrize("name", ["causal_pairs", "dense_splits", "padded_pairs_splits"])
def test_graph_replays_match_eager(name):
    q, k, v, mi, kw = _case(name)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    Dv = v.shape[3]
    out = torch.empty(q.shape[:3] + (Dv,), dtype=q.dtype, device=DEV)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    ws = None
    if kw["kv_splits"] > 1:
        ws = torch.empty(kw["kv_splits"] * q.shape[0] * q.shape[1] * q.shape[2] * (2 * Dv + 4) // 4,
                         dtype=torch.float32, device=DEV)
    # eager reference (also uploads the MaskInfo and its split table: no
    # allocation happens inside the capture)
    splash_fwd(qd, kd, vd, mi, out=out, lse=lse, workspace=ws, **kw)
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
        splash_fwd(qd, kd, vd, mi, out=out, lse=lse, workspace=ws, stream=torch.cuda.current_stream(), **kw)
    torch.cuda.synchronize()
    other = torch.empty_like(out)
    for rep in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"{name}: replay {rep} differs from eager"
        # eager work between replays: another forward into other buffers
        splash_fwd(kd[:, :1].repeat(1, q.shape[1], 1, 1).contiguous(), kd, vd, mi, out=other, workspace=ws,
                   **kw)
        torch.cuda.synchronize()
