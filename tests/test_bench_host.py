"""Host-side pieces of bench.py, on the CPU: the work it counts per launch
(blocks and FLOPs on computed blocks) against the counts that follow from the
workloads' masks block by block (the oracle's block classification), the
one-GPU guard, and the rule that a committed traffic figure is used only for
the kernel source it was measured on."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from block_sparse_attention_make_amd import make_mask_info, synthetic
from oracle import mask_info as omi
from oracle import masks as omasks

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Computed 128 x 128 blocks over all (b, h) and the FLOPs on them
# (2 * 128 * 128 * (D + Dv) per block) for the five measured workloads.
EXPECTED = {
    "tiny_causal_f32": (20, 83_886_080),
    "causal_mha_8k": (33_280, 279_172_874_240),
    "local_gqa_8k": (17_280, 144_955_146_240),
    "chunked_gqa_16k_cap": (34_816, 292_057_776_128),
    "random_dense_2k": (2_048, 17_179_869_184),
    "causal_d96_8k": (33_280, 209_379_655_680),     # causal blocks at D = Dv = 96
}


def _mask_info(w):
    dense = None
    if w.mask.kind == "dense":
        _, _, _, dense = synthetic.make_inputs(w)
    m = w.mask
    return make_mask_info(m.kind, w.Sq, w.Skv, left=m.left, right=m.right, chunk=m.chunk, dense=dense), dense


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_computed_work_matches_block_counts(name):
    w = synthetic.WORKLOADS[name]
    mi, dense = _mask_info(w)
    work = bench.computed_work(w, mi.block_mask)
    # the same count from the oracle's own classification of the whole mask
    full = omasks.materialize(w.mask.kind, w.Sq, w.Skv, left=w.mask.left, right=w.mask.right,
                              chunk=w.mask.chunk, dense=dense)
    labels = omi.classify_fast(full, 128, 128)
    per_head = int((labels > 0).sum()) * (w.Hq if labels.shape[0] == 1 else 1) * w.B
    assert work["blocks_computed"] == per_head == EXPECTED[name][0]
    assert work["flops"] == work["flops_exec"] == EXPECTED[name][1]
    assert work["flops"] == work["blocks_computed"] * 2 * 128 * 128 * (w.D + w.Dv)
    assert work["blocks_total"] == w.B * w.Hq * (w.Sq // 128) * (w.Skv // 128)
    assert work["flops_dense"] == w.B * w.Hq * w.Sq * w.Skv * 2 * (w.D + w.Dv)


def test_backward_counts_five_products_and_executes_seven():
    w = synthetic.WORKLOADS["causal_mha_8k"]
    mi, _ = _mask_info(w)
    work = bench.computed_work(w, mi.block_mask, backward=True)
    per_product = 2 * 128 * 128 * w.D
    assert work["flops"] == 33_280 * 5 * per_product
    assert work["flops_exec"] == 33_280 * 7 * per_product


def test_coarse_blocks_count_every_sub_block():
    """256 x 512 mask blocks: each non-empty block is 8 computed 128 x 128
    sub-blocks, so causal 8k computes more blocks than at 128 x 128."""
    w = synthetic.WORKLOADS["causal_mha_8k"]
    mi = make_mask_info("causal", w.Sq, w.Skv, block_q=256, block_kv=512)
    work = bench.computed_work(w, mi.block_mask, 256, 512)
    coarse = int((mi.block_mask > 0).sum())
    assert work["blocks_computed"] == coarse * 8 * w.Hq
    assert work["blocks_computed"] > 33_280


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_traffic_only_for_the_measured_source(tmp_path):
    other = tmp_path / "other.hip"
    other.write_text("// not the kernel the profile was taken on\n")
    assert bench.measured_traffic("causal_mha_8k", src=str(other)) is None
    assert bench.measured_traffic("no_such_workload") is None
    got = bench.measured_traffic("causal_mha_8k")
    assert got is None or got > 0


def test_per_head_masks_count_each_head_once():
    """A MaskInfo with one mask per query head (Hm = Hq): each head's own
    non-empty blocks are counted once, not multiplied by the head count."""
    import dataclasses
    w = dataclasses.replace(synthetic.WORKLOADS["random_dense_2k"], Hq=2, Hkv=2, Sq=512, Skv=512)
    rng = np.random.default_rng(11)
    dense = rng.random((2, 512, 512)) < 0.1
    dense[0, :, 256:] = False                  # head 0: the right half of the keys is empty
    mi = make_mask_info("dense", 512, 512, dense=dense)
    work = bench.computed_work(w, mi.block_mask)
    labels = omi.classify_fast(dense, 128, 128)
    assert labels.shape[0] == 2
    assert work["blocks_computed"] == int((labels > 0).sum()) == 16 + 8
