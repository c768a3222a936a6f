"""The native (C++) mask compiler against the oracle, bit for bit (CPU).

dtype, shape and bytes of every MaskInfo array, and which arrays are None,
must be identical.  The native side labels computable masks in closed form
and never materialises them; the oracle materialises and applies any/all.
"""
import itertools

import numpy as np
import pytest

from oracle import mask_info as omi
from oracle import masks as omasks

splash = pytest.importorskip("block_sparse_attention_make_amd.splash")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    try:
        splash.load_library()
    except RuntimeError as e:
        pytest.fail(f"native library not built: {e}")


def assert_same(native, ref):
    for name in ("block_mask", "data_next", "mask_next", "partial_mask_blocks", "q_sequence"):
        a, b = getattr(native, name), getattr(ref, name)
        if b is None:
            assert a is None, name
            continue
        assert a is not None, name
        assert a.dtype == b.dtype, (name, a.dtype, b.dtype)
        assert a.shape == b.shape, (name, a.shape, b.shape)
        assert a.tobytes() == b.tobytes(), name


def _spec_kwargs(kind, kw):
    return {k: kw.get(k) for k in ("left", "right", "chunk") if k in kw}


@pytest.mark.parametrize("kind,kw", [
    ("causal", {}), ("local", {"left": 1024, "right": 0}), ("chunked", {"chunk": 2048}),
])
def test_page_workload_masks(kind, kw):
    seq = 16384 if kind == "chunked" else 8192
    nat = splash.make_mask_info(kind, seq, seq, **kw)
    m = omasks.materialize(kind, seq, seq, **kw)
    ref = omi.build(m, 128, 128, computable=True)
    assert_same(nat, ref)


def test_random_dense_workload():
    from block_sparse_attention_make_amd import synthetic
    w = synthetic.WORKLOADS["random_dense_2k"]
    _, _, _, dense = synthetic.make_inputs(w)
    nat = splash.make_mask_info("dense", 2048, 2048, dense=dense)
    ref = omi.build(dense, 128, 128, computable=False)
    assert_same(nat, ref)
    assert nat.partial_mask_blocks.nbytes == 4 * 1024 * 1024


def test_tiny_causal_workload():
    nat = splash.make_mask_info("causal", 512, 512)
    ref = omi.build(omasks.materialize("causal", 512, 512), 128, 128, computable=True)
    assert_same(nat, ref)
    # 6 of 16 blocks empty; after the shrink they survive only as row-end padding
    assert int((nat.block_mask == 0).sum()) == 6
    assert nat.block_mask.shape == (1, 4, 4)


@pytest.mark.parametrize("shrink,downcast", list(itertools.product([True, False], repeat=2)))
def test_computable_small_grid(shrink, downcast):
    cases = [("causal", {}), ("local", {"left": 3, "right": 1}), ("local", {"left": 0, "right": 0}),
             ("local", {"left": None, "right": 5}), ("local", {"left": 7, "right": None}),
             ("local", {"left": None, "right": None}), ("chunked", {"chunk": 3}),
             ("chunked", {"chunk": 4}), ("chunked", {"chunk": 100})]
    for kind, kw in cases:
        for sq, skv, bq, bk in [(8, 8, 2, 2), (12, 8, 4, 2), (6, 15, 3, 5), (16, 16, 4, 4), (9, 27, 3, 9)]:
            nat = splash.make_mask_info(kind, sq, skv, block_q=bq, block_kv=bk, shrink=shrink,
                                        downcast=downcast, **kw)
            ref = omi.build(omasks.materialize(kind, sq, skv, **kw), bq, bk, computable=True,
                            shrink=shrink, downcast=downcast)
            assert_same(nat, ref)


@pytest.mark.parametrize("shrink", [True, False])
def test_random_dense_small(shrink):
    rng = np.random.default_rng(3)
    for _ in range(150):
        hm, nq, nk = int(rng.integers(1, 4)), int(rng.integers(1, 6)), int(rng.integers(1, 7))
        bq, bk = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        p = float(rng.choice([0.0, 0.05, 0.5, 0.95, 1.0]))
        m = rng.random((hm, nq * bq, nk * bk)) < p
        if nq * nk > 1:
            m[:, :bq, :bk] = rng.random((bq, bk)) < 0.5
            m[:, -bq:, -bk:] = m[:, :bq, :bk]
        nat = splash.make_mask_info("dense", nq * bq, nk * bk, dense=m, block_q=bq, block_kv=bk, shrink=shrink)
        ref = omi.build(m, bq, bk, computable=False, shrink=shrink)
        assert_same(nat, ref)


def test_exhaustive_4x4_masks():
    for bits in itertools.product([0, 1], repeat=16):
        m = np.array(bits, dtype=bool).reshape(1, 4, 4)
        if sum(bits) % 5:          # a fifth of the 65,536 masks, spread over all counts
            continue
        nat = splash.make_mask_info("dense", 4, 4, dense=m, block_q=2, block_kv=2)
        assert_same(nat, omi.build(m, 2, 2, computable=False))


def test_dense_nonbinary_bytes_are_normalised():
    m = np.zeros((1, 4, 4), dtype=np.uint8)
    m[0, 0, 0] = 7
    m[0, 3, 3] = 255
    nat = splash.make_mask_info("dense", 4, 4, dense=m, block_q=2, block_kv=2)
    ref = omi.build(m != 0, 2, 2, computable=False)
    assert_same(nat, ref)
    assert set(np.unique(nat.partial_mask_blocks)) <= {0, 1}


def test_downcast_thresholds_match_oracle():
    for nk in (127, 128, 129, 32767, 32768, 32769):
        m = np.zeros((1, 1, nk), dtype=bool)
        m[0, 0, nk - 1] = True
        nat = splash.make_mask_info("dense", 1, nk, dense=m, block_q=1, block_kv=1)
        assert_same(nat, omi.build(m, 1, 1, computable=False))


def test_empty_and_degenerate():
    # all-empty dense mask, zero-length sequences
    m = np.zeros((2, 4, 6), dtype=bool)
    nat = splash.make_mask_info("dense", 4, 6, dense=m, block_q=2, block_kv=2)
    assert_same(nat, omi.build(m, 2, 2, computable=False))
    nat = splash.make_mask_info("causal", 0, 256)
    assert nat.block_mask.shape == (1, 0, 1)
    assert nat.q_sequence.shape == (0,)
    nat = splash.make_mask_info("causal", 256, 0)
    assert nat.block_mask.shape == (1, 2, 1) and not nat.block_mask.any()


@pytest.mark.parametrize("args,msg", [
    (dict(kind="causal", q_len=100, kv_len=128), "block_q"),
    (dict(kind="causal", q_len=128, kv_len=100), "block_kv"),
    (dict(kind="chunked", q_len=128, kv_len=128, chunk=0), "chunk"),
    (dict(kind="causal", q_len=-128, kv_len=128), "lengths"),
])
def test_invalid_masks_rejected(args, msg):
    with pytest.raises(splash.SplashError) as ei:
        splash.make_mask_info(**args)
    assert ei.value.status == splash.EINVAL
    assert msg in str(ei.value)


# ---- key-axis slices (the MaskInfo of one key/value shard) ----

@pytest.mark.parametrize("kind,kw", [
    ("causal", {}), ("local", {"left": 300, "right": 70}), ("local", {"left": None, "right": 10}),
    ("chunked", {"chunk": 200}),
])
@pytest.mark.parametrize("k0,kn", [(0, 384), (256, 512), (640, 256), (896, 0), (0, 1024)])
def test_kv_slice_equals_mask_of_the_slice(kind, kw, k0, kn):
    """The native slice labels computable masks in closed form at the slice's
    key offset; the oracle builds the MaskInfo of the materialised mask's
    columns [k0, k0 + kn).  They must agree byte for byte."""
    sq = skv = 1024 if kn else 1024
    nat = splash.make_mask_info(kind, sq, skv, kv_slice=(k0, kn), **kw)
    m = omasks.materialize(kind, sq, skv, **kw)[:, :, k0:k0 + kn]
    ref = omi.build(m, 128, 128, computable=True)
    assert_same(nat, ref)
    assert nat.kv_len == kn


@pytest.mark.parametrize("k0,kn", [(128, 256), (0, 128), (384, 256)])
def test_kv_slice_dense(k0, kn):
    rng = np.random.default_rng(7)
    dense = rng.random((2, 256, 640)) < 0.15
    dense[:, :, 130:140] = True
    nat = splash.make_mask_info("dense", 256, 640, dense=dense, kv_slice=(k0, kn))
    ref = omi.build(dense[:, :, k0:k0 + kn], 128, 128, computable=False)
    assert_same(nat, ref)


@pytest.mark.parametrize("k0,kn", [(-128, 256), (0, 1152), (64, 128), (128, 100), (1024, 128)])
def test_kv_slice_rejected(k0, kn):
    with pytest.raises(splash.SplashError) as e:
        splash.make_mask_info("causal", 1024, 1024, kv_slice=(k0, kn))
    assert e.value.status == splash.EINVAL


# ---- mask blocks larger than 128 x 128 (the EasyDeL example's 256 x 512) ----

@pytest.mark.parametrize("kind,kw", [("causal", {}), ("local", {"left": 700, "right": 0}),
                                     ("chunked", {"chunk": 1000})])
@pytest.mark.parametrize("bq,bk", [(256, 512), (512, 128), (128, 256)])
def test_coarse_blocks_match_oracle(kind, kw, bq, bk):
    nat = splash.make_mask_info(kind, 2048, 3072, block_q=bq, block_kv=bk, **kw)
    ref = omi.build(omasks.materialize(kind, 2048, 3072, **kw), bq, bk, computable=True)
    assert_same(nat, ref)
