"""The allocation-free decode entry point, splash_decode_static, called
through the raw C ABI: it must give exactly what splash_decode gives with a
caller workspace (same kernels, same key ranges), on two calls in a row, the
second smaller than the first, while the device's free memory does not move
(the call allocates nothing; its scratch is the library's static array)."""
import ctypes

import pytest
import torch

from block_sparse_attention_make_amd import splash, synthetic

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _raw_static(lib, q, k, v, out, lse, cap):
    B, Hq, _, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    return lib.splash_decode_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                    B, Hq, Hkv, Skv, D, D, splash.BF16, float("nan"), cap,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_static_decode_equals_workspace_decode_on_two_calls():
    lib = splash.load_library()
    dev = torch.device("cuda:0")
    # (B, Hq, Hkv, Skv, D, soft cap): the second call is smaller in every size
    shapes = [(4, 32, 8, 20000, 128, None), (2, 8, 4, 3001, 64, 30.0)]
    cases = []
    for seed, (B, Hq, Hkv, Skv, D, cap) in enumerate(shapes):
        q, k, v = (t.to(dev) for t in synthetic.make_qkv(900 + seed, B, Hq, Hkv, 1, Skv, D, D))
        ref_o, ref_l = splash.splash_decode(q, k, v, logits_soft_cap=cap)
        out = torch.full((B, Hq, 1, D), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
        cases.append((q, k, v, cap, ref_o, ref_l, out, lse))
    torch.cuda.synchronize()
    # Free device memory is read around the static calls only; the comparisons
    # (torch ops that may reserve memory in torch's caching allocator) come after.
    free_before = torch.cuda.mem_get_info(dev)[0]
    for i, (q, k, v, cap, ref_o, ref_l, out, lse) in enumerate(cases):
        print(f"static decode call {i}: q {tuple(q.shape)} k {tuple(k.shape)} cap {cap}", flush=True)
        st = _raw_static(lib, q, k, v, out, lse, 0.0 if cap is None else cap)
        assert st == splash.OK, lib.splash_last_error().decode()
        torch.cuda.synchronize()
    free_after = torch.cuda.mem_get_info(dev)[0]
    for i, (q, k, v, cap, ref_o, ref_l, out, lse) in enumerate(cases):
        assert torch.equal(out, ref_o), f"call {i}: out differs from splash_decode"
        assert torch.equal(lse, ref_l), f"call {i}: lse differs from splash_decode"
    assert free_after == free_before, "device free memory moved across the static calls"


def test_static_decode_binding_and_repeat():
    """The Python binding, and the first shape again after the smaller one:
    the shared scratch keeps the previous call's partials, which must not
    leak into the next result."""
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in synthetic.make_qkv(910, 3, 16, 4, 1, 9000, 128, 128))
    ref = splash.splash_decode(q, k, v)
    q2, k2, v2 = (t.to(dev) for t in synthetic.make_qkv(911, 1, 4, 4, 1, 700, 128, 128))
    ref2 = splash.splash_decode(q2, k2, v2)
    a = splash.splash_decode_static(q, k, v)
    b = splash.splash_decode_static(q2, k2, v2)
    c = splash.splash_decode_static(q, k, v)
    torch.cuda.synchronize()
    for got, want in ((a, ref), (b, ref2), (c, ref)):
        assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1])
