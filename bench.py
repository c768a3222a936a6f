"""Benchmark: splash-attention forward TFLOP/s on computed blocks (MI355X).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--sinks N] [--kv-shards P] [--backward] [--decode]
                    [--block-q BQ --block-kv BK]

A step is one splash_fwd call (the whole forward path: block walk over the
MaskInfo, K/V staging, QK^T, soft cap, masking, online softmax, PV, epilogue)
over one batch of the workload, with q/k/v resident in HBM and the MaskInfo
compiled and uploaded beforehand -- the mask compiler is a compile-time pass
(splash-attention explainer, "What is MaskInfo in splash attention?"), timed
separately and reported as mask_compile_ms.

FLOPs on computed blocks = sum over (b, h) of the non-empty grid positions x
2 * 128 * 128 * (D + Dv); softmax and masking work are not counted.  Prints
one JSON line.

Timing: --prewarm-s seconds of back-to-back steps (the clock settles), W
warm-up steps, then K steps back to back between one HIP event pair on the
launch stream, with a device synchronisation on both sides.  --graph
captures one forward step into a HIP graph and times its replays instead
("launch" in the JSON says which; replays measured slower than eager
launches on this stack).  value divides
the FLOPs by the host wall time per step; roofline.achieved divides them by
the event time per step.  kernel_ms_median / kernel_ms_min come from 20 more
steps timed one by one afterwards (an event between launches delays the next
launch by several microseconds, so the timed steps carry none).

--sinks N adds N attention-sink logits per key/value head (splash_fwd_sinks).
--kv-shards P splits the keys into P equal shards and times the per-device
part of ring attention instead: P splash_fwd calls on key-sliced MaskInfos
plus P - 1 lse merges into a float32 accumulator (the computed blocks, and so
the FLOPs, are the same).  It also times the merge kernel alone and reports
its HBM roofline under "merge".
--backward times splash_bwd instead (the forward runs once beforehand): a
step is the delta kernel, the key-major dK/dV kernel and the query-major dQ
kernel.  Its FLOPs are the usual backward count, 5 products of
2 * 128 * 128 * D per computed block (S recomputed, dP, dV, dQ, dK);
roofline.achieved counts the 7 products the two kernels execute (S and dP
are formed in both).
--block-q / --block-kv compile the workload's mask with larger blocks (the
EasyDeL example's 256 x 512); the kernels walk them as 128 x 128 sub-blocks, and
FLOPs count every sub-block of a non-empty block.
--decode times splash_decode on the decode workload (one query per head
against a 32k-key cache; --workload defaults to decode_gqa_32k) and reports
the K/V read bandwidth against HBM's 8 TB/s.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz (AMD: 2.5 PFLOP/s)
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "block_sparse_attention_make_amd", "csrc", "splash_fwd.hip")
DECODE_SRC = os.path.join(ROOT, "block_sparse_attention_make_amd", "csrc", "splash_decode.hip")


def kernel_sha(src=KERNEL_SRC):
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload, src=KERNEL_SRC):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current source of the kernel (src); else None."""
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_sha256") != kernel_sha(src):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def mfma_probe(torch):
    """bf16 MFMA TFLOP/s the GPU sustains (independent 32x32x16 chains, one
    wave per SIMD, 1.5 s warm each): `tflops` on constant operands (the
    matrix cores' ceiling at full clock) and `tflops_random_operands` on
    changing random bf16 operands, like an attention step's, which draw more
    power; None if the probe library is absent."""
    import ctypes
    path = os.path.join(ROOT, "block_sparse_attention_make_amd", "lib", "libsplash_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    props = torch.cuda.get_device_properties(0)
    blocks = props.multi_processor_count
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()

    def rate(fn, iters, mfma_per_iter):
        fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        t0 = time.time()
        while time.time() - t0 < 1.5:
            fn(blocks, iters, sink.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn(blocks, iters, sink.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
        b.record(stream)
        torch.cuda.synchronize()
        flops = blocks * 4 * iters * mfma_per_iter * 32768
        return round(flops / (a.elapsed_time(b) * 1e-3) / 1e12, 1)

    res = {"tflops": rate(lib.splash_probe_mfma, 20000, 4), "cus": blocks}
    if hasattr(lib, "splash_probe_mfma_random"):
        res["tflops_random_operands"] = rate(lib.splash_probe_mfma_random, 10000, 8)
    return res


def read_probe(torch, nbytes):
    """HBM read GB/s the GPU sustains on a plain streaming read of one
    nbytes device buffer (as many bytes as a memory-bound kernel streams per
    launch): 8 workgroups per CU, each reading one contiguous share with
    non-temporal loads; 1 s warm, median of 10 timed launches; None if the
    probe library is absent."""
    import ctypes
    import numpy as np
    path = os.path.join(ROOT, "block_sparse_attention_make_amd", "lib", "libsplash_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.splash_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p]
    blocks = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda:0")

    def one():
        if lib.splash_probe_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(),
                                 ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("read probe launch failed")

    t0 = time.time()
    while time.time() - t0 < 1.0:
        one()
        torch.cuda.synchronize()
    ts = []
    for _ in range(10):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        one()
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return {"gbps": round(nbytes / (float(np.median(ts)) * 1e-3) / 1e9, 1), "bytes": nbytes}


def cpu_baseline_decode(w, q, k, v, budget_s=12.0):
    """The fp64 oracle, as it stands, on (b, query head) rows of the decode
    workload in order, until about budget_s seconds of CPU work; its rate in
    the GPU's unit: the workload's K/V bytes (bf16, each kv head once) times
    the fraction of its query rows done, per second."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention as oatt

    group = w.Hq // w.Hkv
    allowed = np.ones((1, w.Skv), dtype=bool)
    row_bytes = w.Skv * (w.D + w.Dv) * 2
    done = 0
    t0 = time.perf_counter()
    for b in range(w.B):
        kn = k[b].double().numpy()
        vn = v[b].double().numpy()
        for h in range(w.Hq):
            oatt.attention_rows(q[b, h].double().numpy(), kn[h // group], vn[h // group], allowed)
            done += 1
            if time.perf_counter() - t0 > budget_s and done >= 2:
                break
        if time.perf_counter() - t0 > budget_s and done >= 2:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    model, usable = host_cpu()
    return {
        "value": done * row_bytes / group / dt / 1e9,
        "unit": "GB/s",
        "cores": int(threads),
        "cpu_model": model,
        "host_cores_usable": usable,
        "kind": "oracle",
        "sample": (f"fp64 oracle on {done} of {w.B * w.Hq} (b, query head) rows in {dt:.1f} s; bytes counted "
                   f"as the GPU's: the workload's bf16 K/V bytes times the fraction of query rows done"),
    }


def host_cpu():
    """Model name and usable core count of the host the oracle runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return model, usable


def prewarm(step, torch, seconds):
    """Run step() back to back for `seconds` of wall time, synchronising every
    few launches: the GPU's clock ramps up over the first 0.1-1 s of load, so
    a count of warm-up launches alone can leave the timed launches on a cold
    clock.  Returns the seconds spent."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    return time.perf_counter() - t0


def timed_region(step, torch, stream, steps):
    """The timed steps: one HIP event pair on the launch stream around `steps`
    back-to-back calls, bracketed by device synchronisations.  Returns (wall
    seconds, event milliseconds).  An event recorded between launches holds
    the next launch back (several microseconds per launch), so the timed
    launches run without any; per-launch statistics come from
    launch_stats afterwards."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, a.elapsed_time(b)


def launch_stats(step, torch, stream, n=20):
    """Median and minimum of n launches timed one by one (after the timed
    region; each carries the cost of its own event pair)."""
    import numpy as np
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    return float(np.median(ms)), float(np.min(ms))


def computed_work(w, block_mask, block_q=128, block_kv=128, backward=False):
    """Blocks and FLOPs of one launch on workload w with a MaskInfo whose
    block_mask is [Hm, nq', nk'] at block_q x block_kv: every 128 x 128
    sub-block of a non-empty mask block is computed.  Forward: 2 products of
    2 * 128 * 128 * D each per computed block; backward: 5 by the usual count
    (S, dP, dV, dQ, dK) and 7 executed (S and dP in both kernels)."""
    hm = block_mask.shape[0]
    nq, nk = w.Sq // w.block, w.Skv // w.block
    sub = (block_q // w.block) * (block_kv // w.block)   # 128 x 128 sub-blocks per mask block
    computed_slots = int((block_mask > 0).sum()) * sub  # per mask head set
    heads_per_mask = w.Hq if hm == 1 else 1
    blocks_computed = computed_slots * heads_per_mask * w.B
    res = {"blocks_computed": blocks_computed, "blocks_total": nq * nk * w.Hq * w.B}
    if backward:
        res["flops"] = blocks_computed * 5 * 2 * w.block * w.block * w.D
        res["flops_exec"] = blocks_computed * 7 * 2 * w.block * w.block * w.D
        res["flops_dense"] = w.B * w.Hq * w.Sq * w.Skv * 5 * 2 * w.D
    else:
        res["flops"] = res["flops_exec"] = blocks_computed * flops_per_block(w)
        res["flops_dense"] = w.B * w.Hq * w.Sq * w.Skv * 2 * (w.D + w.Dv)
    return res


def flops_per_block(w):
    return 2 * w.block * w.block * (w.D + w.Dv)


def cpu_baseline(w, q, k, v, dense, block_mask, budget_s=12.0):
    """The fp64 oracle, as it stands, on a bounded sample of the workload:
    whole 128-row query blocks of (batch 0, head h), taken round-robin over
    heads and block rows, until about budget_s seconds of CPU work.  Its rate
    is counted in the same unit as the GPU's: FLOPs of the computed blocks of
    the rows it produced, per second.  The oracle's MaskInfo builder is timed
    separately on the workload's whole mask (mask_info_ms, beside the
    library's mask_compile_ms)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention as oatt
    from oracle import mask_info as omi
    from oracle import masks as omasks

    t_mi = time.perf_counter()
    full = omasks.materialize(w.mask.kind, w.Sq, w.Skv, left=w.mask.left, right=w.mask.right,
                              chunk=w.mask.chunk, dense=dense)
    omi.build(full, w.block, w.block, computable=w.mask.kind != "dense")
    mask_info_ms = (time.perf_counter() - t_mi) * 1e3
    del full

    qn = q.double().numpy()
    kn = k.double().numpy()
    vn = v.double().numpy()
    group = w.Hq // w.Hkv
    cols = np.arange(w.Skv)
    nq = w.Sq // w.block
    per_row = (block_mask > 0).sum(axis=-1)          # [Hm, nq] non-empty blocks per block row
    order = [(h, r) for r in range(nq - 1, -1, -1) for h in range(w.Hq)]
    flops = 0.0
    rows_done = 0
    t0 = time.perf_counter()
    for h, r in order:
        rows = np.arange(r * w.block, (r + 1) * w.block)
        if w.mask.kind == "dense":
            allowed = dense[0 if dense.shape[0] == 1 else h][rows]
        else:
            allowed = omasks.allowed_block(w.mask.kind, rows, cols, left=w.mask.left,
                                           right=w.mask.right, chunk=w.mask.chunk)
        oatt.attention_rows(qn[0, h, rows], kn[0, h // group], vn[0, h // group], allowed,
                            soft_cap=w.soft_cap)
        flops += per_row[0 if per_row.shape[0] == 1 else h, r] * flops_per_block(w)
        rows_done += 1
        if time.perf_counter() - t0 > budget_s and rows_done >= 2:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    model, usable = host_cpu()
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "cpu_model": model,
        "host_cores_usable": usable,
        "kind": "oracle",
        "mask_info_ms": round(mask_info_ms, 1),
        "sample": (f"fp64 oracle on {rows_done} of the {w.Hq * nq} query blocks of batch 0 (128 rows each, "
                   f"longest block rows first, round-robin over heads) in {dt:.1f} s; "
                   f"FLOPs counted on computed blocks as for the GPU"),
    }


def bench_decode(args):
    import numpy as np
    import torch

    from block_sparse_attention_make_amd import splash_decode, synthetic

    name = args.workload if args.workload in synthetic.DECODE_WORKLOADS else "decode_gqa_32k"
    w = synthetic.DECODE_WORKLOADS[name]
    dev = torch.device("cuda:0")
    q, k, v = synthetic.make_qkv(w.seed, w.B, w.Hq, w.Hkv, 1, w.Skv, w.D, w.Dv)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out, lse = splash_decode(qd, kd, vd)
    stream = torch.cuda.current_stream(dev)
    ws = torch.empty(1, device=dev)
    import ctypes
    from block_sparse_attention_make_amd.splash import load_library
    nb = ctypes.c_size_t()
    load_library().splash_decode_workspace_size(w.B, w.Hq, w.Hkv, w.Skv, w.D, ctypes.byref(nb))
    ws = torch.empty(max(1, nb.value // 4), dtype=torch.float32, device=dev)

    def step():
        splash_decode(qd, kd, vd, out=out, lse=lse, workspace=ws, stream=stream)
    prewarm_s = prewarm(step, torch, args.prewarm_s)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall, region_ms = timed_region(step, torch, stream, args.steps)
    kav = region_ms / args.steps
    med_ms, min_ms = launch_stats(step, torch, stream)
    kv_bytes = w.B * w.Hkv * w.Skv * (w.D + w.Dv) * 2
    ms = wall * 1e3 / args.steps
    res = {
        "metric": "splash decode K/V read bandwidth (one query per head, every key)",
        "value": round(kv_bytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "kv_len": w.Skv,
                   "head_dim": w.D, "pass": "decode", "parallelism": "single-gpu"},
        "prewarm_s": round(prewarm_s, 2),
        "kernel_ms_median": round(med_ms, 5),
        "kernel_ms_min": round(min_ms, 5),
        "roofline": {"bound": "hbm", "achieved": round(kv_bytes / (kav * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(kv_bytes / (kav * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                     "traffic": measured_traffic(w.name, DECODE_SRC), "kernel": "decode_mfma + decode_merge",
                     "bytes_per_launch": kv_bytes,
                     "kernel_ms_avg": round(kav, 5)},
        "cpu_baseline": None,
    }
    probe = read_probe(torch, kv_bytes)
    if probe is not None:
        res["hbm_read_probe"] = {**probe, "frac_of_probe": round(res["roofline"]["achieved"] / probe["gbps"], 4)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(w, q, k, v)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The GPU's clock settles only after ~100 ms of sustained load, so the default warm-up is long.
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--prewarm-s", type=float, default=2.0,
                    help="seconds of back-to-back steps before the counted warm-up, so the clock has settled")
    ap.add_argument("--workload", default="causal_mha_8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--sinks", type=int, default=0, help="attention-sink logits per kv head")
    ap.add_argument("--kv-shards", type=int, default=1, help="time the key/value-sharded path")
    ap.add_argument("--backward", action="store_true", help="time splash_bwd")
    ap.add_argument("--decode", action="store_true", help="time splash_decode on a decode workload")
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=False,
                    help="time the forward as replays of a captured HIP graph of one step")
    ap.add_argument("--heads-per-wg", type=int, default=0, choices=(0, 1, 2),
                    help="query heads per workgroup: 0 the library's choice, 1, or 2 (two heads of a GQA group "
                         "sharing each K/V stage)")
    ap.add_argument("--kv-splits", default="auto",
                    help="key splits per block row: auto (the library's plan) or 1..8")
    ap.add_argument("--block-q", type=int, default=128, help="mask block rows (a multiple of 128)")
    ap.add_argument("--block-kv", type=int, default=128, help="mask block columns (a multiple of 128)")
    ap.add_argument("--cold", action="store_true",
                    help="also time launches with a 512 MiB buffer rewritten before each (cold L2 and MALL)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (the reference "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the forward shards over (batch, kv-head group) with no exchange).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_attention_make_amd import (lse_merge, make_mask_info, splash_bwd, splash_fwd,
                                                 splash_fwd_kv_sharded, synthetic)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "dispatches": 5}))
        return
    if args.decode:
        return bench_decode(args)
    w = synthetic.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    q, k, v, dense = synthetic.make_inputs(w)
    m = w.mask

    t0 = time.perf_counter()
    mi = make_mask_info(m.kind, w.Sq, w.Skv, left=m.left, right=m.right, chunk=m.chunk, dense=dense,
                        block_q=args.block_q, block_kv=args.block_kv)
    mask_ms = (time.perf_counter() - t0) * 1e3
    mi.upload()
    bm = mi.block_mask
    nq, nk = w.Sq // w.block, w.Skv // w.block
    work = computed_work(w, bm, args.block_q, args.block_kv, args.backward)
    blocks_computed, blocks_total = work["blocks_computed"], work["blocks_total"]
    flops, flops_exec, flops_dense = work["flops"], work["flops_exec"], work["flops_dense"]

    from block_sparse_attention_make_amd.splash import plan_kv_splits
    from block_sparse_attention_make_amd.splash import plan_heads_per_workgroup
    splits = (plan_kv_splits(mi, w.B, w.Hq, 0 if w.dtype == "bf16" else 1) if args.kv_splits == "auto"
              else int(args.kv_splits))
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    out = torch.empty((w.B, w.Hq, w.Sq, w.Dv), dtype=q.dtype, device=dev)
    split_ws = None
    if splits > 1:
        import ctypes
        from block_sparse_attention_make_amd.splash import load_library
        nb = ctypes.c_size_t()
        load_library().splash_fwd_workspace_size(w.B, w.Hq, w.Sq, w.Dv, splits, ctypes.byref(nb))
        split_ws = torch.empty(max(1, nb.value // 4), dtype=torch.float32, device=dev)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    aux = None
    if args.sinks:
        g = torch.Generator().manual_seed(7)
        aux = torch.randn((w.Hkv, args.sinks), generator=g, dtype=torch.float32).to(dev)
    P = args.kv_shards
    if P > 1:
        if args.sinks:
            print("--kv-shards and --sinks do not combine (a sink would count once per shard)", file=sys.stderr)
            sys.exit(2)
        if w.Skv % (128 * P):
            print(f"--kv-shards {P} must split {w.Skv} keys into whole 128-key blocks", file=sys.stderr)
            sys.exit(2)
        n = w.Skv // P
        shard_mis = [make_mask_info(m.kind, w.Sq, w.Skv, left=m.left, right=m.right, chunk=m.chunk,
                                    dense=dense, kv_slice=(s * n, n)) for s in range(P)]
        for smi in shard_mis:
            smi.upload()
        ks = [kd[:, :, s * n:(s + 1) * n].contiguous() for s in range(P)]
        vs = [vd[:, :, s * n:(s + 1) * n].contiguous() for s in range(P)]

    if args.backward:
        if w.dtype != "bf16" or P > 1 or args.sinks:
            print("--backward runs bf16 workloads without shards or sinks", file=sys.stderr)
            sys.exit(2)
        splash_fwd(qd, kd, vd, mi, logits_soft_cap=w.soft_cap, out=out, lse=lse, stream=stream)
        g = torch.Generator().manual_seed(11)
        dout = torch.randn(out.shape, generator=g).to(q.dtype).to(dev)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        delta = torch.empty(lse.shape, dtype=torch.float32, device=dev)

    def step(s=None):
        s = stream if s is None else s
        if args.backward:
            splash_bwd(qd, kd, vd, out, lse, dout, mi, logits_soft_cap=w.soft_cap, dq=dq, dk=dk, dv=dv,
                       delta=delta, stream=s)
        elif P > 1:
            splash_fwd_kv_sharded(qd, ks, vs, shard_mis, logits_soft_cap=w.soft_cap, stream=s)
        else:
            splash_fwd(qd, kd, vd, mi, logits_soft_cap=w.soft_cap, out=out, lse=lse, stream=s,
                       softmax_aux=aux, kv_splits=splits, workspace=split_ws, heads_per_workgroup=args.heads_per_wg)

    prewarm_s = prewarm(step, torch, args.prewarm_s)
    for _ in range(args.warmup):
        step()
    # --graph: the forward's launches (the kernel, and the merge with split
    # keys) captured once and replayed as a HIP graph, as a caller's step
    # loop may do.
    launch = "eager"
    if args.graph and not args.backward and P == 1:
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=torch.cuda.Stream()):
            step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        launch = "graph"
        for _ in range(20):
            graph.replay()
        step = lambda s=None: graph.replay()   # noqa: E731 (replays on the current stream)
    wall, region_ms = timed_region(step, torch, stream, args.steps)
    med_ms, min_ms = launch_stats(step, torch, stream)
    cold = None
    if args.cold:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for a, b in cev:
            flush.fill_(1)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        cms = [a.elapsed_time(b) for a, b in cev]
        cold = {"kernel_ms_median": round(float(np.median(cms)), 5),
                "tflops": round(flops / (float(np.median(cms)) * 1e-3) / 1e12, 2)}
        del flush
    probe = mfma_probe(torch) if not args.backward and P == 1 else None
    merge_info = None
    if P > 1:
        # the merge kernel alone: float32 accumulator (in place) + one bf16 shard result
        rows = w.B * w.Hq * w.Sq
        acc = torch.zeros((rows, w.Dv), dtype=torch.float32, device=dev)
        acc_l = torch.zeros(rows, dtype=torch.float32, device=dev)
        part = torch.randn((rows, w.Dv), dtype=torch.float32, device=dev).to(q.dtype)
        part_l = torch.randn(rows, dtype=torch.float32, device=dev)
        for _ in range(20):
            lse_merge(acc, acc_l, part, part_l, out=acc, lse=acc_l, stream=stream)
        mev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(50)]
        for a, b in mev:
            a.record(stream)
            lse_merge(acc, acc_l, part, part_l, out=acc, lse=acc_l, stream=stream)
            b.record(stream)
        torch.cuda.synchronize()
        m_ms = float(np.mean([a.elapsed_time(b) for a, b in mev]))
        m_bytes = rows * w.Dv * (4 + part.element_size() + 4) + rows * 4 * 3
        merge_info = {"kernel": "lse_merge_kernel", "bound": "hbm", "bytes_per_launch": m_bytes,
                      "kernel_ms_avg": round(m_ms, 5), "achieved": round(m_bytes / (m_ms * 1e-3) / 1e9, 1),
                      "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                      "frac": round(m_bytes / (m_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
    ms_per_step = wall * 1e3 / args.steps
    kern_avg = region_ms / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops_exec / (kern_avg * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    # the committed traffic summaries were taken with the workload's default launch
    default_launch = (args.kv_splits == "auto" and args.heads_per_wg == 0 and not args.sinks and P == 1
                      and not args.backward
                      and args.block_q == w.block and args.block_kv == w.block)
    traffic = measured_traffic(w.name) if default_launch else None

    res = {
        "metric": ("splash bwd TFLOP/s on computed blocks (5 products per block)" if args.backward else
                   "splash fwd TFLOP/s on computed blocks + % bf16 MFMA peak; blocks skipped"),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "seq_len": w.Sq, "head_dim": w.D, "vhead_dim": w.Dv, "mask": m.kind, "block": w.block,
                   "soft_cap": w.soft_cap, "parallelism": "single-gpu",
                   "sinks_per_kv_head": args.sinks, "kv_shards": P, "kv_splits": splits,
                   "heads_per_workgroup": None if args.backward or P > 1 else (
                       args.heads_per_wg or plan_heads_per_workgroup(
                           mi, w.B, w.Hq, w.Hkv, w.D, 0 if w.dtype == "bf16" else 1, splits)),
                   "mask_block": [args.block_q, args.block_kv], "pass": "backward" if args.backward else "forward"},
        "prewarm_s": round(prewarm_s, 2),
        "launch": launch,
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "dense_equiv_tflops": round(flops_dense / (ms_per_step * 1e-3) / 1e12, 2),
        "blocks_skipped": blocks_total - blocks_computed,
        "blocks_total": blocks_total,
        "grid_width": int(bm.shape[-1]),
        "kernel_ms_median": round(med_ms, 5),
        "kernel_ms_min": round(min_ms, 5),
        "mask_compile_ms": round(mask_ms, 3),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": "splash_fwd_wide" if w.dtype == "bf16" else "splash_fwd_kernel",
                     "flops_per_launch": flops,
                     "kernel_ms_avg": round(kern_avg, 5)},
        "cpu_baseline": None,
    }
    if splits > 1 and not args.backward and P == 1:
        res["roofline"]["kernel"] = "splash_fwd_wide (key splits) + merge_splits"
    if args.backward:
        res["roofline"]["kernel"] = "bwd_delta + bwd_dkdv + bwd_dq (executed products: 7 per block)"
        res["roofline"]["flops_per_launch"] = flops_exec
        res["roofline"]["traffic"] = None
        res["vs_baseline"] = None
    if probe is not None:
        res["mfma_probe"] = {**probe, "frac_of_probe": round(achieved / probe["tflops"], 4)}
        if probe.get("tflops_random_operands"):
            res["mfma_probe"]["frac_of_random_probe"] = round(achieved / probe["tflops_random_operands"], 4)
    if cold is not None:
        res["cold_cache"] = cold
    if merge_info is not None:
        res["merge"] = merge_info
        # with shards the timed step holds several kernels: achieved is per step, not per launch
        res["roofline"]["kernel"] = "splash_fwd_wide x P + lse_merge_kernel x (P-1)"
        res["roofline"]["traffic"] = None
    if (not args.no_cpu_baseline and not args.backward and P == 1 and not args.sinks
            and args.block_q == w.block and args.block_kv == w.block):
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, dense, bm, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
