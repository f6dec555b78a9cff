"""Throughput of the tiled GEMM on one MI355X; prints one JSON line.

A step is one GEMM over the 8192 x 8192 x 8192 bf16 workload (row-major A
and B drawn from N(0,1)/sqrt(K), fp32 accumulation, bf16 output) with the
inputs already resident in device memory.  The timed region is exactly
`--steps` back-to-back calls through the C ABI, bracketed by
torch.cuda.synchronize(); each call is also bracketed by HIP events on the
launch stream, whose mean is the kernel time used for the roofline.

Beside the main figure the line carries:
  roofline      the GEMM kernel against the dense bf16 MFMA peak (and against
                that peak scaled to the graphics clock the chip ran at);
  telemetry     graphics and memory clocks, socket power, hotspot temperature
                (amdsmi) over a short soak of the same call after the timed
                region;
  device        name, architecture, compute units, memory, L2 and LDS sizes;
  cold_*        kernel time (median, p90) with the caches flushed by a
                512 MiB write before each call (not with --no-also);
  cpu_baseline  the CPU oracle timed on this host on a bounded sample of the
                same workload (whole output rows), scaled to TFLOP/s;
  also          the same measurement for the 256^3 and 1024x1024x2048 fp16
                GEMMs, the fused bias+ReLU form and the grouped MoE GEMM
                (these also replayed from a HIP graph of 50 or 20 launches,
                the kernel time without the host's launch overhead), the 4096^3 fp32
                GEMM (against the fp32 matrix peak), a 3x3 convolution on the
                GEMM (implicit im2col; batch 32, 56x56, 64 -> 64 channels,
                fp16) and attention scores Q K^T (128 heads, 2048 x 2048,
                d = 128, bf16; bound by writing the 1 GiB of scores).

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 50] [--no-cpu-baseline] [--no-also] [--no-telemetry]
                      [--no-cold]
       python bench.py --table BENCH.json   (the per-workload report table of a bench line, markdown)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s and % of MI355X fp16 MFMA peak (1024x1024x2048 and 8192^3)"
PEAK_MFMA_TFLOPS = 2516.6   # dense fp16/bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # HBM3E
PEAK_F32_TFLOPS = 157.3     # dense fp32 matrix (and vector) peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="gemm_8192_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache timings")
    ap.add_argument("--no-telemetry", action="store_true",
                    help="skip the clock/power soak after the timed region (profiled runs: keeps the timed calls last)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the CPU-baseline sample")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for counter collection: one GEMM, a plain copy of known size, one GEMM; no timing")
    return ap.parse_args()


def pmc_probe(name):
    """GEMM, then an elementwise copy reading and writing COPY_BYTES, then GEMM.
    Under rocprofv3 --pmc the copy calibrates FETCH_SIZE / WRITE_SIZE."""
    import torch

    from tiled_matrix_multiplication_gemm_amd import profiling

    from tiled_matrix_multiplication_gemm_amd import inputs

    if name == CONV_NAME:
        fn = conv_setup()[0]
    elif name == ATTN_NAME:
        fn = attention_setup()[0]
    elif name in inputs.GROUPED_WORKLOADS:
        c, fn = grouped_setup(name)
    else:
        c, fn = dense_setup(name)
    fn()
    torch.cuda.synchronize()
    n = profiling.COPY_BYTES // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    fn()
    torch.cuda.synchronize()
    print("pmc probe done: %s" % name)


def stored_traffic(name):
    """HBM bytes per dispatch from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    from tiled_matrix_multiplication_gemm_amd import profiling

    path = os.path.join(ROOT, "profiles", "%s_traffic.txt" % name)
    if not os.path.exists(path):
        return None
    s = profiling.read_summary(path)
    if s.get("source_hash") != profiling.source_hash():
        return None
    return float(s["traffic_bytes"])


def upload(bits, dt):
    import numpy as np
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.float16 if dt == 0 else torch.bfloat16)


def time_calls(fn, steps: int, warmup: int, per_call: bool = False):
    """Warm up, then time exactly `steps` calls: wall clock over the whole
    region (synchronised on both sides) and HIP events around each call.
    Returns (wall s, mean ms, median ms), plus the sorted per-call ms list
    when per_call is set."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    if per_call:
        return wall, sum(per) / len(per), per[len(per) // 2], per
    return wall, sum(per) / len(per), per[len(per) // 2]


def spread(per):
    """min / median / p90 of a sorted list of per-call times (ms)."""
    return {"min": round(per[0], 5), "median": round(per[len(per) // 2], 5),
            "p90": round(per[min(len(per) - 1, (9 * len(per)) // 10)], 5)}


def device_info():
    """What the runtime reports about the GPU the line was measured on."""
    import torch

    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1)}
    for key, attr in (("l2_bytes", "L2_cache_size"), ("lds_bytes_per_block", "shared_memory_per_block"),
                      ("warp_size", "warp_size"), ("clock_khz", "clock_rate")):
        v = getattr(p, attr, None)
        if isinstance(v, int):
            info[key] = v
    return info


def time_graph(fn, out, calls: int = 50, replays: int = 20):
    """Per-launch time without host launch overhead: `calls` launches of fn
    captured into one HIP graph, the graph replayed `replays` times with HIP
    events around each replay.  Every replay's output is checked against the
    eager one first (the timed replays run the same graph).  Returns the
    median per-launch ms, or None if the graph's output differs."""
    import torch

    fn()
    torch.cuda.synchronize()
    want = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, want):
            return None
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = []
    for _ in range(replays):
        s.record()
        g.replay()
        e.record()
        torch.cuda.synchronize()
        per.append(s.elapsed_time(e) / calls)
    del g
    per.sort()
    return per[len(per) // 2]


FLUSH_BYTES = 512 * 1024 * 1024  # more than the 256 MB last-level cache plus the 8 x 4 MB L2


def time_cold(fn, reps: int):
    """Kernel time with cold caches: before each timed call a 512 MiB buffer
    is written, evicting the last-level cache and every L2, so the operands
    come from HBM.  Returns (median, p90) in ms of the HIP-event times."""
    import torch

    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    fn()
    for i in range(reps):
        flush.fill_(float(i))
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in zip(starts, ends))
    del flush
    return per[len(per) // 2], per[min(len(per) - 1, (9 * len(per)) // 10)]


def dense_setup(name, variant="float"):
    import torch

    import tiled_matrix_multiplication_gemm_amd as mg
    from tiled_matrix_multiplication_gemm_amd import inputs

    c = inputs.dense_workload(name, variant)
    A, B = upload(c.A, c.dtype), upload(c.B, c.dtype)
    C = torch.empty((c.M, c.N), dtype=A.dtype, device="cuda")
    if c.bias is not None:
        bias = upload(c.bias, c.dtype)
        fn = lambda: mg.mg_gemm_bias_relu(A, B, bias, out=C)
    else:
        fn = lambda: mg.mg_gemm(A, B, out=C)
    fn.out = C
    return c, fn


def measure_dense(name, steps, warmup):
    import tiled_matrix_multiplication_gemm_amd as mg

    c, fn = dense_setup(name)
    wall, mean_ms, med_ms, per = time_calls(fn, steps, warmup, per_call=True)
    flops = 2.0 * c.M * c.N * c.K
    d = mg.mg_config_info(mg.mg_last_config())
    hbm_bytes = 2.0 * (c.M * c.K + c.K * c.N + c.M * c.N) + (2.0 * c.N if c.bias is not None else 0.0)
    return dict(case=c, flops=flops, wall=wall, kernel_ms=mean_ms, kernel_ms_median=med_ms, tile_config=d["name"],
                kernel=mg.mg_last_kernel(), compulsory_bytes=hbm_bytes, fn=fn, spread=spread(per))


def grouped_setup(name, variant="float"):
    import numpy as np
    import torch

    import tiled_matrix_multiplication_gemm_amd as mg
    from tiled_matrix_multiplication_gemm_amd import inputs

    c = inputs.grouped_workload(name, variant)
    X, W = upload(c.X, c.dtype), upload(c.W, c.dtype)
    off = torch.from_numpy(c.offsets.astype(np.int32)).cuda()
    Y = torch.empty((c.T, c.N), dtype=X.dtype, device="cuda")
    fn = lambda: mg.mg_grouped_gemm(X, W, off, out=Y)  # noqa: E731
    fn.out = Y
    return c, fn


def measure_grouped(name, steps, warmup):
    import tiled_matrix_multiplication_gemm_amd as mg

    c, fn = grouped_setup(name)
    wall, mean_ms, med_ms, per = time_calls(fn, steps, warmup, per_call=True)
    flops = 2.0 * c.T * c.K * c.N
    hbm_bytes = 2.0 * (c.T * c.K + c.E * c.K * c.N + c.T * c.N) + 4.0 * (c.E + 1)
    cfg = mg.mg_config_info(mg.mg_last_config())["name"]
    return dict(case=c, flops=flops, wall=wall, kernel_ms=mean_ms, kernel_ms_median=med_ms, tile_config=cfg,
                compulsory_bytes=hbm_bytes, fn=fn, spread=spread(per))


def cpu_baseline(case, target_s: float):
    """The oracle, as it is, on whole output rows of the same workload."""
    import numpy as np

    import oracle

    threads = min(16, oracle.default_threads())
    rows = 8
    while True:
        t0 = time.perf_counter()
        oracle.gemm(case.A[:rows], case.B, case.dtype, bias=case.bias, relu=case.relu, nthreads=threads)
        dt = time.perf_counter() - t0
        if dt >= target_s or rows >= case.M:
            break
        # grow the sample towards the target length
        rows = int(min(case.M, max(rows * 2, rows * target_s / max(dt, 1e-3) * 0.9)))
    flops = 2.0 * rows * case.N * case.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d output rows (%dx%dx%d), %.1f s, fp64 accumulation" % (rows, case.M, rows, case.N,
                                                                                       case.K, dt)}


CONV_NAME = "conv3x3_n32_56x56_c64_k64_f16"
ATTN_NAME = "attention_scores_h128_l2048_d128_bf16"


def conv_setup():
    """The 3x3 convolution workload (implicit GEMM) on the device: the call,
    its flops, its compulsory HBM bytes (input, weights and output once) and
    the workspace its configuration needs."""
    import torch

    import tiled_matrix_multiplication_gemm_amd as mg
    from tiled_matrix_multiplication_gemm_amd import inputs

    w = inputs.CONV_WORKLOAD
    cc = inputs.conv_case(w["Nb"], w["H"], w["W"], w["C"], w["OC"], w["KH"], w["KW"], w["dtype"], w["seed_float"],
                          w["stride"], w["pad"], w["dil"])
    x, wt = upload(cc.x, cc.dtype), upload(cc.w, cc.dtype)
    y = torch.empty((w["Nb"], w["H"], w["W"], w["OC"]), dtype=x.dtype, device="cuda")
    M, K = w["Nb"] * w["H"] * w["W"], w["KH"] * w["KW"] * w["C"]
    ws = mg.mg_conv2d_workspace_bytes(mg.conv2d_shape(x.shape, 3, w["OC"], 1, 1, 1), cc.dtype)
    return (lambda: mg.mg_conv2d(x, wt, w["stride"], w["pad"], w["dil"], out=y), 2.0 * M * K * w["OC"],
            2.0 * (x.numel() + wt.numel() + y.numel()), ws)


def attention_setup():
    """The attention-score workload (Q K^T for every head) on the device: the
    call, its flops and its compulsory HBM bytes."""
    import torch

    import tiled_matrix_multiplication_gemm_amd as mg
    from tiled_matrix_multiplication_gemm_amd import inputs

    a = inputs.ATTENTION_WORKLOAD
    ac = inputs.attention_case(a["heads"], a["L"], a["L"], a["d"], a["dtype"], a["seed_float"])
    q, k = upload(ac.Q, ac.dtype), upload(ac.K, ac.dtype)
    S = torch.empty((a["heads"], a["L"], a["L"]), dtype=q.dtype, device="cuda")
    return (lambda: mg.mg_attention_scores(q, k, out=S), 2.0 * a["heads"] * a["L"] * a["L"] * a["d"],
            2.0 * (q.numel() + k.numel() + S.numel()), 0)


def measure_consumers(steps, warmup):
    """fp32 GEMM, convolution and attention-score workloads: kernel time from
    HIP events, TFLOP/s, and compulsory HBM bytes per second."""
    import numpy as np
    import torch

    import tiled_matrix_multiplication_gemm_amd as mg
    from tiled_matrix_multiplication_gemm_amd import inputs

    out = {}
    # fp32 GEMM 4096^3 (the fp32 row of the FlagOS page's table)
    c = inputs.dense_f32(4096, 4096, 4096, seed=110)
    A = torch.from_numpy(c.A.view(np.float32)).cuda()
    B = torch.from_numpy(c.B.view(np.float32)).cuda()
    C = torch.empty((4096, 4096), device="cuda")
    wall, mean_ms, _ = time_calls(lambda: mg.mg_gemm(A, B, out=C), steps, warmup)
    fl = 2.0 * 4096 ** 3
    ach = fl / (mean_ms * 1e-3) / 1e12
    out["gemm_4096_f32"] = {"kernel_tflops": round(ach, 2), "frac_f32_peak": round(ach / PEAK_F32_TFLOPS, 4),
                            "kernel_ms_mean": round(mean_ms, 5)}
    del A, B, C
    # 3x3 convolution, implicit GEMM
    fn, fl, byts, cfg_ws = conv_setup()
    wall, mean_ms, _ = time_calls(fn, steps, warmup)
    ach = fl / (mean_ms * 1e-3) / 1e12
    gbs = byts / (mean_ms * 1e-3) / 1e9
    out[CONV_NAME] = {
        "kernel_tflops": round(ach, 2), "frac_mfma_peak": round(ach / PEAK_MFMA_TFLOPS, 4),
        "hbm_gbs_compulsory": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "kernel_ms_mean": round(mean_ms, 5), "tile_config": mg.mg_config_info(mg.mg_last_config())["name"],
        "workspace_bytes": cfg_ws, "compulsory_bytes": byts, "traffic": stored_traffic(CONV_NAME)}
    del fn
    # attention scores
    fn, fl, byts, _ = attention_setup()
    wall, mean_ms, _ = time_calls(fn, steps, warmup)
    ach = fl / (mean_ms * 1e-3) / 1e12
    gbs = byts / (mean_ms * 1e-3) / 1e9
    out[ATTN_NAME] = {
        "kernel_tflops": round(ach, 2), "frac_mfma_peak": round(ach / PEAK_MFMA_TFLOPS, 4),
        "hbm_gbs_compulsory": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "kernel_ms_mean": round(mean_ms, 5), "tile_config": mg.mg_config_info(mg.mg_last_config())["name"],
        "compulsory_bytes": byts, "traffic": stored_traffic(ATTN_NAME)}
    return out


def measure_shapes(steps, warmup):
    """Shapes off the tile grid (K not a whole number of slices, N % 8 != 0)
    next to the aligned shape of the same size, random N(0,1)/sqrt(K) data."""
    import torch

    import tiled_matrix_multiplication_gemm_amd as mg
    from tiled_matrix_multiplication_gemm_amd import inputs

    out = {}
    for M, N, K, dt in ((4096, 4096, 4096, inputs.F16), (4096, 4096, 4100, inputs.F16),
                        (8192, 8190, 8192, inputs.BF16)):
        c = inputs.random_dense(M, N, K, dt, 7000 + K % 97 + N % 89)
        ld = (N + 7) // 8 * 8
        A = upload(c.A, dt)
        Bfull = torch.zeros((K, ld), dtype=A.dtype, device="cuda")
        Bfull[:, :N] = upload(c.B, dt)
        B = Bfull[:, :N]
        Cfull = torch.empty((M, ld), dtype=A.dtype, device="cuda")
        C = Cfull[:, :N]
        if K % 8:  # a row stride that spans whole 16-byte chunks
            Afull = torch.zeros((M, (K + 7) // 8 * 8), dtype=A.dtype, device="cuda")
            Afull[:, :K] = A
            A = Afull[:, :K]
        fn = lambda: mg.mg_gemm(A, B, out=C)
        _, mean_ms, _, per = time_calls(fn, steps, warmup, per_call=True)
        fl = 2.0 * M * N * K
        out["gemm_%dx%dx%d_%s" % (M, N, K, "bf16" if dt else "f16")] = {
            "kernel_tflops": round(fl / (mean_ms * 1e-3) / 1e12, 2), "kernel_ms_mean": round(mean_ms, 5),
            "warm_ms": spread(per), "kernel": mg.mg_last_kernel(),
            "tile_config": mg.mg_config_info(mg.mg_last_config())["name"]}
        del A, B, C, Bfull, Cfull
    return out


def measure_prepack(steps, warmup):
    """The layout planner: the blocked A [ceil(K/BK), M, BK] on the same
    kernel against the row-major A, and the cost of the blocking copy."""
    import torch

    import tiled_matrix_multiplication_gemm_amd as mg
    from tiled_matrix_multiplication_gemm_amd import inputs

    out = {}
    for name in ("gemm_1024x1024x2048_f16", "gemm_8192_bf16"):
        c = inputs.dense_workload(name, "float")
        A, B = upload(c.A, c.dtype), upload(c.B, c.dtype)
        C = torch.empty((c.M, c.N), dtype=A.dtype, device="cuda")
        BK = mg.mg_config_bk(c.M, c.N, c.K, c.dtype)
        Ap = mg.mg_prepack_a(A, BK)
        n = max(steps, 50) if c.M < 4096 else steps
        _, plain, _, pp = time_calls(lambda: mg.mg_gemm(A, B, out=C), n, warmup, per_call=True)
        _, packed, _, pk = time_calls(lambda: mg.mg_gemm_prepacked(Ap, BK, B, c.M, c.K, out=C), n, warmup,
                                      per_call=True)
        kern = mg.mg_last_kernel()
        _, copy, _, pc = time_calls(lambda: mg.mg_prepack_a(A, BK, out=Ap), n, warmup, per_call=True)
        out[name] = {"plain_ms": spread(pp), "packed_ms": spread(pk), "prepack_copy_ms": spread(pc),
                     "packed_kernel": kern, "bk": BK,
                     "planner": {"uses_to_pay": mg.mg_prepack_uses_to_pay(c.M, c.N, c.K, c.dtype)}}
        del A, B, C, Ap
    return out


def oracle_timing():
    """The oracle per workload on this host (a reported baseline): the full
    output of the 256^3 and 1024x1024x2048 workloads (median of 3 runs), the
    4096-element sample of the 8192^3 and grouped ones, each with all cores
    the process may use (at most 16) and with one; sampled figures are
    extrapolated to the full problem and labelled so."""
    import statistics

    import numpy as np

    import oracle
    from oracle import compare
    from tiled_matrix_multiplication_gemm_amd import inputs

    out = {}
    many = oracle.default_threads()
    for name in ("gemm_256_f16", "gemm_1024x1024x2048_f16", "gemm_bias_relu_1024x1024x2048_f16"):
        c = inputs.dense_workload(name, "float")
        rec = {}
        for label, th in (("threads_%d" % many, many), ("threads_1", 1)):
            ts = []
            for _ in range(3):
                t0 = time.perf_counter()
                oracle.gemm(c.A, c.B, c.dtype, bias=c.bias, relu=c.relu, nthreads=th)
                ts.append(time.perf_counter() - t0)
            t = statistics.median(ts)
            rec[label] = {"s": round(t, 4), "gflops": round(2.0 * c.M * c.N * c.K / t / 1e9, 3)}
        out[name] = dict(rec, sample="full output, median of 3")
    c = inputs.dense_workload("gemm_8192_bf16", "float")
    w = inputs.DENSE_WORKLOADS["gemm_8192_bf16"]
    rows, cols = compare.sample_positions(c.M, c.N, 4096, w["seed_sample"])
    rec = {}
    for label, th in (("threads_%d" % many, many), ("threads_1", 1)):
        t0 = time.perf_counter()
        oracle.gemm_sampled(c.A, c.B, c.dtype, rows, cols, nthreads=th)
        t = time.perf_counter() - t0
        g = 2.0 * 4096 * c.K / t / 1e9
        rec[label] = {"s": round(t, 4), "gflops": round(g, 3),
                      "extrapolated_full_s": round(2.0 * c.M * c.N * c.K / (g * 1e9), 1)}
    out["gemm_8192_bf16"] = dict(rec, sample="4096 sampled outputs (times include decoding the inputs)")
    g = inputs.grouped_workload("grouped_moe_e32_t8192_k1024_n4096_f16", "float")
    wg = inputs.GROUPED_WORKLOADS["grouped_moe_e32_t8192_k1024_n4096_f16"]
    rows, cols = compare.sample_positions(g.T, g.N, 4096, wg["seed_sample"])
    t0 = time.perf_counter()
    oracle.grouped_sampled(g.X, g.W, g.offsets, g.dtype, rows, cols)
    t = time.perf_counter() - t0
    gf = 2.0 * 4096 * g.K / t / 1e9
    out["grouped_moe_e32_t8192_k1024_n4096_f16"] = {
        "threads_1": {"s": round(t, 4), "gflops": round(gf, 3),
                      "extrapolated_full_s": round(2.0 * g.T * g.N * g.K / (gf * 1e9), 1)},
        "sample": "4096 sampled outputs, one thread (times include decoding the inputs)"}
    del np
    return out


PARITY = {  # what the GPU tests check on each workload (tests/test_gpu_parity.py)
    "C1": "bit-exact / tolerance + Higham bound, full output",
    "C2": "bit-exact (also a ties stress) / tolerance + Higham, full output",
    "C3": "bit-exact / tolerance + Higham, full output",
    "C4": "bit-exact / tolerance + Higham, the 4096 sample + edges and the full output",
    "C5": "bit-exact / tolerance + Higham, the 4096 sample + edges and the full output",
}


def table(path):
    """The per-workload report table (markdown) from a bench JSON line."""
    with open(path) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    a, ow = line["also"], line["cpu_baseline"]["per_workload"]
    r = line["roofline"]
    rows = [
        ("C1", "256³ fp16", "latency", a["gemm_256_f16"], 3.36e7, 393216.0, "gemm_256_f16"),
        ("C2", "1024×1024×2048 fp16", "MFMA", a["gemm_1024x1024x2048_f16"], 4.295e9, 10485760.0,
         "gemm_1024x1024x2048_f16"),
        ("C3", "C2 + bias + ReLU", "MFMA", a["gemm_bias_relu_1024x1024x2048_f16"], 4.295e9, 10487808.0,
         "gemm_bias_relu_1024x1024x2048_f16"),
        ("C4", "8192³ bf16", "MFMA (target ≥ 70 %)", {"kernel_ms_mean": r["kernel_ms_mean"], "warm_ms": r["warm_ms"]},
         1.0995e12, 402653184.0, "gemm_8192_bf16"),
        ("C5", "grouped MoE, 32 experts, 8192 tokens, 1024→4096 fp16", "HBM (weights)",
         a["grouped_moe_e32_t8192_k1024_n4096_f16"], 6.872e10, 352321536.0 + 132.0,
         "grouped_moe_e32_t8192_k1024_n4096_f16"),
    ]
    out = ["| cfg | shape / dtype | bound | TFLOP/s (ms; per-call warm min / p90) | % of 2516.6 | % of roofline bound | "
           "HBM GB/s | parity (int / float) | oracle (this host) |", "|---|---|---|---|---|---|---|---|---|"]
    for cfg, shape, bound, rec, fl, byts, key in rows:
        ms = rec.get("graph_kernel_ms") or rec["kernel_ms_mean"]
        tf = fl / (ms * 1e-3) / 1e12
        roof = min(PEAK_MFMA_TFLOPS, fl / byts * PEAK_HBM_GBS / 1e3)
        o = ow[key]
        many = [k for k in o if k.startswith("threads_") and k != "threads_1"]
        if "extrapolated_full_s" in o.get("threads_1", {}):
            th = many[0] if many else "threads_1"
            n = th.split("_")[1]
            orc = "%s core%s: %.3g GFLOP/s on the 4096 sample (extrapolated %.0f s)" % (
                n, "" if n == "1" else "s", o[th]["gflops"], o[th]["extrapolated_full_s"])
        else:
            orc = "%s cores %.3f s, 1 core %.3f s, full output" % (many[0].split("_")[1], o[many[0]]["s"],
                                                                  o["threads_1"]["s"])
        w = rec.get("warm_ms", {})
        out.append("| %s | %s | %s | %.1f (%.4f; %.4f / %.4f) | %.1f %% | %.1f %% | %.0f | %s | %s |" % (
            cfg, shape, bound, tf, ms, w.get("min", ms), w.get("p90", ms), 100 * tf / PEAK_MFMA_TFLOPS,
            100 * tf / roof, byts / (ms * 1e-3) / 1e9, PARITY[cfg], orc))
    return "\n".join(out)


def main():
    if len(sys.argv) == 3 and sys.argv[1] == "--table":
        print(table(sys.argv[2]))
        return
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import tiled_matrix_multiplication_gemm_amd as mg

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mg.lib()
    if args.pmc_probe:
        pmc_probe(args.workload)
        return

    main_res = measure_dense(args.workload, args.steps, args.warmup)
    c = main_res["case"]
    value = main_res["flops"] * args.steps / main_res["wall"] / 1e12
    achieved = main_res["flops"] / (main_res["kernel_ms"] * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["wall"] / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if c.dtype == 1 else "f16",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": c.M, "N": c.N, "K": c.K,
                   "layout": "row-major A[M,K], B[K,N]", "accumulate": "fp32",
                   "tile_config": main_res["tile_config"]},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_MFMA_TFLOPS, 4), "traffic": stored_traffic(args.workload),
                     "compulsory_bytes": main_res["compulsory_bytes"],
                     "kernel_ms_mean": round(main_res["kernel_ms"], 4),
                     "kernel_ms_median": round(main_res["kernel_ms_median"], 4),
                     "kernel": "%s (%s)" % (main_res["kernel"], main_res["tile_config"])},
    }
    # The chip lowers its clock to stay within its power limit; the same
    # kernel's rate at the clock it actually ran at is the fraction of the
    # matrix cores' peak scaled to that clock (256 CU x 4096 flop/clk).
    from tiled_matrix_multiplication_gemm_amd.profiling import soak_telemetry

    tel = None if args.no_telemetry else soak_telemetry(main_res["fn"])
    if not args.no_also and not args.no_cold:
        cmed, cp90 = time_cold(main_res["fn"], 20)
        line["roofline"]["cold_kernel_ms_median"] = round(cmed, 4)
        line["roofline"]["cold_kernel_ms_p90"] = round(cp90, 4)
    line["telemetry"] = tel
    line["device"] = device_info()
    if tel and tel.get("gfx_clock_mhz"):
        peak_clk = 256 * 4096 * tel["gfx_clock_mhz"] * 1e6 / 1e12
        line["roofline"]["peak_at_clock"] = round(peak_clk, 1)
        line["roofline"]["frac_at_clock"] = round(achieved / peak_clk, 4)
    sys.stdout.flush()
    line["roofline"]["warm_ms"] = main_res["spread"]
    if not args.no_also:
        also = {}
        for name in ("gemm_256_f16", "gemm_1024x1024x2048_f16", "gemm_bias_relu_1024x1024x2048_f16"):
            r = measure_dense(name, max(args.steps, 50), max(args.warmup, 10))
            ach = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
            cmed, cp90 = (None, None) if args.no_cold else time_cold(r["fn"], 100)
            gms = time_graph(r["fn"], r["fn"].out)
            gach = gms and r["flops"] / (gms * 1e-3) / 1e12
            also[name] = {"tflops": round(r["flops"] * max(args.steps, 50) / r["wall"] / 1e12, 2),
                          "kernel_tflops": round(ach, 2), "frac_mfma_peak": round(ach / PEAK_MFMA_TFLOPS, 4),
                          "graph_kernel_ms": gms and round(gms, 5), "graph_kernel_tflops": gach and round(gach, 2),
                          "graph_frac_mfma_peak": gach and round(gach / PEAK_MFMA_TFLOPS, 4),
                          "kernel_ms_mean": round(r["kernel_ms"], 5), "warm_ms": r["spread"],
                          "tile_config": r["tile_config"], "kernel": r["kernel"],
                          "cold_kernel_ms_median": cmed and round(cmed, 5), "cold_kernel_ms_p90": cp90 and round(cp90, 5)}
        gname = "grouped_moe_e32_t8192_k1024_n4096_f16"
        r = measure_grouped(gname, args.steps, args.warmup)
        ach = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
        gbs = r["compulsory_bytes"] / (r["kernel_ms"] * 1e-3) / 1e9
        also[gname] = {"tflops": round(r["flops"] * args.steps / r["wall"] / 1e12, 2),
                       "kernel_tflops": round(ach, 2), "frac_mfma_peak": round(ach / PEAK_MFMA_TFLOPS, 4),
                       "hbm_gbs_compulsory": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                       "kernel_ms_mean": round(r["kernel_ms"], 5), "warm_ms": r["spread"],
                       "tile_config": r["tile_config"]}
        gms = time_graph(r["fn"], r["fn"].out, calls=20)
        if gms:
            gach = r["flops"] / (gms * 1e-3) / 1e12
            ggbs = r["compulsory_bytes"] / (gms * 1e-3) / 1e9
            also[gname].update({"graph_kernel_ms": round(gms, 5), "graph_kernel_tflops": round(gach, 2),
                                "graph_hbm_gbs_compulsory": round(ggbs, 1),
                                "graph_frac_hbm_peak": round(ggbs / PEAK_HBM_GBS, 4)})
        if not args.no_cold:
            cmed, cp90 = time_cold(r["fn"], 20)
            also[gname]["cold_kernel_ms_median"] = round(cmed, 5)
            also[gname]["cold_kernel_ms_p90"] = round(cp90, 5)
        also.update(measure_consumers(min(args.steps, 50), min(args.warmup, 10)))
        also["off_grid_shapes"] = measure_shapes(min(args.steps, 50), min(args.warmup, 10))
        also["layout_planner"] = measure_prepack(min(args.steps, 50), min(args.warmup, 10))
        line["also"] = also
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(c, args.cpu_seconds)
        if not args.no_also:
            line["cpu_baseline"]["per_workload"] = oracle_timing()
    print(json.dumps(line))
    sys.stdout.flush()


if __name__ == "__main__":
    main()
