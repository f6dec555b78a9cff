"""Offline sweep of the configuration table on the GPU.

  python -m tiled_matrix_multiplication_gemm_amd.sweep [--rounds 5] [--out FILE] [workload ...]

Times every table row on each workload through the C ABI (forcing the row
with mg_set_config), visiting the rows round-robin for several rounds so that
clock drift and warm-up do not favour the rows measured last, and reports
the median kernel time per row.  The results are the evidence behind the
shape classes of select_config() in csrc/mg_api.hip.  Inputs are the
workloads' seeded float inputs.
"""
from __future__ import annotations

import argparse
import os
import statistics
import sys


def _upload(bits, dt):
    import numpy as np
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.float16 if dt == 0 else torch.bfloat16)


def _setup(name):
    import numpy as np
    import torch

    import tiled_matrix_multiplication_gemm_amd as mg
    from tiled_matrix_multiplication_gemm_amd import inputs

    if name in inputs.GROUPED_WORKLOADS:
        c = inputs.grouped_workload(name)
        X, W = _upload(c.X, c.dtype), _upload(c.W, c.dtype)
        off = torch.from_numpy(c.offsets.astype(np.int32)).cuda()
        Y = torch.empty((c.T, c.N), dtype=X.dtype, device="cuda")
        return (lambda: mg.mg_grouped_gemm(X, W, off, out=Y)), 2.0 * c.T * c.K * c.N
    c = inputs.dense_workload(name)
    A, B = _upload(c.A, c.dtype), _upload(c.B, c.dtype)
    C = torch.empty((c.M, c.N), dtype=A.dtype, device="cuda")
    if c.bias is not None:
        bias = _upload(c.bias, c.dtype)
        return (lambda: mg.mg_gemm_bias_relu(A, B, bias, out=C)), 2.0 * c.M * c.N * c.K
    return (lambda: mg.mg_gemm(A, B, out=C)), 2.0 * c.M * c.N * c.K


def _time(fn, reps):
    import torch

    s = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    e = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        s[i].record()
        fn()
        e[i].record()
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) for a, b in zip(s, e))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("workloads", nargs="*", default=["gemm_8192_bf16", "gemm_1024x1024x2048_f16",
                                                      "grouped_moe_e32_t8192_k1024_n4096_f16"])
    ap.add_argument("--rounds", type=int, default=5)
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()
    import torch

    import tiled_matrix_multiplication_gemm_amd as mg

    lines = ["# table sweep: median kernel time per row over %d round-robin rounds of %d launches"
             % (args.rounds, args.reps),
             "# command: python -m tiled_matrix_multiplication_gemm_amd.sweep %s" % " ".join(sys.argv[1:]),
             "# device: %s" % torch.cuda.get_device_name(0)]
    ncfg = mg.mg_num_configs()
    for name in args.workloads:
        fn, flops = _setup(name)
        times = {c: [] for c in range(ncfg)}
        for cid in range(ncfg):  # warm every row once
            mg.mg_set_config(cid)
            for _ in range(3):
                fn()
        torch.cuda.synchronize()
        for r in range(args.rounds):
            order = list(range(ncfg)) if r % 2 == 0 else list(reversed(range(ncfg)))
            for cid in order:
                mg.mg_set_config(cid)
                times[cid].append(_time(fn, args.reps))
        mg.mg_set_config(-1)
        for cid in range(ncfg):
            med = statistics.median(times[cid])
            d = mg.mg_config_info(cid)
            lines.append("%-40s row %d %-22s %9.4f ms %8.1f TFLOP/s  (rounds: %s)" % (
                name, cid, d["name"], med, flops / med / 1e9, " ".join("%.4f" % t for t in times[cid])))
        print("\n".join(lines[-ncfg:]), flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    main()
