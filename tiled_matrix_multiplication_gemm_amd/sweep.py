"""Offline sweep of the configuration table, and the table generated from it.

  python -m tiled_matrix_multiplication_gemm_amd.sweep run [--out profiles/table_sweep.json] [--rounds 3]
  python -m tiled_matrix_multiplication_gemm_amd.sweep fit [--json profiles/table_sweep.json]
  python -m tiled_matrix_multiplication_gemm_amd.sweep check
  python -m tiled_matrix_multiplication_gemm_amd.sweep energy [--out FILE] [--seconds 2]
  python -m tiled_matrix_multiplication_gemm_amd.sweep counters [--json profiles/table_sweep.json]

The pages tune a GEMM by benchmarking candidate configurations on the target
and keeping the best one ("Using Triton to optimise GEMM across chips",
section 3.3: top-1 per shape, cached; FlagOS cross-chip page, section 5.2:
target description -> candidates -> compile and time -> pick -> store).
Here the candidates are the compiled rows of the table and the picking is
done once, offline:

`run` (GPU) times every row on a grid of shapes -- the five workloads,
squares, tall-skinny and wide outputs, large K, shapes off the tile grid,
grouped (MoE) problems, batched attention-score products -- forcing each row
through mg_set_config and visiting
the rows round-robin so that clock drift does not favour the rows measured
last; it also times split-K counts on the under-filled shapes, the prepacked
A against the row-major A, and a plain copy (HBM rate).  Each time is a
batch of back-to-back calls captured in a HIP graph and replayed, so the
host's cost per call does not hide the kernels' differences on small
shapes.  Raw times go to a JSON file.

`fit` (CPU) fits the time model of select_config() to those times -- per row
t = ceil(tiles / 256) * BM * BN * K * c / rate_row + ceil(tiles / (256 occ)) * f,
where occ is the number of the row's workgroups one CU holds (its LDS ring
in half the CU's LDS: two), whose K loops hide each other's fill and
epilogue -- and writes csrc/mg_rates.h: the fitted per-row
rates, c and f, the copy rate, the prepacked/plain time ratio per row, and
the measured best row of every swept shape (grouped shapes keyed by their
expert count, batched ones by their entry count), which select_config()
returns for that exact shape (the cache of the pages' top-1) before it
consults the model, and likewise the measured best split count of every
shape timed split, which mg_splitk_choose() returns before its model.  Where the model still misjudges a row (the
epilogue-bound batched products, whose two-workgroup row gains more than
the hidden fixed time), the cache picks the measured best.  The fit and the
generated header are both functions of the JSON alone; `check` regenerates
the header and compares it with the committed one.

`counters` (GPU) records the hardware counters behind the table's choices:
one rocprofv3 --pmc pass per counter group, each running the table's own row
on every swept shape, and stores per shape the MFMA-busy fraction, the LDS
bank-conflict ratio and the L2 hit rate in the JSON (key "counters"; the
generated header does not depend on it).

`energy` (GPU) soaks the 8192^3 bf16 GEMM per variant (tile row, GROUP_M,
XCD renumbering, input data) and records throughput, graphics clock and
socket power: the chip runs this GEMM at its power limit, where throughput
is power divided by energy per flop.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
DEFAULT_JSON = os.path.join(ROOT, "profiles", "table_sweep.json")
HEADER = os.path.join(PKG, "csrc", "mg_rates.h")
CUS = 256

F16, BF16 = 0, 1
# (M, N, K, dtype): the dense shape grid
DENSE_SHAPES = [
    (256, 256, 256, F16), (1024, 1024, 2048, F16), (8192, 8192, 8192, BF16),      # the dense workloads
    (512, 512, 512, F16), (1024, 1024, 1024, F16), (2048, 2048, 2048, F16), (4096, 4096, 4096, BF16),
    (3072, 3072, 3072, F16), (2048, 2048, 8192, BF16), (4096, 1024, 4096, F16), (1024, 4096, 4096, F16),
    (16384, 128, 4096, F16), (65536, 64, 1152, F16), (25088, 128, 1152, F16), (100352, 64, 576, F16),
    (12544, 256, 2304, F16), (256, 16384, 4096, F16), (128, 4096, 16384, BF16),  # tall-skinny and wide
    (256, 256, 65536, BF16), (512, 512, 32768, BF16), (1024, 1024, 16384, F16),  # large K
    (4096, 4096, 4100, F16), (8192, 8190, 8192, BF16), (1000, 1000, 1000, F16), (3000, 5000, 4096, BF16),
    (4096, 11008, 4096, BF16), (4096, 4096, 11008, BF16), (512, 4096, 4096, BF16),  # MLP projections
]
# (E, T, N, K, dtype): grouped problems, balanced routing drawn like the MoE workload
GROUPED_SHAPES = [(32, 8192, 4096, 1024, F16), (8, 2048, 1024, 1024, F16), (64, 16384, 1408, 2048, BF16),
                  (16, 4096, 2048, 512, F16), (8, 8192, 14336, 4096, BF16)]
# (heads, Lq, Lk, d, dtype): attention-score products Q K^T, one batched
# launch over the heads (B given transposed)
BATCHED_SHAPES = [(128, 2048, 2048, 128, BF16), (256, 1024, 1024, 64, F16), (64, 4096, 4096, 128, BF16),
                  (32, 512, 512, 64, F16)]
SPLIT_SHAPES = [(256, 256, 65536, BF16), (512, 512, 32768, BF16), (1024, 1024, 16384, F16),
                (128, 4096, 16384, BF16), (2048, 2048, 16384, BF16), (1024, 1024, 2048, F16)]
PACKED_SHAPES = [(1024, 1024, 2048, F16), (4096, 4096, 4096, BF16), (8192, 8192, 8192, BF16)]
SPLITS = [1, 2, 4, 8, 16]


# ---- GPU side -------------------------------------------------------------------
def _time(fn, target_ms=4.0, rounds=1):
    """Median per-call ms over `rounds` replays of a HIP graph that holds a
    batch of back-to-back calls (HIP events around each replay).  The graph
    keeps the host's cost per call, which at small sizes is larger than the
    kernel, out of the comparison between rows; every timed call writes into
    buffers allocated beforehand, so the captured calls allocate nothing."""
    import torch

    fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    fn()
    e.record()
    torch.cuda.synchronize()
    one = max(s.elapsed_time(e), 1e-3)
    reps = int(min(200, max(3, target_ms / one)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # a call on the capture stream before capturing
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(rounds):
        s.record()
        g.replay()
        e.record()
        torch.cuda.synchronize()
        out.append(s.elapsed_time(e) / reps)
    del g
    return statistics.median(out)


def _dense_tensors(M, N, K, dt, seed):
    import torch

    from tiled_matrix_multiplication_gemm_amd import inputs

    c = inputs.random_dense(M, N, K, dt, seed)
    tdt = torch.float16 if dt == F16 else torch.bfloat16

    def padded(bits, rows, cols):
        import numpy as np

        ld = (cols + 7) // 8 * 8
        full = np.zeros((rows, ld), dtype=np.uint16)
        full[:, :cols] = bits
        return torch.from_numpy(full.view(np.int16)).cuda().view(tdt)[:, :cols]

    A, B = padded(c.A, M, K), padded(c.B, K, N)
    C = torch.empty((M, (N + 7) // 8 * 8), dtype=tdt, device="cuda")[:, :N]
    return A, B, C


def run(out_path, rounds):
    import numpy as np
    import torch

    import tiled_matrix_multiplication_gemm_amd as mg
    from tiled_matrix_multiplication_gemm_amd import inputs

    rows = [r for r in range(mg.mg_num_configs())]
    res = {"device": torch.cuda.get_device_name(0), "rounds": rounds, "cus": CUS,
           "rows": {str(r): mg.mg_config_info(r) for r in rows}, "dense": [], "grouped": [], "batched": [],
           "splitk": [], "packed": []}
    for (M, N, K, dt) in DENSE_SHAPES:
        A, B, C = _dense_tensors(M, N, K, dt, 11 + M % 97 + N % 89 + K % 83)
        times = {r: [] for r in rows}
        for rnd in range(rounds):
            for r in (rows if rnd % 2 == 0 else rows[::-1]):
                mg.mg_set_config(r)
                try:
                    times[r].append(_time(lambda: mg.mg_gemm(A, B, out=C)))
                finally:
                    mg.mg_set_config(-1)
        rec = {"M": M, "N": N, "K": K, "dtype": dt,
               "ms": {str(r): round(statistics.median(v), 5) for r, v in times.items()},
               "table_row_at_sweep": mg.mg_select_config(M, N, K, dt)}
        res["dense"].append(rec)
        print("dense %5d x %5d x %5d: %s" % (M, N, K, " ".join("%d:%.4f" % (r, float(t)) for r, t in
                                                           sorted((int(a), b) for a, b in rec["ms"].items()))),
              flush=True)
        del A, B, C
    for (E, T, N, K, dt) in GROUPED_SHAPES:
        g = inputs.random_grouped(E=E, T=T, K=K, N=N, dtype=dt, seed=300 + E)
        tdt = torch.float16 if dt == F16 else torch.bfloat16
        X = torch.from_numpy(np.ascontiguousarray(g.X).view(np.int16)).cuda().view(tdt)
        W = torch.from_numpy(np.ascontiguousarray(g.W).view(np.int16)).cuda().view(tdt)
        off = torch.from_numpy(g.offsets.astype(np.int32)).cuda()
        Y = torch.empty((T, N), dtype=tdt, device="cuda")
        times = {r: [] for r in rows}
        for rnd in range(rounds):
            for r in (rows if rnd % 2 == 0 else rows[::-1]):
                mg.mg_set_config(r)
                try:
                    times[r].append(_time(lambda: mg.mg_grouped_gemm(X, W, off, out=Y)))
                finally:
                    mg.mg_set_config(-1)
        rec = {"E": E, "T": T, "N": N, "K": K, "dtype": dt, "counts": [int(x) for x in g.counts],
               "ms": {str(r): round(statistics.median(v), 5) for r, v in times.items()}}
        res["grouped"].append(rec)
        print("grouped E=%d T=%d N=%d K=%d: %s" % (E, T, N, K, rec["ms"]), flush=True)
        del X, W, Y
    for (H, Lq, Lk, d, dt) in BATCHED_SHAPES:
        tdt = torch.float16 if dt == F16 else torch.bfloat16
        q = (torch.randn((H, Lq, d), device="cuda") * d ** -0.25).to(tdt)
        k = (torch.randn((H, Lk, d), device="cuda") * d ** -0.25).to(tdt)
        S = torch.empty((H, Lq, Lk), dtype=tdt, device="cuda")
        times = {r: [] for r in rows}
        for rnd in range(rounds):
            for r in (rows if rnd % 2 == 0 else rows[::-1]):
                mg.mg_set_config(r)
                try:
                    times[r].append(_time(lambda: mg.mg_attention_scores(q, k, out=S)))
                except RuntimeError:
                    pass  # a row without a direct-to-LDS kernel refuses the transposed K
                finally:
                    mg.mg_set_config(-1)
        rec = {"batch": H, "M": Lq, "N": Lk, "K": d, "dtype": dt,
               "ms": {str(r): round(statistics.median(v), 5) for r, v in times.items() if v}}
        res["batched"].append(rec)
        print("batched %d x %d x %d x %d: %s" % (H, Lq, Lk, d, rec["ms"]), flush=True)
        del q, k, S
    for (M, N, K, dt) in SPLIT_SHAPES:
        A, B, C = _dense_tensors(M, N, K, dt, 77 + K % 101)
        ms = {}
        for s in SPLITS:
            if s == 1:
                ms["1"] = round(_time(lambda: mg.mg_gemm(A, B, out=C), rounds=rounds), 5)
            else:
                ws = torch.empty((mg.mg_splitk_workspace_bytes(M, N, s),), dtype=torch.uint8, device="cuda")
                ms[str(s)] = round(_time(lambda: mg.mg_gemm_splitk(A, B, splits=s, workspace=ws, out=C),
                                         rounds=rounds), 5)
                del ws
        res["splitk"].append({"M": M, "N": N, "K": K, "dtype": dt, "ms": ms})
        print("split-K %d x %d x %d: %s" % (M, N, K, ms), flush=True)
        del A, B, C
    for (M, N, K, dt) in PACKED_SHAPES:
        A, B, C = _dense_tensors(M, N, K, dt, 55 + K % 101)
        rec = {"M": M, "N": N, "K": K, "dtype": dt, "plain_ms": {}, "packed_ms": {}}
        for r in rows:
            d = mg.mg_config_info(r)
            if not d["direct_lds"] or d["direct_ksplit"] > 1:
                continue
            mg.mg_set_config(r)
            try:
                BK = d["bk"]
                Ap = mg.mg_prepack_a(A, BK)
                plain, packed = [], []
                for rnd in range(rounds):
                    plain.append(_time(lambda: mg.mg_gemm(A, B, out=C)))
                    packed.append(_time(lambda: mg.mg_gemm_prepacked(Ap, BK, B, M, K, out=C)))
                rec["plain_ms"][str(r)] = round(statistics.median(plain), 5)
                rec["packed_ms"][str(r)] = round(statistics.median(packed), 5)
                if r == 0:
                    rec["copy_ms"] = round(_time(lambda: mg.mg_prepack_a(A, BK, out=Ap), rounds=rounds), 5)
                    rec["copy_bytes"] = 2 * M * K + 2 * ((K + BK - 1) // BK) * M * BK
                del Ap
            finally:
                mg.mg_set_config(-1)
        res["packed"].append(rec)
        print("packed %d x %d x %d: plain %s packed %s copy %s" % (M, N, K, rec["plain_ms"], rec["packed_ms"],
                                                                 rec.get("copy_ms")), flush=True)
        del A, B, C
    n = 1 << 27
    src = torch.ones(n, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    cms = _time(lambda: dst.copy_(src), rounds=rounds)
    res["copy"] = {"bytes": 4 * n, "ms": round(cms, 5), "gbs": round(4 * n / (cms * 1e-3) / 1e9, 1)}
    with open(out_path, "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
    print("wrote", out_path)


# ---- counters of the table's choices ----------------------------------------------
# One rocprofv3 --pmc pass per group (each group is collected in one pass by
# the hardware); every pass runs the same fixed sequence of GEMMs.
COUNTER_PASSES = [
    ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE"],
    ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE"],
    ["TCC_HIT_sum", "TCC_MISS_sum"],
]
COUNTER_CALLS = 2  # calls per shape; the counters of the last one are kept


def _device_dense(M, N, K, dt):
    """Random operands drawn on the device, rows padded to 16 bytes (the
    counters do not depend on the values, and drawing the largest shapes on
    the host would dominate each pass)."""
    import torch

    tdt = torch.float16 if dt == F16 else torch.bfloat16

    def mat(rows, cols, scale):
        ld = (cols + 7) // 8 * 8
        return (torch.randn((rows, ld), device="cuda") * scale).to(tdt)[:, :cols]

    A, B = mat(M, K, K ** -0.5), mat(K, N, 1.0)
    C = torch.empty((M, (N + 7) // 8 * 8), dtype=tdt, device="cuda")[:, :N]
    return A, B, C


def counters_run(json_path, order_path):
    """(GPU, under rocprofv3 --pmc) COUNTER_CALLS calls of every swept shape
    with the row the table picks, dense shapes then grouped ones in the
    JSON's order; writes that order with the row and kernel family used."""
    import numpy as np
    import torch

    import tiled_matrix_multiplication_gemm_amd as mg

    with open(json_path) as f:
        data = json.load(f)
    torch.manual_seed(0)
    order = []
    for rec in data["dense"]:
        M, N, K, dt = rec["M"], rec["N"], rec["K"], rec["dtype"]
        A, B, C = _device_dense(M, N, K, dt)
        for _ in range(COUNTER_CALLS):
            mg.mg_gemm(A, B, out=C)
        torch.cuda.synchronize()
        order.append({"M": M, "N": N, "K": K, "dtype": dt, "E": 0, "B": 1, "row": mg.mg_last_config(),
                      "family": mg.mg_last_kernel()})
        print("counters: dense %d x %d x %d row %d" % (M, N, K, order[-1]["row"]), flush=True)
        del A, B, C
    for rec in data["grouped"]:
        E, T, N, K, dt = rec["E"], rec["T"], rec["N"], rec["K"], rec["dtype"]
        tdt = torch.float16 if dt == F16 else torch.bfloat16
        X = torch.randn((T, K), device="cuda").to(tdt)
        W = (torch.randn((E, K, N), device="cuda") * 0.02).to(tdt)
        off = torch.from_numpy(np.concatenate([[0], np.cumsum(rec["counts"])]).astype(np.int32)).cuda()
        Y = torch.empty((T, N), dtype=tdt, device="cuda")
        for _ in range(COUNTER_CALLS):
            mg.mg_grouped_gemm(X, W, off, out=Y)
        torch.cuda.synchronize()
        order.append({"M": T, "N": N, "K": K, "dtype": dt, "E": E, "B": 1, "row": mg.mg_last_config(),
                      "family": mg.mg_last_kernel()})
        print("counters: grouped E=%d T=%d N=%d K=%d row %d" % (E, T, N, K, order[-1]["row"]), flush=True)
        del X, W, Y
    for rec in data.get("batched", []):
        H, Lq, Lk, d, dt = rec["batch"], rec["M"], rec["N"], rec["K"], rec["dtype"]
        tdt = torch.float16 if dt == F16 else torch.bfloat16
        q = (torch.randn((H, Lq, d), device="cuda") * d ** -0.25).to(tdt)
        k = (torch.randn((H, Lk, d), device="cuda") * d ** -0.25).to(tdt)
        S = torch.empty((H, Lq, Lk), dtype=tdt, device="cuda")
        for _ in range(COUNTER_CALLS):
            mg.mg_attention_scores(q, k, out=S)
        torch.cuda.synchronize()
        order.append({"M": Lq, "N": Lk, "K": d, "dtype": dt, "E": 0, "B": H, "row": mg.mg_last_config(),
                      "family": mg.mg_last_kernel()})
        print("counters: batched %d x %d x %d x %d row %d" % (H, Lq, Lk, d, order[-1]["row"]), flush=True)
        del q, k, S
    with open(order_path, "w") as f:
        json.dump(order, f)


def derived_counters(v):
    """MFMA-busy fraction, LDS bank-conflict ratio and L2 hit rate from one
    dispatch's summed counters (those whose inputs are present)."""
    from tiled_matrix_multiplication_gemm_amd.profiling import SHADER_ENGINES, SIMDS

    out = {}
    if v.get("SQ_BUSY_CYCLES") and "SQ_VALU_MFMA_BUSY_CYCLES" in v:
        out["mfma_busy_fraction"] = round((v["SQ_VALU_MFMA_BUSY_CYCLES"] / SIMDS) /
                                          (v["SQ_BUSY_CYCLES"] / SHADER_ENGINES), 4)
    if "SQ_LDS_BANK_CONFLICT" in v and "SQ_LDS_IDX_ACTIVE" in v:
        out["lds_bank_conflict_ratio"] = round(v["SQ_LDS_BANK_CONFLICT"] / max(v["SQ_LDS_IDX_ACTIVE"], 1.0), 4)
    if "TCC_HIT_sum" in v and "TCC_MISS_sum" in v:
        out["l2_hit_rate"] = round(v["TCC_HIT_sum"] / max(v["TCC_HIT_sum"] + v["TCC_MISS_sum"], 1.0), 4)
    return out


def merge_counter_rows(order, passes):
    """Attach counters to the shapes of `order`.  `passes` holds, per pass,
    the rows of its counter_collection CSV (dicts with Dispatch_Id,
    Kernel_Name, Counter_Name, Counter_Value).  The GEMM dispatches of a pass
    (kernel names holding "gemm_"), in dispatch order, are COUNTER_CALLS per
    shape of `order`; the last call of each shape is kept.  Every pass must
    see the same kernels."""
    vals = [dict() for _ in order]
    names = [None] * len(order)
    for rows in passes:
        disp = {}
        for r in rows:
            if "gemm_" not in r["Kernel_Name"]:
                continue
            name, v = disp.setdefault(int(r["Dispatch_Id"]), (r["Kernel_Name"], {}))
            v[r["Counter_Name"]] = v.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        ids = sorted(disp)
        if len(ids) != COUNTER_CALLS * len(order):
            raise RuntimeError("%d GEMM dispatches for %d shapes" % (len(ids), len(order)))
        for i in range(len(order)):
            name, v = disp[ids[COUNTER_CALLS * (i + 1) - 1]]
            if names[i] is not None and names[i] != name:
                raise RuntimeError("passes ran different kernels for shape %d" % i)
            names[i] = name
            vals[i].update(v)
    out = []
    for o, v, name in zip(order, vals, names):
        rec = dict(o)
        rec["kernel"] = name
        rec["values"] = {k: round(x, 1) for k, x in sorted(v.items())}
        rec.update(derived_counters(v))
        out.append(rec)
    return out


def counters(json_path, work_dir, timeout_s):
    """Run the counter passes as child processes (rocprofv3 wraps the
    program directly) and merge their counters into the JSON."""
    from tiled_matrix_multiplication_gemm_amd.profiling import _counter_rows

    os.makedirs(work_dir, exist_ok=True)
    order_path = os.path.join(work_dir, "counter_order.json")
    passes, cmds = [], []
    for i, group in enumerate(COUNTER_PASSES):
        d = os.path.join(work_dir, "pmc_%d" % i)
        cmd = ["timeout", "-s", "KILL", str(timeout_s), "rocprofv3", "--pmc", *group, "--output-format", "csv",
               "-d", d, "-o", "run", "--", sys.executable, "-m", "tiled_matrix_multiplication_gemm_amd.sweep",
               "counters-run", "--json", json_path, "--order", order_path]
        shown = " ".join(cmd).replace(sys.executable, "python").replace(ROOT + os.sep, "")
        print("pass %d: %s" % (i, shown), flush=True)
        if os.path.exists(order_path):
            os.remove(order_path)
        rc = subprocess.run(cmd, cwd=ROOT).returncode
        # rocprofv3 itself may end abnormally after the program has finished
        # and written its results; the pass counts if both are there
        if not os.path.exists(order_path):
            raise SystemExit("counter pass %d failed (exit %d) before the program finished" % (i, rc))
        if rc != 0:
            print("pass %d: profiler exit %d after the program finished; results kept" % (i, rc), flush=True)
        passes.append(_counter_rows(d))
        cmds.append(shown)
    with open(order_path) as f:
        order = json.load(f)
    with open(json_path) as f:
        data = json.load(f)
    data["counters"] = {"commands": cmds, "calls_per_shape": COUNTER_CALLS,
                        "shapes": merge_counter_rows(order, passes)}
    with open(json_path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    for r in data["counters"]["shapes"]:
        print("%6d x %5d x %5d E=%2d B=%3d row %d  mfma busy %s  lds conflicts %s  l2 hit %s" % (
            r["M"], r["N"], r["K"], r["E"], r.get("B", 1), r["row"], r.get("mfma_busy_fraction"),
            r.get("lds_bank_conflict_ratio"), r.get("l2_hit_rate")), flush=True)


# (label, row, GROUP_M, XCD renumbering, inputs) of the 8192^3 bf16 GEMM
ENERGY_VARIANTS = [
    ("table: 256x256, 8 waves, GROUP_M 4, XCD on", 0, 4, 1, "float"),
    ("GROUP_M 8", 0, 8, 1, "float"),
    ("GROUP_M 16", 0, 16, 1, "float"),
    ("GROUP_M 32", 0, 32, 1, "float"),
    ("GROUP_M 1 (row-major tile order)", 0, 1, 1, "float"),
    ("XCD renumbering off", 0, 4, 0, "float"),
    ("256x256, 4 waves of 128x128 (row 6)", 6, 4, 1, "float"),
    ("128x256 (row 3)", 3, 4, 1, "float"),
    ("256x128 (row 4)", 4, 4, 1, "float"),
    ("inputs: integers in [-4, 4]", 0, 4, 1, "int"),
    ("inputs: all zeros", 0, 4, 1, "zeros"),
]


def energy(out_path, seconds, cmdline):
    """Throughput, graphics clock and socket power of the 8192^3 bf16 GEMM per
    variant (tile row, raster, input data), each soaked back to back for
    `seconds` with amdsmi sampled beside it; variants in forward then reverse
    order, the two soaks' medians averaged.  At the power limit the energy
    per flop is power / throughput."""
    import numpy as np
    import torch

    import tiled_matrix_multiplication_gemm_amd as mg
    from tiled_matrix_multiplication_gemm_amd import inputs, profiling

    c = inputs.dense_workload("gemm_8192_bf16", "float")
    ci = inputs.dense_workload("gemm_8192_bf16", "int")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    data = {"float": (up(c.A), up(c.B)), "int": (up(ci.A), up(ci.B))}
    data["zeros"] = (torch.zeros_like(data["float"][0]), torch.zeros_like(data["float"][1]))
    C = torch.empty((8192, 8192), dtype=torch.bfloat16, device="cuda")
    flops = 2.0 * 8192 ** 3
    res = {v[0]: [] for v in ENERGY_VARIANTS}
    for order in (ENERGY_VARIANTS, ENERGY_VARIANTS[::-1]):
        for (label, row, gm, xcd, kind) in order:
            A, B = data[kind]
            mg.mg_set_config(row)
            mg.mg_set_raster(gm, xcd)
            try:
                for _ in range(20):
                    mg.mg_gemm(A, B, out=C)
                t = profiling.soak_telemetry(lambda: mg.mg_gemm(A, B, out=C), seconds, with_rate=True)
            finally:
                mg.mg_set_config(-1)
                mg.mg_set_raster(-1, -1)
            if t is None:
                raise RuntimeError("amdsmi telemetry is not available")
            res[label].append(t)
            print("%-45s %.4f ms %s MHz %s W" % (label, t["ms_per_call"], t["gfx_clock_mhz"], t["socket_power_w"]),
                  flush=True)
    lines = ["# 8192^3 bf16 GEMM per variant: back-to-back calls soaked for %.1f s each, variants in forward then"
             " reverse order (mean of the two soaks); clock and socket power: amdsmi medians over the second half"
             " of each soak; energy per flop = power / throughput" % seconds,
             "# command: %s" % cmdline,
             "# device: %s" % torch.cuda.get_device_name(0),
             "%-45s %9s %9s %9s %8s %9s" % ("variant", "ms", "TFLOP/s", "MHz", "W", "pJ/flop")]
    for (label, *_rest) in ENERGY_VARIANTS:
        v = res[label]
        ms = sum(x["ms_per_call"] for x in v) / len(v)
        mhz = sum(x["gfx_clock_mhz"] or 0 for x in v) / len(v)
        w = sum(x["socket_power_w"] or 0 for x in v) / len(v)
        tf = flops / (ms * 1e-3) / 1e12
        lines.append("%-45s %9.4f %9.1f %9.0f %8.0f %9.3f" % (label, ms, tf, mhz, w, w / (tf * 1e12) * 1e12))
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ---- the fit (CPU) -------------------------------------------------------------
def _cdiv(a, b):
    return -(-a // b)


LDS_PER_CU = 160 * 1024


def _occupancy(data, r):
    """Workgroups of row r that one CU runs at once: as many of its LDS rings
    as fit in the CU's 160 KB, at most two (the waves of every row fit the
    registers of two workgroups)."""
    return max(1, min(2, LDS_PER_CU // int(data["rows"][str(r)]["direct_lds_bytes"])))


def _model_rows(data):
    """Rows the model chooses among: those with a pipelined direct-to-LDS kernel."""
    out = []
    for k, d in sorted(data["rows"].items(), key=lambda kv: int(kv[0])):
        if d["direct_lds"] and d["direct_ksplit"] == 1:
            out.append((int(k), d["bm"], d["bn"]))
    return out


def grouped_tiles(T, E, N, bm, bn):
    """Tiles of a grouped problem with balanced routing (the host does not
    read the device offsets): E experts of T / E rows each."""
    rows_per = _cdiv(T, max(E, 1))
    return max(E, 1) * _cdiv(rows_per, bm) * _cdiv(N, bn)


def fit(data):
    """Per-row relative rates, the seconds per output element and k of a
    256 x 256 tile (c) and the fixed time per round of tiles (f), fitted to
    the dense times by alternating least squares on relative error.  Each CU
    works through ceil(tiles / CUs) tiles; a row that holds two workgroups
    per CU pays the fixed time (ring fill, epilogue) once per two of them,
    since the other workgroup's K loop runs beside it."""
    rows = _model_rows(data)
    obs = []  # (row, bm, bn, tiles per CU, rounds, K, seconds)
    for rec in data["dense"]:
        for (r, bm, bn) in rows:
            t = rec["ms"].get(str(r))
            if t is None:
                continue
            tiles = _cdiv(rec["M"], bm) * _cdiv(rec["N"], bn)
            obs.append((r, bm, bn, _cdiv(tiles, data["cus"]), _cdiv(tiles, data["cus"] * _occupancy(data, r)),
                        rec["K"], float(t) * 1e-3))
    rate = {r: 1.0 for (r, _, _) in rows}
    c, f = 0.205e-3 / (65536.0 * 8192.0), 3e-6
    for _ in range(50):
        # c, f by weighted linear least squares on t = a c + b f (a: work, b: rounds), weights 1 / t^2
        saa = sab = sbb = sat = sbt = 0.0
        for (r, bm, bn, per_cu, rnd, K, t) in obs:
            a = per_cu * bm * bn * K / rate[r]
            w = 1.0 / (t * t)
            saa += w * a * a
            sab += w * a * rnd
            sbb += w * rnd * rnd
            sat += w * a * t
            sbt += w * rnd * t
        det = saa * sbb - sab * sab
        c = (sat * sbb - sab * sbt) / det
        f = max(0.0, (saa * sbt - sab * sat) / det)
        # rates: median over shapes of the implied rate (row 0 fixed at 1)
        for (r, _, _) in rows:
            imp = [per_cu * bm * bn * K * c / max(t - rnd * f, 1e-9)
                   for (rr, bm, bn, per_cu, rnd, K, t) in obs if rr == r]
            rate[r] = statistics.median(imp) if imp else 1.0
        base = rate[rows[0][0]]
        for r in rate:
            rate[r] /= base
    return {"rate": {str(r): round(rate[r], 4) for r in rate}, "c": c, "f": f}


def model_seconds(F, data, r, bm, bn, tiles, K):
    """Modelled time of `tiles` tiles of row r with K-deep products."""
    cus = data["cus"]
    return (_cdiv(tiles, cus) * bm * bn * K * F["c"] / F["rate"][str(r)] +
            _cdiv(tiles, cus * _occupancy(data, r)) * F["f"])


def model_pick(data, F, M, N, K, E=0):
    best, best_t = None, None
    for (r, bm, bn) in _model_rows(data):
        tiles = grouped_tiles(M, E, N, bm, bn) if E else _cdiv(M, bm) * _cdiv(N, bn)
        t = model_seconds(F, data, r, bm, bn, tiles, K)
        if best_t is None or t < best_t:
            best, best_t = r, t
    return best


def packed_ratio(data):
    """packed time / plain time per row (median over the swept shapes)."""
    per = {}
    for rec in data["packed"]:
        for r, p in rec["packed_ms"].items():
            per.setdefault(r, []).append(p / rec["plain_ms"][r])
    return {r: round(statistics.median(v), 4) for r, v in per.items()}


def copy_rate(data):
    """Bytes per second of the blocking copy (mg_prepack_a), median over shapes."""
    v = [rec["copy_bytes"] / (rec["copy_ms"] * 1e-3) for rec in data["packed"] if "copy_ms" in rec]
    return statistics.median(v)


def summarize(data):
    """The fit, the best row of every swept shape, and how the model does."""
    F = fit(data)
    nrows = len(data["rows"])
    best = []
    lost = []
    agree = 0
    for rec in data["dense"]:
        ms = {int(r): float(t) for r, t in rec["ms"].items() if int(r) in dict((a, 0) for a, _, _ in _model_rows(data))}
        b = min(ms, key=lambda r: ms[r])
        m = model_pick(data, F, rec["M"], rec["N"], rec["K"])
        agree += m == b
        lost.append(ms[m] / ms[b] - 1.0)
        best.append({"M": rec["M"], "N": rec["N"], "K": rec["K"], "dtype": rec["dtype"], "best_row": b,
                     "best_ms": ms[b], "model_row": m, "model_ms": ms[m]})
    gbest = []
    for rec in data["grouped"]:
        ms = {int(r): float(t) for r, t in rec["ms"].items() if int(r) in dict((a, 0) for a, _, _ in _model_rows(data))}
        b = min(ms, key=lambda r: ms[r])
        m = model_pick(data, F, rec["T"], rec["N"], rec["K"], rec["E"])
        gbest.append({"E": rec["E"], "T": rec["T"], "N": rec["N"], "K": rec["K"], "dtype": rec["dtype"],
                      "best_row": b, "best_ms": ms[b], "model_row": m, "model_ms": ms[m]})
    bbest = []
    for rec in data.get("batched", []):
        ms = {int(r): float(t) for r, t in rec["ms"].items() if int(r) in dict((a, 0) for a, _, _ in _model_rows(data))}
        b = min(ms, key=lambda r: ms[r])
        bbest.append({"batch": rec["batch"], "M": rec["M"], "N": rec["N"], "K": rec["K"], "dtype": rec["dtype"],
                      "best_row": b, "best_ms": ms[b]})
    sbest = []
    for rec in data.get("splitk", []):
        ms = {int(s): float(t) for s, t in rec["ms"].items()}
        sbest.append({"M": rec["M"], "N": rec["N"], "K": rec["K"], "splits": min(ms, key=lambda s: ms[s])})
    return {"fit": F, "rows": nrows, "dense_best": best, "grouped_best": gbest, "batched_best": bbest,
            "splitk_best": sbest,
            "model_agrees": "%d of %d dense shapes" % (agree, len(best)),
            "model_time_lost_max": round(max(lost), 4), "model_time_lost_median": round(statistics.median(lost), 4),
            "packed_ratio": packed_ratio(data), "copy_bytes_per_s": copy_rate(data),
            "splitk": splitk_fit(data, F)}


def splitk_fit(data, F):
    """Rate at which split partials are written and read back (bytes / s):
    the extra time of the best split over its kernel time in the model."""
    vals = []
    for rec in data["splitk"]:
        for s, t in rec["ms"].items():
            s = int(s)
            if s == 1:
                continue
            extra_bytes = 2.0 * s * rec["M"] * rec["N"] * 4
            # kernel part from the model with the row split-K picks (the model's best of rows 0-2)
            tk = min(model_seconds(F, data, r, bm, bn, _cdiv(rec["M"], bm) * _cdiv(rec["N"], bn) * s, rec["K"] / s)
                     for (r, bm, bn) in _model_rows(data) if r in (0, 1, 2))
            extra = float(t) * 1e-3 - tk
            if extra > 0:
                vals.append(extra_bytes / extra)
    return {"partial_bytes_per_s": statistics.median(vals) if vals else 4e12}


def header_text(data, json_rel):
    S = summarize(data)
    F = S["fit"]
    rows = _model_rows(data)
    lines = [
        "// Generated by `python -m tiled_matrix_multiplication_gemm_amd.sweep fit` from %s" % json_rel,
        "// (timings of every table row on MI355X); do not edit by hand.  The time",
        "// model of select_config(): t = ceil(tiles / 256) * BM * BN * K * kSecPerElemK / rate",
        "// + ceil(tiles / (256 * occ)) * kFixedSec, occ = workgroups per CU; exact shapes of the",
        "// sweep return their measured best row.",
        "#pragma once",
        "",
        "#include <stdint.h>",
        "",
        "namespace mg {",
        "namespace rates {",
        "",
        "struct RowRate {",
        "    int id, bm, bn;",
        "    int occ;      // workgroups one CU runs at once",
        "    double rate;  // per-CU output rate relative to row %d" % rows[0][0],
        "};",
        "inline constexpr RowRate kRows[] = {",
    ]
    for (r, bm, bn) in rows:
        lines.append("    {%d, %d, %d, %d, %.4f}," % (r, bm, bn, _occupancy(data, r), F["rate"][str(r)]))
    lines += ["};",
              "inline constexpr double kSecPerElemK = %.6e;  // one output element times one k, rate 1" % F["c"],
              "inline constexpr double kFixedSec = %.6e;     // per round of tiles: fill, drain, epilogue" % F["f"],
              "inline constexpr double kCopyBytesPerSec = %.6e;  // the blocking copy of A" % S["copy_bytes_per_s"],
              "inline constexpr double kPartialBytesPerSec = %.6e;  // split-K partials, written and read" %
              S["splitk"]["partial_bytes_per_s"],
              "// packed-A time / row-major time, per row (-1: not measured)",
              "inline constexpr double kPackedRatio[] = {%s};" % ", ".join(
                  "%.4f" % S["packed_ratio"].get(str(r), -1.0) for r in range(S["rows"])),
              "",
              "struct Swept {",
              "    int64_t M, N, K;",
              "    int32_t experts;  // 0: dense",
              "    int64_t batch;    // entries of a batched product (1: one)",
              "    int32_t row;",
              "};",
              "// the measured best row of every swept shape (cached top-1)",
              "inline constexpr Swept kSwept[] = {"]
    for b in S["dense_best"]:
        lines.append("    {%d, %d, %d, 0, 1, %d}," % (b["M"], b["N"], b["K"], b["best_row"]))
    for b in S["grouped_best"]:
        lines.append("    {%d, %d, %d, %d, 1, %d}," % (b["T"], b["N"], b["K"], b["E"], b["best_row"]))
    for b in S["batched_best"]:
        lines.append("    {%d, %d, %d, 0, %d, %d}," % (b["M"], b["N"], b["K"], b["batch"], b["best_row"]))
    lines += ["};", "",
              "struct SweptSplit {",
              "    int64_t M, N, K;",
              "    int32_t splits;",
              "};",
              "// the measured best split count of every shape the sweep timed split (cached top-1)",
              "inline constexpr SweptSplit kSweptSplit[] = {"]
    for b in S["splitk_best"]:
        lines.append("    {%d, %d, %d, %d}," % (b["M"], b["N"], b["K"], b["splits"]))
    lines += ["};", "", "}  // namespace rates", "}  // namespace mg", ""]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("run")
    a.add_argument("--out", default=DEFAULT_JSON)
    a.add_argument("--rounds", type=int, default=3)
    b = sub.add_parser("fit")
    b.add_argument("--json", default=DEFAULT_JSON)
    c = sub.add_parser("check")
    c.add_argument("--json", default=DEFAULT_JSON)
    e = sub.add_parser("energy")
    e.add_argument("--out", default=os.path.join(ROOT, "profiles", "gemm_8192_bf16_energy.txt"))
    e.add_argument("--seconds", type=float, default=2.0)
    g = sub.add_parser("counters")
    g.add_argument("--json", default=DEFAULT_JSON)
    g.add_argument("--work", default=os.path.join(ROOT, "gpurun_out", "sweep_counters"))
    g.add_argument("--timeout", type=int, default=300)
    h = sub.add_parser("counters-run")
    h.add_argument("--json", default=DEFAULT_JSON)
    h.add_argument("--order", required=True)
    args = ap.parse_args()
    if args.what == "run":
        run(args.out, args.rounds)
        return
    if args.what == "counters":
        counters(os.path.abspath(args.json), os.path.abspath(args.work), args.timeout)
        return
    if args.what == "counters-run":
        counters_run(args.json, args.order)
        return
    if args.what == "energy":
        energy(args.out, args.seconds, "python -m tiled_matrix_multiplication_gemm_amd.sweep " + " ".join(sys.argv[1:]))
        return
    with open(args.json) as f:
        data = json.load(f)
    rel = os.path.relpath(args.json, ROOT)
    text = header_text(data, rel)
    if args.what == "fit":
        with open(HEADER, "w") as f:
            f.write(text)
        S = summarize(data)
        print(json.dumps({k: v for k, v in S.items() if k not in ("dense_best", "grouped_best")}, indent=1))
    else:
        with open(HEADER) as f:
            ok = f.read() == text
        print("mg_rates.h matches the sweep" if ok else "mg_rates.h differs from the sweep")
        sys.exit(0 if ok else 1)


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    main()
