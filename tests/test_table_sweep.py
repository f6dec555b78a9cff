"""The configuration table is a product of the offline sweep.

profiles/table_sweep.json holds the times of every row on every swept shape
(measured on MI355X by `sweep run`); csrc/mg_rates.h is generated from it by
`sweep fit`.  These CPU tests check that the committed header is exactly
what the fit produces from the committed JSON, that the compiled library
picks the measured best row for every swept shape, that off-sweep shapes get
the model's choice (recomputed here in Python from the JSON alone), and that
the split-K count and the layout planner's decision follow the same model.
"""
import json
import math
import os
import re

import pytest

import tiled_matrix_multiplication_gemm_amd as mg
from tiled_matrix_multiplication_gemm_amd import sweep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def data():
    with open(os.path.join(ROOT, "profiles", "table_sweep.json")) as f:
        return json.load(f)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mg.LIB_PATH):
        pytest.skip("library not built")
    L = mg.lib()
    L.mg_set_config(-1)
    return L


def test_header_is_generated_from_the_json(data):
    with open(sweep.HEADER) as f:
        assert f.read() == sweep.header_text(data, os.path.relpath(sweep.DEFAULT_JSON, sweep.ROOT))


def test_occupancy_follows_the_lds_ring(data):
    """The model counts two workgroups per CU for exactly the rows whose
    direct-to-LDS ring fits in half of a CU's 160 KB, and the generated
    header carries the same counts."""
    occ = {r: sweep._occupancy(data, r) for r, _, _ in sweep._model_rows(data)}
    for r, o in occ.items():
        lds = int(data["rows"][str(r)]["direct_lds_bytes"])
        assert o == (2 if 2 * lds <= 160 * 1024 else 1), (r, lds, o)
    assert {r for r, o in occ.items() if o == 2} == {1, 2, 4, 9}
    text = open(os.path.join(ROOT, "tiled_matrix_multiplication_gemm_amd", "csrc", "mg_rates.h")).read()
    for r, o in occ.items():
        assert re.search(r"\{%d, \d+, \d+, %d, [0-9.]+\}," % (r, o), text), (r, o)


def test_every_swept_shape_takes_its_measured_best_row(data, L):
    S = sweep.summarize(data)
    model = {r for r, _, _ in sweep._model_rows(data)}  # rows with the one-ring direct-to-LDS kernel
    for b in S["dense_best"]:
        ms = {int(r): t for r, t in next(r for r in data["dense"] if (r["M"], r["N"], r["K"]) ==
                                         (b["M"], b["N"], b["K"]))["ms"].items()}
        assert ms[b["best_row"]] == min(ms[r] for r in ms if r in model)
        assert L.mg_select_config(b["M"], b["N"], b["K"], b["dtype"], 0, 1) == b["best_row"], b
    for b in S["grouped_best"]:
        assert L.mg_select_config(b["T"], b["N"], b["K"], b["dtype"], b["E"], 1) == b["best_row"], b
    assert S["batched_best"], "the sweep times batched (attention-score) shapes"
    for b in S["batched_best"]:
        ms = next(r for r in data["batched"] if (r["batch"], r["M"], r["N"], r["K"]) ==
                  (b["batch"], b["M"], b["N"], b["K"]))["ms"]
        assert float(ms[str(b["best_row"])]) == min(float(t) for r, t in ms.items() if int(r) in model)
        assert L.mg_select_config(b["M"], b["N"], b["K"], b["dtype"], 0, b["batch"]) == b["best_row"], b
        # the same shape as one dense problem is not the cached batched one
        assert L.mg_select_config(b["M"], b["N"], b["K"], b["dtype"], 0, 1) == sweep.model_pick(
            data, sweep.fit(data), b["M"], b["N"], b["K"]) or (b["M"], b["N"], b["K"]) in {
            (d["M"], d["N"], d["K"]) for d in data["dense"]}


OFF_SWEEP = [(8192, 4096, 4096), (777, 1300, 960), (100000, 96, 2048), (64, 64, 64), (2560, 2560, 2560),
             (16384, 16384, 1024), (300, 9000, 4096), (1, 1, 1)]


@pytest.mark.parametrize("M,N,K", OFF_SWEEP)
def test_off_sweep_shapes_take_the_models_choice(data, L, M, N, K):
    F = sweep.fit(data)
    assert L.mg_select_config(M, N, K, 0, 0, 1) == sweep.model_pick(data, F, M, N, K)


@pytest.mark.parametrize("E,T,N,K", [(4, 1000, 512, 256), (128, 65536, 2048, 1024), (32, 8192, 1024, 4096)])
def test_grouped_shapes_take_the_models_choice(data, L, E, T, N, K):
    F = sweep.fit(data)
    assert L.mg_select_config(T, N, K, 0, E, 1) == sweep.model_pick(data, F, T, N, K, E)


def _py_splitk_choose(data, M, N, K):
    F = sweep.fit(data)
    S = sweep.summarize(data)
    for b in S["splitk_best"]:
        if (b["M"], b["N"], b["K"]) == (M, N, K):
            return b["splits"]
    rows = [x for x in sweep._model_rows(data) if x[0] in (0, 1, 2)]
    best_s, best_t = 1, 0.0
    s = 1
    while s <= 64:
        if s > 1 and K // s < 256:
            break
        t = min(sweep.model_seconds(F, data, r, bm, bn, sweep._cdiv(M, bm) * sweep._cdiv(N, bn) * s,
                                    sweep._cdiv(K, s)) for (r, bm, bn) in rows)
        if s > 1:
            t += 2.0 * s * M * N * 4.0 / S["splitk"]["partial_bytes_per_s"]
        if best_t == 0.0 or t < best_t * 0.95:
            best_t, best_s = t, s
        s *= 2
    return best_s


@pytest.mark.parametrize("M,N,K", [(256, 256, 65536), (512, 512, 32768), (1024, 1024, 16384), (128, 4096, 16384),
                                   (2048, 2048, 16384), (1024, 1024, 2048), (8192, 8192, 8192),
                                   (384, 384, 24576), (768, 1536, 12288), (4096, 512, 8192)])
def test_split_count_follows_the_model(data, L, M, N, K):
    """Swept shapes take their measured best count, the others the model's."""
    assert L.mg_splitk_choose(M, N, K) == _py_splitk_choose(data, M, N, K)


def test_split_choice_against_the_measured_times(data, L):
    """Where the sweep timed split counts, the chosen count is within 35 % of
    the fastest measured one, and never splits an output that fills the GPU."""
    for rec in data["splitk"]:
        ms = {int(s): t for s, t in rec["ms"].items()}
        s = L.mg_splitk_choose(rec["M"], rec["N"], rec["K"])
        if s in ms:
            assert ms[s] <= 1.35 * min(ms.values()), (rec, s)
    assert L.mg_splitk_choose(8192, 8192, 8192) == 1


def test_layout_planner_gate(data, L):
    """The planner prepacks only where the sweep measured the blocked A
    faster on the chosen row, after enough reuses to pay for the copy."""
    S = sweep.summarize(data)
    ratio = {int(r): v for r, v in S["packed_ratio"].items()}
    F = S["fit"]
    rows = {r: (bm, bn) for (r, bm, bn) in sweep._model_rows(data)}
    for (M, N, K) in [(1024, 1024, 2048), (8192, 8192, 8192), (4096, 4096, 4096), (2048, 2048, 2048),
                      (12544, 256, 2304), (65536, 64, 1152), (777, 1300, 960)]:
        got = L.mg_prepack_uses_to_pay(M, N, K, 0)
        row = L.mg_select_config(M, N, K, 0, 0, 1)
        if ratio.get(row, -1.0) <= 0.0 or ratio[row] >= 1.0:
            assert got == -1, (M, N, K, row)
            continue
        bm, bn = rows[row]
        t = sweep.model_seconds(F, data, row, bm, bn, sweep._cdiv(M, bm) * sweep._cdiv(N, bn), K)
        bk = mg.mg_config_info(row)["bk"]
        copy = (2.0 * M * K + 2.0 * sweep._cdiv(K, bk) * M * bk) / S["copy_bytes_per_s"]
        want = math.ceil(copy / (t * (1.0 - ratio[row])))
        assert got == want and got > 1, (M, N, K, got, want)
    # the two workloads' rows measured the blocked A slower: never prepack
    assert L.mg_prepack_uses_to_pay(1024, 1024, 2048, 0) == -1
    assert L.mg_prepack_uses_to_pay(8192, 8192, 8192, 1) == -1


def test_counters_cover_every_table_choice(data):
    """The sweep JSON carries the hardware counters of the row the table
    picks for each swept shape (`sweep counters`): one entry per shape, its
    row the measured best, the direct-to-LDS or K-split kernel, and the
    derived ratios within their ranges."""
    S = sweep.summarize(data)
    best = {(b["M"], b["N"], b["K"], 0, 1): b["best_row"] for b in S["dense_best"]}
    best.update({(b["T"], b["N"], b["K"], b["E"], 1): b["best_row"] for b in S["grouped_best"]})
    best.update({(b["M"], b["N"], b["K"], 0, b["batch"]): b["best_row"] for b in S["batched_best"]})
    shapes = data["counters"]["shapes"]
    key = lambda c: (c["M"], c["N"], c["K"], c["E"], c.get("B", 1))  # noqa: E731
    assert sorted(key(c) for c in shapes) == sorted(best)
    for c in shapes:
        assert c["row"] == best[key(c)], c
        assert ("gemm_dlds_kernel" in c["kernel"]) == (c["row"] != 7), c
        assert 0.0 < c["mfma_busy_fraction"] <= 1.0
        assert 0.0 <= c["lds_bank_conflict_ratio"] < 1.0
        assert 0.0 <= c["l2_hit_rate"] <= 1.0
    assert len(data["counters"]["commands"]) == len(sweep.COUNTER_PASSES)


def _pass_rows(kernels_and_counters, other_kernel="elementwise_kernel"):
    """Counter-collection rows as rocprofv3 writes them: each GEMM dispatch
    preceded by an unrelated kernel, each counter split over two instances."""
    rows, did = [], 100
    for name, cv in kernels_and_counters:
        did += 1
        rows.append({"Dispatch_Id": str(did), "Kernel_Name": other_kernel, "Counter_Name": next(iter(cv)),
                     "Counter_Value": "7"})
        did += 1
        for counter, v in cv.items():
            for half in (0.25 * v, 0.75 * v):
                rows.append({"Dispatch_Id": str(did), "Kernel_Name": name, "Counter_Name": counter,
                             "Counter_Value": repr(half)})
    return rows


def test_counter_merge_keeps_the_last_call_and_sums_instances():
    order = [{"M": 64, "N": 64, "K": 64, "E": 0, "row": 2}, {"M": 128, "N": 128, "K": 64, "E": 0, "row": 1}]
    assert sweep.COUNTER_CALLS == 2
    ka, kb = "void mg::gemm_dlds_kernel<A>(mg::KArgs)", "void mg::gemm_dlds_kernel<B>(mg::KArgs)"
    p0 = _pass_rows([(ka, {"SQ_VALU_MFMA_BUSY_CYCLES": 1.0, "SQ_BUSY_CYCLES": 1.0}),
                     (ka, {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 6.0, "SQ_BUSY_CYCLES": 32 * 10.0}),
                     (kb, {"SQ_VALU_MFMA_BUSY_CYCLES": 1.0, "SQ_BUSY_CYCLES": 1.0}),
                     (kb, {"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 3.0, "SQ_BUSY_CYCLES": 32 * 10.0})])
    p1 = _pass_rows([(ka, {"SQ_LDS_BANK_CONFLICT": 1.0, "SQ_LDS_IDX_ACTIVE": 1.0}),
                     (ka, {"SQ_LDS_BANK_CONFLICT": 1.0, "SQ_LDS_IDX_ACTIVE": 8.0}),
                     (kb, {"SQ_LDS_BANK_CONFLICT": 1.0, "SQ_LDS_IDX_ACTIVE": 1.0}),
                     (kb, {"SQ_LDS_BANK_CONFLICT": 0.0, "SQ_LDS_IDX_ACTIVE": 8.0})])
    p2 = _pass_rows([(ka, {"TCC_HIT_sum": 1.0, "TCC_MISS_sum": 1.0}), (ka, {"TCC_HIT_sum": 3.0, "TCC_MISS_sum": 1.0}),
                     (kb, {"TCC_HIT_sum": 1.0, "TCC_MISS_sum": 1.0}), (kb, {"TCC_HIT_sum": 1.0, "TCC_MISS_sum": 4.0})])
    a, b = sweep.merge_counter_rows(order, [p0, p1, p2])
    assert (a["kernel"], b["kernel"]) == (ka, kb)
    assert a["values"]["SQ_VALU_MFMA_BUSY_CYCLES"] == 6144.0  # both instances, last call
    assert (a["mfma_busy_fraction"], a["lds_bank_conflict_ratio"], a["l2_hit_rate"]) == (0.6, 0.125, 0.75)
    assert (b["mfma_busy_fraction"], b["lds_bank_conflict_ratio"], b["l2_hit_rate"]) == (0.3, 0.0, 0.2)


def test_counter_merge_refuses_mismatched_passes():
    order = [{"M": 64, "N": 64, "K": 64, "E": 0, "row": 2}]
    ka, kb = "void mg::gemm_dlds_kernel<A>(mg::KArgs)", "void mg::gemm_dlds_kernel<B>(mg::KArgs)"
    one = _pass_rows([(ka, {"TCC_HIT_sum": 1.0})])
    two = _pass_rows([(ka, {"TCC_HIT_sum": 1.0}), (ka, {"TCC_HIT_sum": 1.0})])
    other = _pass_rows([(kb, {"TCC_HIT_sum": 1.0}), (kb, {"TCC_HIT_sum": 1.0})])
    with pytest.raises(RuntimeError):
        sweep.merge_counter_rows(order, [one])  # one dispatch where two calls were made
    with pytest.raises(RuntimeError):
        sweep.merge_counter_rows(order, [two, other])  # the passes ran different kernels
