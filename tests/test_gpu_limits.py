"""Sizes at the library's limits, against the oracle.

* An output of more than 2^31 elements (65537 x 32776 fp16, K = 64): 64-bit
  output addressing in the direct-to-LDS kernel's epilogue.  Integer inputs
  make every output exact, so besides the seeded 4096-element sample and the
  edge set (checked against the oracle) every row sum and every column sum
  of the output is compared with the exact sums A (B 1) and (1^T A) B,
  computed here from the inputs in int64: a wrong, missing or doubled
  element anywhere changes its row's and its column's sum.
* Leading strides whose tile spans do not fit the direct-to-LDS kernel's
  31-bit per-tile load offsets: the problem falls back to the general
  kernel (row-major operands), or is refused with
  MG_ERR_UNSUPPORTED_LAYOUT (a transposed operand, which only the
  direct-to-LDS kernel reads); an output stride that puts rows more than
  2^31 elements from the base stays on the direct-to-LDS kernel (its stores
  are 64-bit addressed).
* Grouped weights of more than 2^31 elements (160 experts of 4096 x 4096):
  the experts whose weights start past that point, against the oracle.
* Grouped expert offsets that break the rules: nothing outside Y is
  written, and the result is the product over the partition the kernel
  clamps them to.
* The largest token count the grouped entry point takes (T = 2^31 - 1),
  with one expert holding all but 100 of them, and a dense output of
  2^31 - 1 rows on a fast and a general row: the device-side count of an
  expert's row tiles must not overflow 32 bits, and launches of more
  workgroups than one grid dimension holds must run every tile (checked
  on every output row).
"""
import numpy as np
import pytest

import tiled_matrix_multiplication_gemm_amd as mg
from oracle import compare
from tiled_matrix_multiplication_gemm_amd import inputs
from tests.gpu_util import (CANARY, F16, announce, assert_bitexact, to_dev, to_host, torch_dtype)

pytestmark = pytest.mark.gpu

# Leading stride (elements) beyond the direct-to-LDS kernel's reach for
# every row: a 64-row (or 64-k-row) tile span of it is more than 2^31 bytes.
HUGE_LD = (1 << 24) + 8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mg.lib()
    yield
    mg.mg_set_config(-1)
    torch.cuda.empty_cache()


def exact(bits):
    """fp16 bit patterns of integers -> int64 values."""
    return np.asarray(bits).view(np.float16).astype(np.int64)


def test_output_beyond_2_31_elements(orc):
    import torch

    M, N, K = 65537, 32776, 64
    assert M * N > 2 ** 31
    c = inputs.integer_dense(M, N, K, F16, 9101, name="beyond_2_31")
    announce("dense %dx%dx%d fp16 integer (output > 2^31 elements)" % (M, N, K))
    A, B = to_dev(c.A, F16), to_dev(c.B, F16)
    guard = 4096
    buf = torch.full((guard + M * N + guard,), CANARY, dtype=torch.int16, device="cuda")
    C = buf[guard: guard + M * N].view(torch_dtype(F16)).view(M, N)
    mg.mg_gemm(A, B, out=C)
    torch.cuda.synchronize()
    assert mg.mg_last_kernel() == "gemm_dlds_kernel"
    assert bool((buf[:guard] == CANARY).all()) and bool((buf[guard + M * N:] == CANARY).all()), \
        "write outside the output"
    del A, B
    rows, cols = compare.sample_positions(M, N, 4096, 9102)
    er, ec = compare.edge_positions(M, N)
    rows, cols = np.concatenate([rows, er]), np.concatenate([cols, ec])
    got_s = to_host(C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()])
    _, ref_q = orc.gemm_sampled(c.A, c.B, F16, rows, cols)
    assert_bitexact(got_s, ref_q, F16, "sample + edges")
    # every row and column sum (|C| <= 16 K = 1024: every output is an exact fp16 integer)
    Ai, Bi = exact(c.A), exact(c.B)
    want_rows = Ai @ Bi.sum(axis=1)
    want_cols = Ai.sum(axis=0) @ Bi
    got_cols = np.zeros(N, dtype=np.int64)
    step = 4096
    for r0 in range(0, M, step):
        blk = to_host(C[r0: r0 + step]).view(np.float16).astype(np.float64)
        assert np.all(np.isfinite(blk)), "non-finite output in rows %d.." % r0
        assert np.array_equal(blk.sum(axis=1).astype(np.int64), want_rows[r0: r0 + step]), "row sums, rows %d.." % r0
        got_cols += blk.sum(axis=0).astype(np.int64)
    assert np.array_equal(got_cols, want_cols), "column sums"


def strided_dev(bits, ld, dt):
    """bits [R, C] on the device as a view with row stride ld."""
    import torch

    R, Cc = bits.shape
    store = torch.empty((R - 1) * ld + Cc, dtype=torch_dtype(dt), device="cuda")
    v = store.as_strided((R, Cc), (ld, 1))
    v.copy_(to_dev(bits, dt))
    return v


@pytest.mark.parametrize("which", ["a", "b"])
def test_operand_stride_beyond_the_direct_kernel_falls_back(orc, which):
    import torch

    M, N, K = 100, 136, 72
    c = inputs.integer_dense(M, N, K, F16, 9200 + (which == "b"), epilogue=True, name="huge_ld")
    announce("dense %dx%dx%d, ld%s = %d (general kernel)" % (M, N, K, which, HUGE_LD))
    A = strided_dev(c.A, HUGE_LD, F16) if which == "a" else to_dev(c.A, F16)
    B = strided_dev(c.B, HUGE_LD, F16) if which == "b" else to_dev(c.B, F16)
    out = mg.mg_gemm_bias_relu(A, B, to_dev(c.bias, F16))
    torch.cuda.synchronize()
    assert mg.mg_last_kernel() == "gemm_tile_kernel"
    _, ref_q = orc.gemm(c.A, c.B, F16, bias=c.bias, relu=True)
    assert_bitexact(to_host(out), ref_q, F16, "ld%s = %d" % (which, HUGE_LD))
    del A, B, out
    torch.cuda.empty_cache()


def test_output_stride_beyond_2_31_elements_stays_direct(orc):
    import torch

    M, N, K = 200, 136, 128
    c = inputs.integer_dense(M, N, K, F16, 9300, name="huge_ldc")
    announce("dense %dx%dx%d, ldc = %d (rows past 2^31 elements)" % (M, N, K, HUGE_LD))
    assert (M - 1) * HUGE_LD > 2 ** 31
    store = torch.full(((M - 1) * HUGE_LD + N,), CANARY, dtype=torch.int16, device="cuda")
    C = store.view(torch_dtype(F16)).as_strided((M, N), (HUGE_LD, 1))
    mg.mg_gemm(to_dev(c.A, F16), to_dev(c.B, F16), out=C)
    torch.cuda.synchronize()
    assert mg.mg_last_kernel() == "gemm_dlds_kernel"
    _, ref_q = orc.gemm(c.A, c.B, F16)
    assert_bitexact(to_host(C), ref_q, F16, "ldc = %d" % HUGE_LD)
    # the gap after each row is untouched (sampled: the first 64 elements of every gap)
    gaps = store.as_strided((M - 1, 64), (HUGE_LD, 1), N)
    assert bool((gaps == CANARY).all()), "write between rows"
    del C, store
    torch.cuda.empty_cache()


def test_transposed_operand_beyond_the_direct_kernel_is_refused():
    import torch

    M, N, K = 64, 64, 64
    announce("dense %dx%dx%d, A transposed with ld = %d (refused)" % (M, N, K, HUGE_LD))
    At = torch.zeros((K - 1) * HUGE_LD + M, dtype=torch.float16, device="cuda").as_strided((K, M), (HUGE_LD, 1))
    B = torch.zeros((K, N), dtype=torch.float16, device="cuda")
    with pytest.raises(RuntimeError, match="UNSUPPORTED_LAYOUT"):
        mg.mg_gemm(At.t(), B)
    del At
    torch.cuda.empty_cache()


def test_grouped_weights_beyond_2_31_elements(orc):
    """160 experts of 4096 x 4096 weights (2.7e9 elements): the weights of the
    last experts start beyond 2^31 elements from the base.  Tokens go to
    experts 0, 1, 130 and 159 only (130 and 159 lie past the limit); every
    output row is checked bit-exact against the dense oracle of its expert
    (the grouped oracle is the per-expert dense one)."""
    import torch

    E, K, N = 160, 4096, 4096
    live = {0: 40, 1: 1, 130: 257, 159: 33}
    assert 130 * K * N > 2 ** 31
    counts = np.zeros(E, dtype=np.int64)
    for e, n in live.items():
        counts[e] = n
    off = inputs.offsets_from_counts(counts)
    T = int(off[-1])
    rng = np.random.default_rng(9400)
    X = inputs.to_bits(rng.integers(-4, 5, size=(T, K)).astype(np.float64), F16)
    Wl = {e: inputs.to_bits(rng.integers(-4, 5, size=(K, N)).astype(np.float64), F16) for e in live}
    announce("grouped E=%d K=%d N=%d T=%d, weights beyond 2^31 elements" % (E, K, N, T))
    W = torch.zeros((E, K, N), dtype=torch_dtype(F16), device="cuda")
    for e, w in Wl.items():
        W[e].copy_(to_dev(w, F16))
    Y = mg.mg_grouped_gemm(to_dev(X, F16), W, torch.from_numpy(off.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    got = to_host(Y)
    del W, Y
    torch.cuda.empty_cache()
    for e in live:
        r0, r1 = int(off[e]), int(off[e + 1])
        _, ref_q = orc.gemm(X[r0:r1], Wl[e], F16)
        assert_bitexact(got[r0:r1], ref_q, F16, "expert %d" % e)


@pytest.mark.parametrize("E", [12, 70])
def test_grouped_offsets_out_of_order_stay_inside_the_buffers(orc, E):
    """Expert offsets that break the rules (negative, decreasing, past T):
    the kernel clamps each offset into [0, T] and raises it to at least the
    previous one, so it computes the grouped product for that clamped
    partition (checked against the oracle), leaves every row outside it
    untouched, and writes nothing outside Y.  Both ways of reading the
    offsets are covered (held in lanes below 64 experts, read from memory
    above)."""
    import torch

    T, N, K = 700, 136, 128
    rng = np.random.default_rng(9500 + E)
    raw = rng.integers(-100, T + 200, size=E + 1).astype(np.int64)
    raw[0] = 30  # rows 0..29 belong to no expert
    clamped = np.empty_like(raw)
    a = min(max(int(raw[0]), 0), T)
    clamped[0] = a
    for e in range(E):
        b = min(max(int(raw[e + 1]), a), T)
        clamped[e + 1] = b
        a = b
    assert clamped[-1] < T or clamped[0] > 0  # some rows lie outside the partition
    X = inputs.to_bits(rng.integers(-4, 5, size=(T, K)).astype(np.float64), F16)
    W = inputs.to_bits(rng.integers(-4, 5, size=(E, K, N)).astype(np.float64), F16)
    announce("grouped E=%d T=%d with offsets out of order" % (E, T))
    from tests.gpu_util import Guarded

    out = Guarded(T, N, F16)
    mg.mg_grouped_gemm(to_dev(X, F16), to_dev(W, F16), torch.from_numpy(raw.astype(np.int32)).cuda(), out=out.mat)
    torch.cuda.synchronize()
    assert out.guards_intact(), "write outside Y"
    got = out.result()
    lo, hi = int(clamped[0]), int(clamped[-1])
    assert np.all(got[:lo] == CANARY) and np.all(got[hi:] == CANARY), "rows outside the partition written"
    _, ref_q = orc.grouped_gemm(X[lo:hi], W, clamped - lo, F16)
    assert_bitexact(got[lo:hi], ref_q, F16, "clamped partition")


P_BLOCK = 65521  # rows of the repeated input block: a prime, so a row offset error lands on another block row


def periodic_rows(P, K, seed):
    """A seeded P x K block of small integers, and a device matrix of T rows
    whose row r is block row r % P (filled by copies on the device)."""
    rng = np.random.default_rng(seed)
    return rng, inputs.to_bits(rng.integers(-4, 5, size=(P, K)).astype(np.float64), F16)


def fill_periodic(X, blk):
    import torch

    T, K = X.shape
    P = blk.shape[0]
    q = T // P
    d = to_dev(blk, F16)
    X[: q * P].view(q, P, K).copy_(d.unsqueeze(0).expand(q, P, K))
    X[q * P:].copy_(d[: T - q * P])


def assert_periodic_output(Y, r0, r1, E, label, chunk=1 << 26):
    """Every row r in [r0, r1) of the device matrix Y must equal row r % P
    of E (the oracle's product of the repeated block; fp16 bit patterns).
    The comparison runs on the device, chunk by chunk, against E repeated."""
    import torch

    P, N = E.shape
    Ed = torch.from_numpy(np.ascontiguousarray(E).view(np.int16)).cuda()
    big = Ed.repeat((chunk + P - 1) // P + 1, 1)
    Yi = Y.view(torch.int16)
    for a in range(r0, r1, chunk):
        b = min(a + chunk, r1)
        ph = a % P
        got = Yi[a:b]
        want = big[ph: ph + (b - a)]
        if not torch.equal(got, want):
            bad = (got != want).any(dim=1).nonzero()
            first = a + int(bad[0])
            raise AssertionError("%s: %d rows differ in rows %d..%d, first %d (got %s, want %s)" % (
                label, int(bad.numel()), a, b, first, to_host(Yi[first]).tolist(),
                E[first % P].tolist()))


@pytest.mark.parametrize("row", [2, 5])
def test_dense_output_rows_past_2_31(orc, row):
    """M = 2^31 - 1 rows, N = K = 8, forced onto the 64 x 64 direct-to-LDS
    row (33.5 million workgroups) and the general kernel's 128 x 128 row
    (16.8 million): both launches pass the 2^32 work-items one grid
    dimension holds, so they run as several rows of workgroups.  A repeats
    a seeded block of P rows, so C repeats the oracle's product of that
    block; every row of C is compared with it (C starts as the canary, so a
    tile that never runs shows up)."""
    import torch

    M, N, K, P = 2 ** 31 - 1, 8, 8, P_BLOCK
    rng, blk = periodic_rows(P, K, 9700 + row)
    B = inputs.to_bits(rng.integers(-4, 5, size=(K, N)).astype(np.float64), F16)
    announce("dense M = 2^31 - 1, N = K = 8 on row %d" % row)
    A = torch.empty((M, K), dtype=torch.float16, device="cuda")
    fill_periodic(A, blk)
    C = torch.full((M, N), CANARY, dtype=torch.int16, device="cuda").view(torch.float16)
    mg.mg_set_config(row)
    try:
        mg.mg_gemm(A, to_dev(B, F16), out=C)
        torch.cuda.synchronize()
    finally:
        mg.mg_set_config(-1)
    assert mg.mg_last_config() == row
    del A
    _, E = orc.gemm(blk, B, F16)
    assert_periodic_output(C, 0, M, E, "row %d" % row)
    del C
    torch.cuda.empty_cache()


def test_grouped_largest_token_count(orc):
    """T = 2^31 - 1 tokens (K = N = 8): expert 0 takes rows 0..99, expert 1
    the other 2^31 - 101 (8.4 million workgroups: a launch past 2^32
    work-items).  X repeats a seeded block of P rows, copied on the device;
    the oracle multiplies the same block on the host, so none of its inputs
    comes back from the device, and every row of Y is compared with the
    oracle's product for its expert (Y starts as the canary)."""
    import torch

    T, K, N, P = 2 ** 31 - 1, 8, 8, P_BLOCK
    rng, blk = periodic_rows(P, K, 9600)
    W = inputs.to_bits(rng.integers(-4, 5, size=(2, K, N)).astype(np.float64), F16)
    off = np.array([0, 100, T], dtype=np.int64)
    announce("grouped T = 2^31 - 1, K = N = 8, experts of 100 and 2^31 - 101 rows")
    X = torch.empty((T, K), dtype=torch.float16, device="cuda")
    fill_periodic(X, blk)
    Y = torch.full((T, N), CANARY, dtype=torch.int16, device="cuda").view(torch.float16)
    mg.mg_grouped_gemm(X, to_dev(W, F16), torch.from_numpy(off.astype(np.int32)).cuda(), out=Y)
    torch.cuda.synchronize()
    del X
    for e in range(2):
        _, E = orc.gemm(blk, W[e], F16)
        assert_periodic_output(Y, int(off[e]), int(off[e + 1]), E, "expert %d" % e)
    del Y
    torch.cuda.empty_cache()
