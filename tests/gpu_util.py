"""Helpers shared by the GPU tests: moving fp16/bf16 bit patterns between
numpy and torch, guard bands around outputs, and the comparison gates."""
from __future__ import annotations

import sys

import numpy as np

from oracle import compare

F16, BF16 = 0, 1
CANARY = 0x7FFF  # NaN in both fp16 (exponent 0x1F, fraction 0x3FF) and bf16 (exponent 0xFF, fraction 0x7F): never a result here


def announce(msg: str) -> None:
    sys.stdout.write("[gpu-case] %s\n" % msg)
    sys.stdout.flush()


def torch_dtype(dtype: int):
    import torch

    return torch.float16 if dtype == F16 else torch.bfloat16


def to_dev(bits: np.ndarray, dtype: int):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch_dtype(dtype)).cuda()


def to_host(t) -> np.ndarray:
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class Guarded:
    """An output matrix with canary-filled guard bands before and after it
    (and in the padding of each row when ld > cols)."""

    def __init__(self, rows: int, cols: int, dtype: int, ld: int | None = None, guard: int = 2048):
        import torch

        self.rows, self.cols, self.ld, self.guard = rows, cols, ld or cols, guard
        total = guard + rows * self.ld + guard
        self.buf = torch.full((total,), CANARY, dtype=torch.int16, device="cuda")
        self.flat = self.buf.view(torch_dtype(dtype))
        self.mat = self.flat[guard: guard + rows * self.ld].view(rows, self.ld)[:, :cols]

    def result(self) -> np.ndarray:
        return to_host(self.mat)

    def guards_intact(self) -> bool:
        h = to_host(self.buf)
        body = h[self.guard: self.guard + self.rows * self.ld].reshape(self.rows, self.ld) if self.rows else None
        ok = np.all(h[: self.guard] == CANARY) and np.all(h[self.guard + self.rows * self.ld:] == CANARY)
        if body is not None and self.ld > self.cols:
            ok = ok and np.all(body[:, self.cols:] == CANARY)
        return bool(ok)


def assert_bitexact(got, ref_q, dtype, label=""):
    bad = compare.bitexact_mismatches(got, ref_q)
    assert bad.size == 0, "%s bit-exact: %s" % (label, compare.describe(bad, got, compare.to_f64(ref_q, dtype), dtype,
                                                                       np.shape(got)))


def assert_tolerance(got, ref, dtype, label=""):
    bad = compare.tolerance_mismatches(got, ref, dtype)
    assert bad.size == 0, "%s tolerance: %s" % (label, compare.describe(bad, got, ref, dtype, np.shape(got)))
