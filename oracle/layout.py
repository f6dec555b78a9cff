"""Index bookkeeping of the tiled GEMM, written from the pages -- TEST INFRASTRUCTURE ONLY.

Plain integer code for the parts of the method that move data around without
arithmetic on values:

* the blocked re-layout of A, ``[M, K] -> [K/BK, M, BK]`` ("layout planner",
  "Using Triton to optimise GEMM across chips", section 3.2);
* the grouped program-id order used for L2 reuse (the matmul example of the
  Gluon/Triton portability page; explained in "Triton study notes", section
  2.3.7, with its 9x9 worked example);
* the shared-memory budget of a tile configuration (FlagOS cross-chip page,
  section 2.1);
* im2col, which turns a convolution into a GEMM (FlagOS cross-chip page,
  section 5.3).

None of this is imported by the library.
"""
from __future__ import annotations

import numpy as np


def prepacked_shape(M: int, K: int, BK: int) -> tuple[int, int, int]:
    """Shape of the blocked A: ceil(K/BK) panels of M rows by BK columns."""
    return ((K + BK - 1) // BK, M, BK)


def prepack_a(A: np.ndarray, BK: int) -> np.ndarray:
    """Blocked layout of A: Ap[kb, m, kk] = A[m, kb*BK + kk], zero past K.

    The page says only "similar to [K/BLOCK_K, M, BLOCK_K]"; this exact order
    is taken, and the last K block is padded with zeros (bit pattern 0, which
    is +0.0 in fp16 and bf16)."""
    M, K = A.shape
    nkb, _, _ = prepacked_shape(M, K, BK)
    Ap = np.zeros((nkb, M, BK), dtype=A.dtype)
    for kb in range(nkb):
        k0 = kb * BK
        k1 = min(K, k0 + BK)
        Ap[kb, :, : k1 - k0] = A[:, k0:k1]
    return Ap


def unpack_a(Ap: np.ndarray, K: int) -> np.ndarray:
    """Inverse of prepack_a (drops the zero padding)."""
    nkb, M, BK = Ap.shape
    A = np.empty((M, K), dtype=Ap.dtype)
    for kb in range(nkb):
        k0 = kb * BK
        k1 = min(K, k0 + BK)
        A[:, k0:k1] = Ap[kb, :, : k1 - k0]
    return A


def prepacked_index(m: int, k: int, M: int, BK: int) -> int:
    """Flat element index of A[m, k] inside the blocked layout."""
    return ((k // BK) * M + m) * BK + (k % BK)


def grouped_pid(pid: int, num_pid_m: int, num_pid_n: int, group_m: int) -> tuple[int, int]:
    """Program id -> (tile row, tile column) in grouped order.

    Tiles are visited GROUP_M rows at a time, column by column inside the
    group; the last group may hold fewer rows.  This is the mapping of the
    Gluon/Triton page's matmul example (the yfxerp page's version of the same
    idea lost operators in extraction and is not a bijection as printed)."""
    per_group = group_m * num_pid_n
    group_id = pid // per_group
    first_m = group_id * group_m
    rows_here = min(num_pid_m - first_m, group_m)
    local = pid % per_group
    return first_m + local % rows_here, local // rows_here


def row_major_pid(pid: int, num_pid_m: int, num_pid_n: int) -> tuple[int, int]:
    return pid // num_pid_n, pid % num_pid_n


def blocks_loaded(tiles, k_blocks: int) -> int:
    """Input blocks a set of output tiles must read when each distinct A row
    panel and B column panel is read once: (rows + columns) * K-blocks.  This
    is the counting behind the 9x9 example of "Triton study notes" 2.3.7."""
    rows = {t[0] for t in tiles}
    cols = {t[1] for t in tiles}
    return (len(rows) + len(cols)) * k_blocks


def lds_bytes(BM: int, BN: int, BK: int, elem_bytes: int, stages: int) -> int:
    """Shared-memory footprint of one tile configuration: one A tile and one
    B tile per pipeline stage (FlagOS cross-chip page, section 2.1)."""
    return (BM * BK + BK * BN) * elem_bytes * stages


def im2col(x, KH, KW, stride=(1, 1), pad=(0, 0), dil=(1, 1)):
    """im2col of an NHWC image batch (FlagOS cross-chip page, section 5.3:
    convolution becomes a GEMM).  Row m = (n OH + oh) OW + ow of the result
    holds, at column k = (kh KW + kw) C + c, the input value x[n, ih, iw, c]
    with ih = oh sh - ph + kh dh and iw = ow sw - pw + kw dw, or 0 where
    (ih, iw) lies outside the image.  Pure data movement, any element type;
    the zero is the all-zero bit pattern (+0.0)."""
    Nb, H, W, C = x.shape
    sh, sw = stride
    ph, pw = pad
    dh, dw = dil
    OH = (H + 2 * ph - dh * (KH - 1) - 1) // sh + 1
    OW = (W + 2 * pw - dw * (KW - 1) - 1) // sw + 1
    xp = np.zeros((Nb, H + 2 * ph, W + 2 * pw, C), dtype=x.dtype)
    xp[:, ph:ph + H, pw:pw + W, :] = x
    out = np.zeros((Nb, OH, OW, KH, KW, C), dtype=x.dtype)
    for kh in range(KH):
        for kw in range(KW):
            # padded row index of (oh, kh) is oh sh + kh dh
            out[:, :, :, kh, kw, :] = xp[:, kh * dh: kh * dh + sh * (OH - 1) + 1: sh,
                                         kw * dw: kw * dw + sw * (OW - 1) + 1: sw, :]
    return out.reshape(Nb * OH * OW, KH * KW * C)
