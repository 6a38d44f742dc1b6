"""Helpers for the GPU parity tests: host<->device marshalling and the
comparison rules.

Comparison rules (same on every GPU test):
  * integer stages (activation codes, scale bits, code sums, block dots) are
    compared bit for bit;
  * fp32 row outputs must satisfy |y_gpu - y_ref| <= 1e-5 * T + 1e-7 with
    y_ref and T = sum of |every separately scaled fp term| from the oracle.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

DEV = "cuda:0"


def say(*a):
    """Name the case on the real stderr before a GPU step (survives a crash)."""
    print("[gpu-case]", *a, file=sys.__stderr__, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    torch.cuda.synchronize()
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def quantize(qg, x: np.ndarray, K: int | None = None):
    """Run qgemv_quantize_act on host fp32 x [M][ldx]; returns device (q, d, s)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None]
    M, ldx = x.shape
    K = ldx if K is None else K
    xd = dev(x)
    q, d, s = qg.act_buffers(M, K, DEV)
    qg.qgemv_quantize_act(xd, M, K, ldx, q, d, s)
    return q, d, s


def act_host(q, d, s):
    return host(q), host(d, np.uint16), host(s)


def gemv(qg, fmt: str, w_dev, N: int, K: int, act) -> np.ndarray:
    q, d, s = act
    y = torch.full((N,), float("nan"), dtype=torch.float32, device=DEV)
    qg.GEMV[fmt](w_dev, N, K, q, d, s, y)
    return host(y)


def block_dots(qg, fmt: str, w_dev, N: int, K: int, q_dev, row0: int, nrows: int) -> np.ndarray:
    nblk = oracle.nblk(fmt, K)
    out = torch.full((nrows, nblk), -(2**31), dtype=torch.int32, device=DEV)
    qg.qgemv_block_dots(qg.FMT_ID[fmt], w_dev, N, K, row0, nrows, q_dev, out)
    return host(out)


def check_y(y: np.ndarray, y_ref: np.ndarray, T: np.ndarray, what: str = ""):
    y = np.asarray(y, np.float64)
    tol = oracle.tolerance(T)
    err = np.abs(y - y_ref)
    bad = ~(err <= tol)
    if bad.any():
        i = int(np.argmax(np.where(bad, err / tol, 0)))
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{y.size} outputs outside tolerance; worst at {i}: "
            f"gpu {y[i]!r} ref {y_ref[i]!r} |err| {err[i]:.3e} tol {tol[i]:.3e}")
    return float(np.max(err / tol)) if y.size else 0.0


def sample_rows(N: int, n: int, seed: int = 0) -> np.ndarray:
    """First, last and a seeded random spread of rows (sorted, unique)."""
    g = np.random.default_rng(seed)
    rows = set(range(min(N, 64))) | set(range(max(0, N - 64), N))
    rows |= set(g.choice(N, size=min(N, n), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def oracle_rows(fmt, w_host, N, K, q, d, s, rows: np.ndarray):
    """Oracle y and T for an arbitrary set of rows (contiguous runs batched)."""
    y = np.empty(rows.size)
    T = np.empty(rows.size)
    i = 0
    while i < rows.size:
        j = i
        while j + 1 < rows.size and rows[j + 1] == rows[j] + 1:
            j += 1
        yy, TT = oracle.gemv(fmt, w_host, N, K, q, d, s, rows=(int(rows[i]), j - i + 1))
        y[i:j + 1] = yy
        T[i:j + 1] = TT
        i = j + 1
    return y, T
