"""Q6_K load-time repack (qgemv_q6_k_repack) and the GEMV on the repacked
layout (qgemv_q6_k_r8) on the GPU.

The repack is a pure permutation of bytes: it is checked bit for bit against
the layout as documented in include/qgemv.h, restated here with numpy (tiles
of 8 super-blocks: ql[8][128] | qh[8][64] | sc[8][16] | d[8], slots past the
row's super-blocks zero).  The GEMV on the repacked weights is checked against
the oracle on the native weights (same tolerance), its block dots bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import act_host, check_y, dev, host, quantize, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qg():
    import block_quantized_gemv_w4a8_amd as qg
    return qg


def repack_reference(w: np.ndarray, N: int, K: int) -> np.ndarray:
    nsb = (K + 255) // 256
    ntile = (nsb + 7) // 8
    sb = w.reshape(N, nsb, 210)
    out = np.zeros((N, ntile, 1680), dtype=np.uint8)
    for S in range(nsb):
        T, i = divmod(S, 8)
        out[:, T, 128 * i:128 * i + 128] = sb[:, S, 0:128]          # ql
        out[:, T, 1024 + 64 * i:1024 + 64 * i + 64] = sb[:, S, 128:192]  # qh
        out[:, T, 1536 + 16 * i:1536 + 16 * i + 16] = sb[:, S, 192:208]  # sc
        out[:, T, 1664 + 2 * i:1664 + 2 * i + 2] = sb[:, S, 208:210]    # d
    return out.reshape(N, ntile * 1680)


def repack(qg, w_dev, N, K):
    rb = qg.q6_k_r8_row_bytes(K)
    wr = torch.full((N, rb), 0x5A, dtype=torch.uint8, device="cuda:0")
    qg.qgemv_q6_k_repack(w_dev, N, K, wr)
    return wr


@pytest.mark.parametrize("N,K", [(3, 256), (5, 4096), (7, 14336), (2, 2304), (4, 896)])
def test_repack_bytes(qg, N, K):
    g = np.random.default_rng(N * 31 + K)
    w = synth.q6_k_weights(g, N, K)
    say("q6_k repack", N, K)
    wr = host(repack(qg, dev(w), N, K))
    assert np.array_equal(wr, repack_reference(w.reshape(N, -1), N, K))


# K = 8448 (132 units) and 16640 (260 units): split-K slices start at tile
# boundaries, so the last of the four slices holds no unit of the row
# (4096 x 1792: one GPU's K slice of the down product split 8 ways)
@pytest.mark.parametrize("N,K", [(1, 256), (37, 896), (130, 2304), (300, 4096), (129, 8192),
                                 (64, 14336), (33, 32768), (1000, 1024), (70, 8448),
                                 (129, 16640), (4096, 1792)])
def test_r8_gemv_against_oracle(qg, N, K):
    g = np.random.default_rng(N + 3 * K)
    w = synth.q6_k_weights(g, N, K)
    x, _ = synth.activation(g, 1, K)
    act = quantize(qg, x)
    q, d, s = act_host(*act)
    wr = repack(qg, dev(w), N, K)
    y = torch.full((N,), float("nan"), device="cuda:0")
    say("q6_k_r8 gemv", N, K)
    qg.qgemv_q6_k_r8(wr, N, K, *act, y)
    y_ref, T = oracle.gemv("q6_k", w, N, K, q, d, s)
    check_y(host(y), y_ref, T, f"q6_k_r8 N={N} K={K}")
    nr = min(N, 64)
    nblk = oracle.nblk("q6_k", K)
    dots = torch.full((nr, nblk), -(2**31), dtype=torch.int32, device="cuda:0")
    qg.qgemv_block_dots(qg.QGEMV_FMT_Q6_K_R8, wr, N, K, 0, nr, act[0], dots)
    assert np.array_equal(host(dots), oracle.block_dots("q6_k", w, N, K, q, rows=(0, nr)))


def test_r8_lm_head_full_size(qg):
    c = synth.config3()
    N, K = c["N"], c["K"]
    act = quantize(qg, c["x"])
    q, d, s = act_host(*act)
    wr = repack(qg, dev(c["w"]), N, K)
    assert wr.shape[1] == 3360          # no padding at K = 4096 (16 super-blocks)
    y = torch.empty(N, device="cuda:0")
    say("q6_k_r8 lm_head full size")
    qg.qgemv_q6_k_r8(wr, N, K, *act, y)
    yh = host(y)
    for r0 in (0, 64000, N - 512):
        y_ref, T = oracle.gemv("q6_k", c["w"], N, K, q, d, s, rows=(r0, 512))
        check_y(yh[r0:r0 + 512], y_ref, T, f"lm_head r8 rows {r0}")
    # the native layout gives the same products within the tolerance, and the
    # same bits where both take the whole row in one slice (K = 4096)
    yn = torch.empty(N, device="cuda:0")
    qg.qgemv_q6_k(dev(c["w"]), N, K, *act, yn)
    assert np.array_equal(host(yn).view(np.uint32), yh.view(np.uint32))
