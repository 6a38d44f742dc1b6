"""Small-M (prefill chunk) Q4_K product on the GPU against the oracle; row m of
the batched product is the batch-1 product of activation row m."""
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


def small_m(qg, wd, N, K, act, M, variant):
    q, d, s = act
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    qg.qgemm_q4_k_small_m(wd, N, K, M, q, d, s, y, variant)
    return host(y)


def variants(qg):
    return [qg.QGEMV_VARIANT_DOT4, qg.QGEMV_VARIANT_MFMA, qg.QGEMV_VARIANT_AUTO]


@pytest.mark.parametrize("M,N,K", [(1, 100, 256), (2, 65, 896), (3, 257, 4096), (5, 64, 4864),
                                   (8, 300, 4096), (9, 129, 1024), (16, 64, 4096),
                                   (17, 33, 768), (33, 70, 512), (48, 130, 2048),
                                   (64, 96, 4096), (64, 1000, 1024), (7, 20, 32768)])
def test_small_m_shapes(qg, M, N, K):
    g = np.random.default_rng(M * 100 + N)
    w = synth.q4_k_weights(g, N, K)
    x, _ = synth.activation(g, M, K)
    act = quantize(qg, x)
    q, d, s = act_host(*act)
    wd = dev(w)
    Y_ref, TT = oracle.gemm("q4_k", w, N, K, q, d, s)
    for v in variants(qg):
        say("small_m", M, N, K, "variant", v)
        Y = small_m(qg, wd, N, K, act, M, v)
        check_y(Y.reshape(-1), Y_ref.reshape(-1), TT.reshape(-1), f"small_m M={M} N={N} K={K} v={v}")


def test_config4_m8_m64(qg):
    c = synth.config4()
    N, K = c["N"], c["K"]
    wd = dev(c["w"])
    rows = np.concatenate([np.arange(256), np.arange(N - 256, N), np.arange(7000, 7256)])
    for M, x in [(8, c["x8"]), (64, c["x64"])]:
        act = quantize(qg, x)
        q, d, s = act_host(*act)
        Y_ref = np.empty((M, rows.size))
        TT = np.empty((M, rows.size))
        for r0 in (0, 7000, N - 256):
            yy, tt = oracle.gemm("q4_k", c["w"], N, K, q, d, s, rows=(r0, 256))
            sl = {0: slice(0, 256), N - 256: slice(256, 512), 7000: slice(512, 768)}[r0]
            Y_ref[:, sl] = yy
            TT[:, sl] = tt
        for v in variants(qg):
            say("config4", M, "variant", v)
            Y = small_m(qg, wd, N, K, act, M, v)
            assert np.all(np.isfinite(Y))
            check_y(Y[:, rows].reshape(-1), Y_ref.reshape(-1), TT.reshape(-1), f"config4 M={M}")


def test_row_independence(qg):
    """Row m of an M-row call equals a 1-row call on activation row m, bit for bit."""
    g = np.random.default_rng(5)
    N, K, M = 200, 4096, 8
    w = synth.q4_k_weights(g, N, K)
    x, _ = synth.activation(g, M, K)
    wd = dev(w)
    q, d, s = quantize(qg, x)
    for v in (qg.QGEMV_VARIANT_DOT4, qg.QGEMV_VARIANT_MFMA):
        Y = small_m(qg, wd, N, K, (q, d, s), M, v)
        for m in (0, 3, 7):
            Ym = small_m(qg, wd, N, K, (q[m:m + 1], d[m:m + 1], s[m:m + 1]), 1, v)
            assert np.array_equal(Y[m].view(np.uint32), Ym[0].view(np.uint32)), (v, m)


def test_variants_agree_and_mfma_matches_dots(qg):
    """MFMA and DOT4 give the same rows within the tolerance of the definition,
    and the MFMA result of one row matches the batch-1 GEMV within it too."""
    g = np.random.default_rng(9)
    N, K, M = 333, 2304, 24
    w = synth.q4_k_weights(g, N, K)
    x, _ = synth.activation(g, M, K)
    act = quantize(qg, x)
    q, d, s = act_host(*act)
    wd = dev(w)
    Y_ref, TT = oracle.gemm("q4_k", w, N, K, q, d, s)
    for v in (qg.QGEMV_VARIANT_DOT4, qg.QGEMV_VARIANT_MFMA):
        Y = small_m(qg, wd, N, K, act, M, v)
        check_y(Y.reshape(-1), Y_ref.reshape(-1), TT.reshape(-1), f"variant {v}")
