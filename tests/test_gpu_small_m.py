"""Small-M (prefill chunk) products on the GPU against the oracle, for Q4_K,
Q6_K and Q4_0 weights; row m of the batched product is the batch-1 product
of activation row m."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import act_host, check_y, dev, host, quantize, say

pytestmark = pytest.mark.gpu

WEIGHTS = {"q4_k": synth.q4_k_weights, "q6_k": synth.q6_k_weights, "q4_0": synth.q4_0_weights}


@pytest.fixture(scope="module")
def qg():
    import block_quantized_gemv_w4a8_amd as qg
    return qg


def small_m(qg, fmt, wd, N, K, act, M, variant):
    q, d, s = act
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
    qg.SMALL_M[fmt](wd, N, K, M, q, d, s, y, variant)
    return host(y)


def variants(qg):
    return [qg.QGEMV_VARIANT_DOT4, qg.QGEMV_VARIANT_MFMA, qg.QGEMV_VARIANT_AUTO,
            qg.QGEMV_VARIANT_MFMA_STAGED, qg.QGEMV_VARIANT_MFMA_STREAM,
            qg.QGEMV_VARIANT_MFMA_RESIDENT]


SHAPES = [(1, 100, 256), (2, 65, 896), (3, 257, 4096), (5, 64, 4864), (8, 300, 4096),
          (9, 129, 1024), (16, 64, 4096), (17, 33, 768), (33, 70, 512), (48, 130, 2048),
          (64, 96, 4096), (64, 1000, 1024), (50, 300, 2048), (7, 20, 32768)]
# Q4_0 rows need not hold whole 256-weight units: K = 32, 96, 1056, 4128
Q40_EXTRA = [(3, 40, 32), (17, 50, 96), (8, 90, 1056), (64, 70, 4128)]


@pytest.mark.parametrize("fmt,M,N,K", [("q4_k",) + sh for sh in SHAPES] +
                         [("q6_k",) + sh for sh in SHAPES] +
                         [("q4_0",) + sh for sh in SHAPES + Q40_EXTRA])
def test_small_m_shapes(qg, fmt, M, N, K):
    g = np.random.default_rng(M * 100 + N + 7 * K)
    w = WEIGHTS[fmt](g, N, K)
    x, _ = synth.activation(g, M, K)
    act = quantize(qg, x)
    q, d, s = act_host(*act)
    wd = dev(w)
    Y_ref, TT = oracle.gemm(fmt, w, N, K, q, d, s)
    for v in variants(qg):
        say("small_m", fmt, M, N, K, "variant", v)
        Y = small_m(qg, fmt, wd, N, K, act, M, v)
        check_y(Y.reshape(-1), Y_ref.reshape(-1), TT.reshape(-1),
                f"small_m {fmt} M={M} N={N} K={K} v={v}")


# Wide matrices (at least 512 row tiles of 16: N = 8200 gives 513, the last
# ragged) take the configurations that share each staged activation over 64
# or 32 weight rows, one per bucket of M; every output against the oracle.
WIDE = [("q4_k", 8, 1024), ("q4_k", 12, 2304), ("q4_k", 16, 1024), ("q4_k", 20, 1024),
        ("q4_k", 40, 1024), ("q4_k", 57, 1280), ("q4_k", 64, 1024),
        ("q6_k", 8, 1024), ("q6_k", 24, 1024), ("q6_k", 33, 1024), ("q6_k", 64, 1024),
        ("q4_0", 5, 2336), ("q4_0", 8, 1056), ("q4_0", 17, 1056), ("q4_0", 40, 1056), ("q4_0", 50, 1056),
        ("q4_0", 64, 1056)]


@pytest.mark.parametrize("fmt,M,K", WIDE)
def test_small_m_wide_matrices(qg, fmt, M, K):
    N = 8200
    g = np.random.default_rng(M * 31 + K + len(fmt))
    w = WEIGHTS[fmt](g, N, K)
    x, _ = synth.activation(g, M, K)
    act = quantize(qg, x)
    q, d, s = act_host(*act)
    wd = dev(w)
    Y_ref, TT = oracle.gemm(fmt, w, N, K, q, d, s)
    for v in (qg.QGEMV_VARIANT_MFMA, qg.QGEMV_VARIANT_AUTO, qg.QGEMV_VARIANT_MFMA_STAGED,
              qg.QGEMV_VARIANT_MFMA_STREAM):
        say("small_m wide", fmt, M, N, K, "variant", v)
        Y = small_m(qg, fmt, wd, N, K, act, M, v)
        check_y(Y.reshape(-1), Y_ref.reshape(-1), TT.reshape(-1),
                f"small_m wide {fmt} M={M} N={N} K={K} v={v}")


def sampled(fmt, w, N, K, act, windows):
    q, d, s = act
    M = q.shape[0]
    parts_y, parts_t = [], []
    for r0, nr in windows:
        yy, tt = oracle.gemm(fmt, w, N, K, q, d, s, rows=(r0, nr))
        parts_y.append(yy)
        parts_t.append(tt)
    rows = np.concatenate([np.arange(r0, r0 + nr) for r0, nr in windows])
    return rows, np.concatenate(parts_y, axis=1), np.concatenate(parts_t, axis=1)


def test_config4_m8_m64(qg):
    c = synth.config4()
    N, K = c["N"], c["K"]
    wd = dev(c["w"])
    for M, x in [(8, c["x8"]), (64, c["x64"])]:
        act = quantize(qg, x)
        rows, Y_ref, TT = sampled("q4_k", c["w"], N, K, act_host(*act),
                                  [(0, 256), (7000, 256), (N - 256, 256)])
        for v in variants(qg):
            say("config4", M, "variant", v)
            Y = small_m(qg, "q4_k", wd, N, K, act, M, v)
            assert np.all(np.isfinite(Y))
            check_y(Y[:, rows].reshape(-1), Y_ref.reshape(-1), TT.reshape(-1), f"config4 M={M}")


def test_q6_k_down_shape_m8_m64(qg):
    """The prefill chunk through the Llama-3.1-8B down projection (Q6_K 4096 x 14336)."""
    g = np.random.default_rng(11)
    N, K = 4096, 14336
    w = synth.q6_k_weights(g, N, K)
    wd = dev(w)
    x64, _ = synth.activation(g, 64, K)
    for M in (8, 64):
        act = quantize(qg, x64[:M])
        rows, Y_ref, TT = sampled("q6_k", w, N, K, act_host(*act), [(0, 128), (2000, 64), (N - 128, 128)])
        for v in (qg.QGEMV_VARIANT_MFMA, qg.QGEMV_VARIANT_AUTO):
            say("q6_k down shape", M, "variant", v)
            Y = small_m(qg, "q6_k", wd, N, K, act, M, v)
            assert np.all(np.isfinite(Y))
            check_y(Y[:, rows].reshape(-1), Y_ref.reshape(-1), TT.reshape(-1), f"q6_k down M={M}")


def test_q4_0_config0_shape_m64(qg):
    c = synth.config0()
    g = np.random.default_rng(12)
    x64, _ = synth.activation(g, 64, 896)
    act = quantize(qg, x64)
    q, d, s = act_host(*act)
    Y_ref, TT = oracle.gemm("q4_0", c["w"], 896, 896, q, d, s)
    for v in variants(qg):
        say("q4_0 config0 shape M=64 variant", v)
        Y = small_m(qg, "q4_0", dev(c["w"]), 896, 896, act, 64, v)
        check_y(Y.reshape(-1), Y_ref.reshape(-1), TT.reshape(-1), f"q4_0 896 M=64 v={v}")


@pytest.mark.parametrize("fmt", ["q4_k", "q6_k", "q4_0"])
def test_row_independence(qg, fmt):
    """Row m of an M-row call equals a 1-row call on activation row m, bit for bit."""
    g = np.random.default_rng(5)
    N, K, M = 200, 4096, 8
    w = WEIGHTS[fmt](g, N, K)
    x, _ = synth.activation(g, M, K)
    wd = dev(w)
    q, d, s = quantize(qg, x)
    for v in (qg.QGEMV_VARIANT_DOT4, qg.QGEMV_VARIANT_MFMA, qg.QGEMV_VARIANT_MFMA_STAGED,
              qg.QGEMV_VARIANT_MFMA_STREAM):
        Y = small_m(qg, fmt, wd, N, K, (q, d, s), M, v)
        for m in (0, 3, 7):
            Ym = small_m(qg, fmt, wd, N, K, (q[m:m + 1], d[m:m + 1], s[m:m + 1]), 1, v)
            assert np.array_equal(Y[m].view(np.uint32), Ym[0].view(np.uint32)), (fmt, v, m)


def test_rows_variant_is_the_gemv(qg):
    """For Q6_K and Q4_0 the DOT4 variant is the batch-1 GEMV on each row: equal bit for bit."""
    g = np.random.default_rng(13)
    for fmt in ("q6_k", "q4_0"):
        N, K, M = 300, 2048, 5
        w = WEIGHTS[fmt](g, N, K)
        x, _ = synth.activation(g, M, K)
        wd = dev(w)
        q, d, s = quantize(qg, x)
        Y = small_m(qg, fmt, wd, N, K, (q, d, s), M, qg.QGEMV_VARIANT_DOT4)
        for m in range(M):
            y = torch.empty(N, dtype=torch.float32, device="cuda:0")
            qg.GEMV[fmt](wd, N, K, q[m], d[m], s[m], y)
            assert np.array_equal(Y[m].view(np.uint32), host(y).view(np.uint32)), (fmt, m)
    # Q4_K under AUTO with one row is the batch-1 GEMV itself
    N, K = 300, 4096
    w = synth.q4_k_weights(g, N, K)
    x, _ = synth.activation(g, 1, K)
    wd = dev(w)
    q, d, s = quantize(qg, x)
    Y = small_m(qg, "q4_k", wd, N, K, (q, d, s), 1, qg.QGEMV_VARIANT_AUTO)
    y = torch.empty(N, dtype=torch.float32, device="cuda:0")
    qg.qgemv_q4_k(wd, N, K, q[0], d[0], s[0], y)
    assert np.array_equal(Y[0].view(np.uint32), host(y).view(np.uint32))


@pytest.mark.parametrize("fmt,M,N,K", [("q6_k", 8, 8200, 1024), ("q6_k", 40, 8192, 512),
                                       ("q4_0", 20, 8224, 896), ("q4_0", 64, 8192, 256),
                                       ("q4_k", 3, 8192, 2304)])
def test_wide_shapes(qg, fmt, M, N, K):
    """Matrices with many row tiles take the configuration without the K split."""
    g = np.random.default_rng(N + K + M)
    w = WEIGHTS[fmt](g, N, K)
    x, _ = synth.activation(g, M, K)
    act = quantize(qg, x)
    rows, Y_ref, TT = sampled(fmt, w, N, K, act_host(*act), [(0, 200), (4000, 100), (N - 150, 150)])
    say("small_m wide", fmt, M, N, K)
    Y = small_m(qg, fmt, dev(w), N, K, act, M, qg.QGEMV_VARIANT_MFMA)
    check_y(Y[:, rows].reshape(-1), Y_ref.reshape(-1), TT.reshape(-1), f"wide {fmt} M={M} N={N} K={K}")


# Every bucket edge of M on both matrix widths, with ragged tiles (N not a
# multiple of 64) and, for Q4_0, K not a multiple of 256 (a partial last unit).
EDGE_M = [1, 2, 7, 8, 9, 16, 17, 32, 33, 48, 49, 64]


@pytest.mark.parametrize("fmt", ["q4_k", "q6_k", "q4_0"])
@pytest.mark.parametrize("wide", [False, True])
def test_small_m_bucket_edges(qg, fmt, wide):
    N = 8200 if wide else 600
    K = 1056 if fmt == "q4_0" else 1280
    g = np.random.default_rng(N + K + len(fmt))
    w = WEIGHTS[fmt](g, N, K)
    wd = dev(w)
    x64, _ = synth.activation(g, 64, K)
    windows = [(0, 96), (N // 2, 40), (N - 70, 70)]
    for M in EDGE_M:
        act = quantize(qg, x64[:M])
        rows, Y_ref, TT = sampled(fmt, w, N, K, act_host(*act), windows)
        say("small_m edges", fmt, "wide" if wide else "narrow", M)
        for v in (qg.QGEMV_VARIANT_MFMA_STREAM, qg.QGEMV_VARIANT_MFMA_STAGED):
            Y = small_m(qg, fmt, wd, N, K, act, M, v)
            assert np.all(np.isfinite(Y))
            check_y(Y[:, rows].reshape(-1), Y_ref.reshape(-1), TT.reshape(-1),
                    f"edges {fmt} wide={wide} M={M} v={v}")


@pytest.mark.parametrize("fmt", ["q4_k", "q6_k", "q4_0"])
def test_small_m_deterministic_and_row_independent(qg, fmt):
    """Same inputs, same bits; row m of an M-row call equals a call on that
    row alone within the same bucket of M."""
    g = np.random.default_rng(77)
    N, K = 8256, 2048
    w = WEIGHTS[fmt](g, N, K)
    wd = dev(w)
    x, _ = synth.activation(g, 8, K)
    q, d, s = quantize(qg, x)
    for v in (qg.QGEMV_VARIANT_MFMA_STREAM, qg.QGEMV_VARIANT_MFMA):
        Y1 = small_m(qg, fmt, wd, N, K, (q, d, s), 8, v)
        Y2 = small_m(qg, fmt, wd, N, K, (q, d, s), 8, v)
        assert np.array_equal(Y1.view(np.uint32), Y2.view(np.uint32))
        for m in (0, 5, 7):
            Ym = small_m(qg, fmt, wd, N, K, (q[m:m + 1], d[m:m + 1], s[m:m + 1]), 1, v)
            assert np.array_equal(Y1[m].view(np.uint32), Ym[0].view(np.uint32)), (fmt, v, m)


# The DOT4 variant passes up to four activation rows at a time through the
# batch-1 streaming kernel with the batch-1 slices: for rows of more than 32
# units (the rows that kernel takes) each output row has the bits of the
# batch-1 GEMV on its activation row.  Covers split-K widths 1, 2 and 4,
# M = 2, 3 (a group of four with one repeated row), 4, 5 and 7 (two groups).
ROWS_BITS = [("q4_k", 2, 700, 4096), ("q4_k", 3, 513, 8192), ("q4_k", 5, 130, 14336),
             ("q6_k", 2, 301, 4096), ("q6_k", 4, 300, 14336), ("q6_k", 7, 64, 8192),
             ("q4_0", 2, 333, 4096), ("q4_0", 4, 100, 4128), ("q4_0", 5, 64, 14336)]


@pytest.mark.parametrize("fmt,M,N,K", ROWS_BITS)
def test_small_m_dot4_rows_equal_gemv_bits(qg, fmt, M, N, K):
    g = np.random.default_rng(M * 7 + N + K)
    w = WEIGHTS[fmt](g, N, K)
    x, _ = synth.activation(g, M, K)
    q, d, s = quantize(qg, x)
    wd = dev(w)
    say("small_m dot4 rows vs gemv", fmt, M, N, K)
    Y = small_m(qg, fmt, wd, N, K, (q, d, s), M, qg.QGEMV_VARIANT_DOT4)
    for m in range(M):
        y1 = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda:0")
        qg.GEMV[fmt](wd, N, K, q[m], d[m], s[m], y1)
        assert np.array_equal(Y[m].view(np.uint32), host(y1).view(np.uint32)), (fmt, M, m)
    qh, dh, sh = act_host(q, d, s)
    Y_ref, TT = oracle.gemm(fmt, w, N, K, qh, dh, sh)
    check_y(Y.reshape(-1), Y_ref.reshape(-1), TT.reshape(-1), f"dot4 rows {fmt} M={M}")


@pytest.mark.parametrize("M", [4, 12, 16])
def test_small_m_very_wide_q4k_resident_route(qg, M):
    """Q4_K matrices of at least six 16-row tiles per compute unit take the
    register-resident kernel under MFMA and AUTO from 9 to 16 rows, and the
    staged kernel's two-block tiles up to 8 rows (N = 24600: 1538 tiles, the
    last ragged); every output against the oracle, and the same bits as the
    forced RESIDENT or STAGED variant."""
    N, K = 24600, 1024
    g = np.random.default_rng(M + 99)
    w = WEIGHTS["q4_k"](g, N, K)
    x, _ = synth.activation(g, M, K)
    act = quantize(qg, x)
    q, d, s = act_host(*act)
    wd = dev(w)
    Y_ref, TT = oracle.gemm("q4_k", w, N, K, q, d, s)
    say("small_m very wide q4_k", M)
    Yr = small_m(qg, "q4_k", wd, N, K, act, M, qg.QGEMV_VARIANT_MFMA_RESIDENT)
    check_y(Yr.reshape(-1), Y_ref.reshape(-1), TT.reshape(-1), f"resident M={M}")
    Ys = small_m(qg, "q4_k", wd, N, K, act, M, qg.QGEMV_VARIANT_MFMA_STAGED)
    check_y(Ys.reshape(-1), Y_ref.reshape(-1), TT.reshape(-1), f"staged M={M}")
    routed = Yr if M > 8 else Ys
    for v in (qg.QGEMV_VARIANT_MFMA, qg.QGEMV_VARIANT_AUTO):
        Y = small_m(qg, "q4_k", wd, N, K, act, M, v)
        assert np.array_equal(Y.view(np.uint32), routed.view(np.uint32)), v
