"""Batch-1 GEMV on the GPU against the oracle: block dots bit for bit, fp32
outputs within 1e-5 * sum|terms| + 1e-7, at sizes that span several
workgroups and ragged tails, and at the full workload sizes (sampled rows)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (act_host, block_dots, check_y, dev, gemv, host, oracle_rows, quantize,
                      sample_rows, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qg():
    import block_quantized_gemv_w4a8_amd as qg
    return qg


def run_case(qg, fmt, N, K, seed, full_dots=True):
    say("gemv", fmt, "N", N, "K", K, "seed", seed)
    g = np.random.default_rng(seed)
    w = synth.weights(fmt, g, N, K)
    x, _ = synth.activation(g, 1, K)
    act = quantize(qg, x)
    q, d, s = act_host(*act)
    # the GPU activation is itself bit-exact
    rq, rd, rs = oracle.quantize_act(x)
    assert np.array_equal(q, rq) and np.array_equal(d, rd) and np.array_equal(s, rs)
    wd = dev(w)
    y = gemv(qg, fmt, wd, N, K, act)
    assert np.all(np.isfinite(y))
    y_ref, T = oracle.gemv(fmt, w, N, K, q, d, s)
    check_y(y, y_ref, T, f"{fmt} N={N} K={K}")
    if full_dots:
        dots = block_dots(qg, fmt, wd, N, K, act[0], 0, N)
        ref = oracle.block_dots(fmt, w, N, K, q)
        assert np.array_equal(dots, ref), f"block dots differ {fmt} N={N} K={K}"
    return wd, act, y


SHAPES = {
    "q4_0": [(1, 32), (3, 64), (65, 96), (257, 896), (64, 4096), (33, 4864), (5, 32768),
             (1000, 160)],
    "q4_k": [(1, 256), (3, 288), (65, 896), (257, 1024), (64, 4096), (33, 4864),
             (17, 14336), (5, 32768), (1000, 512)],
    "q6_k": [(1, 256), (3, 288), (65, 896), (257, 1024), (64, 4096), (33, 4864),
             (17, 14336), (5, 32768), (1000, 512)],
    "q8_0": [(1, 32), (3, 96), (65, 896), (64, 4096), (33, 4864), (5, 32768)],
}


@pytest.mark.parametrize("fmt,N,K", [(f, N, K) for f, v in SHAPES.items() for N, K in v])
def test_gemv_shapes(qg, fmt, N, K):
    run_case(qg, fmt, N, K, seed=N * 7 + K)


@pytest.mark.parametrize("fmt", ["q4_0", "q4_k", "q6_k", "q8_0"])
def test_gemv_deterministic_and_partial_dots(qg, fmt):
    N, K = 300, 1024 if fmt in ("q4_k", "q6_k") else 992
    wd, act, y1 = run_case(qg, fmt, N, K, seed=99, full_dots=False)
    y2 = gemv(qg, fmt, wd, N, K, act)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    # a row window of the block dots equals the same rows of the full set
    full = block_dots(qg, fmt, wd, N, K, act[0], 0, N)
    part = block_dots(qg, fmt, wd, N, K, act[0], 123, 77)
    assert np.array_equal(part, full[123:200])


def test_gemv_empty_and_refusals_leave_output(qg):
    N, K = 64, 256
    g = np.random.default_rng(0)
    wd = dev(synth.q4_k_weights(g, N, K))
    x, _ = synth.activation(g, 1, K)
    q, d, s = quantize(qg, x)
    y = torch.full((N,), 5.0, device="cuda:0")
    qg.qgemv_q4_k(wd, 0, K, q, d, s, y)          # empty: no-op
    with pytest.raises(qg.QgemvError):
        qg.qgemv_q4_k(wd, N, 48, q, d, s, y)      # bad K: refused
    with pytest.raises(qg.QgemvError):
        qg.qgemv_q4_k(wd, N, 65536, q, d, s, y)   # beyond K_MAX: declined
    assert np.all(host(y) == 5.0)


def test_config0_q4_0(qg):
    c = synth.config0()
    say("config0")
    act = quantize(qg, c["x"])
    q, d, s = act_host(*act)
    wd = dev(c["w"])
    y = gemv(qg, "q4_0", wd, c["N"], c["K"], act)
    y_ref, T = oracle.gemv("q4_0", c["w"], c["N"], c["K"], q, d, s)
    check_y(y, y_ref, T, "config0")
    dots = block_dots(qg, "q4_0", wd, c["N"], c["K"], act[0], 0, c["N"])
    assert np.array_equal(dots, oracle.block_dots("q4_0", c["w"], c["N"], c["K"], q))


def test_config1_q4_k_layer(qg):
    c = synth.config1()
    for name, m in c["mats"].items():
        say("config1", name, m["N"], m["K"])
        act = quantize(qg, m["x"])
        q, d, s = act_host(*act)
        assert np.array_equal(q, oracle.quantize_act(m["x"])[0])
        wd = dev(m["w"])
        y = gemv(qg, "q4_k", wd, m["N"], m["K"], act)
        y_ref, T = oracle.gemv("q4_k", m["w"], m["N"], m["K"], q, d, s)
        check_y(y, y_ref, T, f"config1 {name}")
        dots = block_dots(qg, "q4_k", wd, m["N"], m["K"], act[0], 0, m["N"])
        assert np.array_equal(dots, oracle.block_dots("q4_k", m["w"], m["N"], m["K"], q))


def test_config3_lm_head_q6_k(qg):
    c = synth.config3()
    N, K = c["N"], c["K"]
    say("config3", N, K)
    act = quantize(qg, c["x"])
    q, d, s = act_host(*act)
    wd = dev(c["w"])
    y = gemv(qg, "q6_k", wd, N, K, act)
    assert np.all(np.isfinite(y))
    rows = sample_rows(N, 4096, seed=3)
    y_ref, T = oracle_rows("q6_k", c["w"], N, K, q, d, s, rows)
    check_y(y[rows], y_ref, T, "config3 sampled rows")
    # block dots bit-exact on two windows (start and end of the matrix)
    for r0, nr in [(0, 512), (N - 512, 512)]:
        dots = block_dots(qg, "q6_k", wd, N, K, act[0], r0, nr)
        ref = oracle.block_dots("q6_k", c["w"], N, K, q, rows=(r0, nr))
        assert np.array_equal(dots, ref)


# Q8_0 and Q4_0 at the gate/up shape (14336 x 4096), as the benchmark times
# them: sampled rows against the oracle, block dots bit-exact at both ends.
@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_gate_up_shape_q8_0_q4_0(qg, fmt):
    N, K = 14336, 4096
    g = np.random.default_rng(13 + len(fmt))
    w = synth.weights(fmt, g, N, K)
    x, _ = synth.activation(g, 1, K)
    say("gate/up shape", fmt, N, K)
    act = quantize(qg, x)
    q, d, s = act_host(*act)
    wd = dev(w)
    y = gemv(qg, fmt, wd, N, K, act)
    assert np.all(np.isfinite(y))
    rows = sample_rows(N, 2048, seed=5)
    y_ref, T = oracle_rows(fmt, w, N, K, q, d, s, rows)
    check_y(y[rows], y_ref, T, f"{fmt} {N}x{K} sampled rows")
    for r0, nr in [(0, 256), (N - 256, 256)]:
        dots = block_dots(qg, fmt, wd, N, K, act[0], r0, nr)
        assert np.array_equal(dots, oracle.block_dots(fmt, w, N, K, q, rows=(r0, nr)))


# Matrices with at least 256 rows per compute unit (65536 on MI355X) take the
# dynamic-row kernel: one 8-wave workgroup per compute unit whose waves pull
# rows from a counter in LDS.  Tall, ragged shapes (N not a multiple of its 8-row
# groups) for every format and split-K width, checked on sampled rows (the
# first and last 64 and a seeded spread) and, with the activation quantised
# in the launch, against the two-call path bit for bit.
DYN_SHAPES = [("q4_0", 2304), ("q4_k", 2304), ("q6_k", 2304), ("q8_0", 2304), ("q6_k_r8", 2304),
              ("q4_k", 4864), ("q6_k", 4864), ("q4_k", 8448), ("q6_k_r8", 8448),
              ("q4_0", 16640)]


@pytest.mark.parametrize("fmt,K", DYN_SHAPES)
def test_dynamic_row_kernel(qg, fmt, K):
    N = 65600 + 3
    g = np.random.default_rng(K + len(fmt))
    base = "q6_k" if fmt == "q6_k_r8" else fmt
    w = synth.weights(base, g, N, K)
    x, _ = synth.activation(g, 1, K)
    act = quantize(qg, x)
    q, d, s = act_host(*act)
    wd = dev(w)
    if fmt == "q6_k_r8":
        wr = torch.empty((N, qg.q6_k_r8_row_bytes(K)), dtype=torch.uint8, device="cuda:0")
        qg.qgemv_q6_k_repack(wd, N, K, wr)
        wd = wr
    say("dynamic-row gemv", fmt, N, K)
    y = gemv(qg, fmt, wd, N, K, act)
    assert np.all(np.isfinite(y))
    rows = sample_rows(N, 1500, seed=K)
    y_ref, T = oracle_rows(base, w, N, K, q, d, s, rows)
    check_y(y[rows], y_ref, T, f"dynamic-row {fmt} N={N} K={K}")
    # the same product with x quantised in the launch
    xd = dev(np.ascontiguousarray(x.reshape(-1), dtype=np.float32))
    q2, d2, s2 = qg.act_buffers(1, K, "cuda:0")
    y2 = torch.full((N,), float("nan"), device="cuda:0")
    qg.qgemv_quantize_gemv(qg.FMT_ID[fmt], wd, N, K, xd, q2, d2, s2, y2)
    assert np.array_equal(host(y2).view(np.uint32), y.view(np.uint32))
