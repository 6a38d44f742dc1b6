"""Activation quantisation inside the product's own launch on the GPU
(qgemv_quantize_gemv, qgemv_quantize_q4_k_swiglu).

Each must equal, bit for bit, qgemv_quantize_act followed by the unfused
product on those codes: the codes, scales and sums it writes to q/d/s, and
every output.  The codes are also checked against the oracle's quantisation
of x, and the products against the oracle within the GEMV tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import act_host, check_y, dev, host, oracle_rows, quantize, sample_rows, say

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A


@pytest.fixture(scope="module")
def qg():
    import block_quantized_gemv_w4a8_amd as qg
    return qg


def act_out(qg, K):
    q, d, s = qg.act_buffers(1, K, "cuda:0")
    for t in (q, d, s):
        t.view(torch.uint8).fill_(SENTINEL)     # padding blocks must be written as zero
    return q, d, s


def same_bits(a, b):
    return np.array_equal(host(a).view(np.uint8), host(b).view(np.uint8))


def weights_dev(qg, fmt, w, N, K):
    """Device weights; Q6_K_R8 is the repacked copy of Q6_K weights."""
    wd = dev(w)
    if fmt != "q6_k_r8":
        return wd
    wr = torch.empty((N, qg.q6_k_r8_row_bytes(K)), dtype=torch.uint8, device="cuda:0")
    qg.qgemv_q6_k_repack(wd, N, K, wr)
    return wr


def fused_gemv(qg, fmt, wd, N, K, xd):
    q, d, s = act_out(qg, K)
    y = torch.full((N,), float("nan"), device="cuda:0")
    qg.qgemv_quantize_gemv(qg.FMT_ID[fmt], wd, N, K, xd, q, d, s, y)
    return (q, d, s), y


def two_call_gemv(qg, fmt, wd, N, K, x):
    act = quantize(qg, x)
    y = torch.full((N,), float("nan"), device="cuda:0")
    qg.GEMV[fmt](wd, N, K, *act, y)
    return act, y


# (N, K): rows of <= 32 units take the two launches inside the entry; longer
# rows the one-launch kernel with 1, 2 or 4 waves per row; K % 256 != 0 leaves
# zero activation blocks past K; K = 32768 exceeds the kernel's LDS with the
# activation row and falls back as well.
# Q6_K_R8 16032 x 4096 is one GPU's lm_head rows split 8 ways.
SHAPES = {
    "q4_0": [(1, 32), (65, 896), (257, 2080), (64, 4096), (33, 4128), (17, 14336), (3, 32768)],
    "q4_k": [(1, 256), (65, 1024), (257, 2304), (64, 4096), (33, 4384), (17, 14336),
             (3, 32768)],
    "q6_k": [(1, 256), (65, 1024), (257, 2304), (64, 4096), (33, 4384), (17, 14336),
             (3, 32768)],
    "q8_0": [(3, 96), (65, 896), (64, 4096), (33, 4864), (17, 14336)],
    "q6_k_r8": [(65, 1024), (64, 4096), (33, 4864), (9, 8448), (17, 14336), (5, 16640),
                (3, 32768), (16032, 4096)],
}


@pytest.mark.parametrize("fmt,N,K", [(f, N, K) for f, v in SHAPES.items() for N, K in v])
def test_quantize_gemv_shapes(qg, fmt, N, K):
    g = np.random.default_rng(N * 13 + K)
    base = "q6_k" if fmt == "q6_k_r8" else fmt
    w = synth.weights(base, g, N, K)
    x, _ = synth.activation(g, 1, K)
    wd = weights_dev(qg, fmt, w, N, K)
    xd = dev(np.ascontiguousarray(x.reshape(-1), dtype=np.float32))
    say("quantize_gemv", fmt, "N", N, "K", K)
    act, y = fused_gemv(qg, fmt, wd, N, K, xd)
    # the codes are the oracle's quantisation of x
    q, d, s = act_host(*act)
    rq, rd, rs = oracle.quantize_act(x)
    assert np.array_equal(q.reshape(-1), rq.reshape(-1))
    assert np.array_equal(d.reshape(-1), rd.reshape(-1))
    assert np.array_equal(s.reshape(-1), rs.reshape(-1))
    yh = host(y)
    y_ref, T = oracle.gemv(base, w, N, K, q, d, s)
    check_y(yh, y_ref, T, f"quantize_gemv {fmt} N={N} K={K}")
    # equal to the two calls it stands for, bit for bit
    act2, y2 = two_call_gemv(qg, fmt, wd, N, K, x)
    for a, b in zip(act, act2):
        assert same_bits(a, b)
    assert same_bits(y, y2)


def test_quantize_gemv_repeat_and_zero_blocks(qg):
    """Whole zero blocks of x (d = 0, q = 0, s = 0) and a second call on the
    same buffers give the same bits as the two-call path."""
    fmt, N, K = "q6_k_r8", 300, 4096
    g = np.random.default_rng(5)
    w = synth.weights("q6_k", g, N, K)
    x, _ = synth.activation(g, 1, K)
    x = x.reshape(-1).copy()
    x[32 * 7:32 * 9] = 0.0
    x[K - 32:] = 0.0
    wd = weights_dev(qg, fmt, w, N, K)
    xd = dev(x.astype(np.float32))
    say("quantize_gemv zero blocks")
    act, y = fused_gemv(qg, fmt, wd, N, K, xd)
    qg.qgemv_quantize_gemv(qg.FMT_ID[fmt], wd, N, K, xd, *act, y)
    act2, y2 = two_call_gemv(qg, fmt, wd, N, K, x[None])
    for a, b in zip(act, act2):
        assert same_bits(a, b)
    assert same_bits(y, y2)
    dh = host(act[1], np.uint16).reshape(-1)
    assert dh[7] == 0 and dh[8] == 0 and dh[K // 32 - 1] == 0


def test_quantize_gemv_lm_head_full_size(qg):
    """The large-vocab output projection (128256 x 4096 Q6_K, repacked) in the
    launch configuration the benchmark times."""
    c = synth.config3()
    N, K = c["N"], c["K"]
    wr = weights_dev(qg, "q6_k_r8", c["w"], N, K)
    xd = dev(np.ascontiguousarray(c["x"].reshape(-1), dtype=np.float32))
    say("quantize_gemv lm_head full size")
    act, y = fused_gemv(qg, "q6_k_r8", wr, N, K, xd)
    q, d, s = act_host(*act)
    rq, rd, rs = oracle.quantize_act(c["x"])
    assert np.array_equal(q.reshape(-1), rq.reshape(-1))
    assert np.array_equal(d.reshape(-1), rd.reshape(-1))
    yh = host(y)
    rows = sample_rows(N, 2048, seed=3)
    y_ref, T = oracle_rows("q6_k", c["w"], N, K, q, d, s, rows)
    check_y(yh[rows], y_ref, T, "lm_head quantize_gemv sampled rows")
    _, y2 = two_call_gemv(qg, "q6_k_r8", wr, N, K, c["x"])
    assert same_bits(y, y2)


def swiglu_fused_x(qg, wd, N, K, xd):
    act = act_out(qg, K)
    out = act_out(qg, N)
    gu = torch.full((2 * N,), float("nan"), device="cuda:0")
    h = torch.full((N,), float("nan"), device="cuda:0")
    qg.qgemv_quantize_q4_k_swiglu(wd, N, K, xd, *act, *out, gu, h)
    return act, out, gu, h


@pytest.mark.parametrize("N,K", [(32, 256), (96, 896), (320, 4096), (64, 4864), (544, 1024),
                                 (160, 14336), (8256, 2048), (24736, 512),
                                 (1792, 4096)])
def test_quantize_swiglu_shapes(qg, N, K):
    g = np.random.default_rng(N * 11 + K)
    w = synth.q4_k_weights(g, 2 * N, K)
    x, _ = synth.activation(g, 1, K)
    wd = dev(w)
    xd = dev(np.ascontiguousarray(x.reshape(-1), dtype=np.float32))
    say("quantize_swiglu", N, K)
    act, out, gu, h = swiglu_fused_x(qg, wd, N, K, xd)
    q, d, s = act_host(*act)
    rq, rd, rs = oracle.quantize_act(x)
    assert np.array_equal(q.reshape(-1), rq.reshape(-1))
    assert np.array_equal(d.reshape(-1), rd.reshape(-1))
    assert np.array_equal(s.reshape(-1), rs.reshape(-1))
    y_ref, T = oracle.gemv("q4_k", w, 2 * N, K, q, d, s)
    check_y(host(gu), y_ref, T, f"quantize_swiglu gate|up N={N} K={K}")
    # equal to quantize_act + the fused product on those codes
    act2 = quantize(qg, x)
    out2 = act_out(qg, N)
    gu2 = torch.empty(2 * N, device="cuda:0")
    h2 = torch.empty(N, device="cuda:0")
    qg.qgemv_q4_k_swiglu_quantize(wd, N, K, *act2, *out2, gu2, h2)
    for a, b in zip(act, act2):
        assert same_bits(a, b)
    for a, b in zip(out, out2):
        assert same_bits(a, b)
    assert same_bits(gu, gu2) and same_bits(h, h2)


def test_config2_chain_with_fused_quantisation(qg):
    """x -> quantize+gate|up+SwiGLU+quantise -> down Q6_K (repacked), equal
    bit for bit to the chain with the separate activation quantisation."""
    c = synth.config2()
    Kgu, Nd, Kd = c["K_gu"], c["N_down"], c["K_down"]
    wgu = dev(c["w_gu"])
    wdn = weights_dev(qg, "q6_k_r8", c["w_down"], Nd, Kd)
    xd = dev(np.ascontiguousarray(c["x"].reshape(-1), dtype=np.float32))
    say("config2 chain, fused quantisation")
    act, out, gu, h = swiglu_fused_x(qg, wgu, Kd, Kgu, xd)
    y = torch.empty(Nd, device="cuda:0")
    qg.qgemv_q6_k_r8(wdn, Nd, Kd, *out, y)
    qb, db, sb = act_host(*out)
    y_ref, T = oracle.gemv("q6_k", c["w_down"], Nd, Kd, qb, db, sb)
    check_y(host(y), y_ref, T, "down after fused quantisation")
    act2 = quantize(qg, c["x"])
    out2 = act_out(qg, Kd)
    qg.qgemv_q4_k_swiglu_quantize(wgu, Kd, Kgu, *act2, *out2, None, None)
    for a, b in zip(out, out2):
        assert same_bits(a, b)


def test_config0_and_config1_quantize_gemv(qg):
    """The launch-bound workloads: Q4_0 896x896 and every matrix of the
    Qwen2.5-0.5B-shaped Q4_K layer (K = 896 rows take the lanes-per-row
    kernel, down's K = 4864 the LDS-streaming one), each with its activation
    quantised in the launch; equal to the two-call path bit for bit and to
    the oracle within the tolerance."""
    c0 = synth.config0()
    cases = [("q4_0", c0["w"], 896, 896, c0["x"], "config0")]
    for name, m in synth.config1()["mats"].items():
        cases.append(("q4_k", m["w"], m["N"], m["K"], m["x"], f"config1 {name}"))
    for fmt, w, N, K, x, what in cases:
        say("quantize_gemv", what)
        wd = dev(w)
        xd = dev(np.ascontiguousarray(x.reshape(-1), dtype=np.float32))
        act, y = fused_gemv(qg, fmt, wd, N, K, xd)
        q, d, s = act_host(*act)
        y_ref, T = oracle.gemv(fmt, w, N, K, q, d, s)
        check_y(host(y), y_ref, T, f"quantize_gemv {what}")
        act2, y2 = two_call_gemv(qg, fmt, wd, N, K, x)
        for a, b in zip(act, act2):
            assert same_bits(a, b), what
        assert same_bits(y, y2), what
