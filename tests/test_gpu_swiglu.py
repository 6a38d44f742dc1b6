"""The fused gate|up -> SwiGLU -> quantise product on the GPU.

It must equal, bit for bit, the two-launch path (qgemv_q4_k on the 2N rows,
then qgemv_silu_mul_quantize), and against the oracle: [gate | up] within the
GEMV tolerance, h within 1e-6 |h| of float64 silu(g) * u of the GPU's own
[gate | up], and the activation codes, scales and sums equal to the oracle's
quantisation of the GPU's h."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import act_host, check_y, dev, host, quantize, say

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A


@pytest.fixture(scope="module")
def qg():
    import block_quantized_gemv_w4a8_amd as qg
    return qg


def out_buffers(qg, N):
    q, d, s = qg.act_buffers(1, N, "cuda:0")
    for t in (q, d, s):
        t.view(torch.uint8).fill_(SENTINEL)     # padding must be overwritten with zeros
    return q, d, s


def fused(qg, wd, N, K, act, with_fp=True):
    q, d, s = act
    qo, do, so = out_buffers(qg, N)
    gu = torch.full((2 * N,), float("nan"), device="cuda:0") if with_fp else None
    h = torch.full((N,), float("nan"), device="cuda:0") if with_fp else None
    qg.qgemv_q4_k_swiglu_quantize(wd, N, K, q, d, s, qo, do, so, gu, h)
    return (qo, do, so), gu, h


def two_launch(qg, wd, N, K, act):
    q, d, s = act
    gu = torch.empty(2 * N, device="cuda:0")
    qg.qgemv_q4_k(wd, 2 * N, K, q, d, s, gu)
    qo, do, so = out_buffers(qg, N)
    h = torch.empty(N, device="cuda:0")
    qg.qgemv_silu_mul_quantize(gu, N, qo, do, so, h)
    return (qo, do, so), gu, h


def same_bits(a, b):
    return np.array_equal(host(a).view(np.uint8), host(b).view(np.uint8))


def check_against_oracle(w, N, K, act, out, gu, h):
    qa, da, sa = act_host(*act)
    y_ref, T = oracle.gemv("q4_k", w, 2 * N, K, qa, da, sa)
    guh = host(gu)
    check_y(guh, y_ref, T, f"swiglu gate|up N={N} K={K}")
    hh = host(h)
    href = oracle.silu_mul(guh)
    assert np.all(np.abs(hh - href) <= 1e-6 * np.abs(href) + 1e-30)
    rq, rd, rs = oracle.quantize_act(hh[None], K=N)
    qo, do, so = act_host(*out)
    assert np.array_equal(qo.reshape(-1), rq.reshape(-1))
    assert np.array_equal(do.reshape(-1), rd.reshape(-1))
    assert np.array_equal(so.reshape(-1), rs.reshape(-1))


# N = 8256 and 24736 give a workgroup of the dynamic-row kernel two and up
# to four output blocks (one unit per 256 blocks), with a ragged remainder
# (N = 1792, K = 4096: one GPU's gate|up rows when the FFN is split 8 ways)
@pytest.mark.parametrize("N,K", [(32, 256), (96, 896), (320, 4096), (64, 4864), (160, 32768),
                                 (544, 1024), (1056, 2048), (8256, 2048), (24736, 512),
                                 (1792, 4096)])
def test_fused_shapes(qg, N, K):
    g = np.random.default_rng(N * 7 + K)
    w = synth.q4_k_weights(g, 2 * N, K)
    x, _ = synth.activation(g, 1, K)
    act = quantize(qg, x)
    wd = dev(w)
    say("swiglu fused", N, K)
    out, gu, h = fused(qg, wd, N, K, act)
    check_against_oracle(w, N, K, act, out, gu, h)
    ref_out, ref_gu, ref_h = two_launch(qg, wd, N, K, act)
    assert same_bits(gu, ref_gu) and same_bits(h, ref_h)
    for a, b in zip(out, ref_out):
        assert same_bits(a, b)
    # without the optional fp32 outputs: the same activation
    out2, _, _ = fused(qg, wd, N, K, act, with_fp=False)
    for a, b in zip(out2, ref_out):
        assert same_bits(a, b)


def test_config2_fused_chain(qg):
    """quantize(x) -> fused gate|up+SwiGLU+quantise -> down Q6_K, checked at
    every stage, and equal to the unfused chain bit for bit."""
    c = synth.config2()
    Ngu, Kgu, Nd, Kd = c["N_gu"], c["K_gu"], c["N_down"], c["K_down"]
    assert Ngu == 2 * Kd
    wgu, wdn = dev(c["w_gu"]), dev(c["w_down"])
    act = quantize(qg, c["x"])
    say("config2 fused chain")
    out, gu, h = fused(qg, wgu, Kd, Kgu, act)
    check_against_oracle(c["w_gu"], Kd, Kgu, act, out, gu, h)
    y = torch.empty(Nd, device="cuda:0")
    qg.qgemv_q6_k(wdn, Nd, Kd, *out, y)
    qb, db, sb = act_host(*out)
    y_ref, T = oracle.gemv("q6_k", c["w_down"], Nd, Kd, qb, db, sb)
    check_y(host(y), y_ref, T, "down after fused")
    ref_out, ref_gu, _ = two_launch(qg, wgu, Kd, Kgu, act)
    assert same_bits(gu, ref_gu)
    for a, b in zip(out, ref_out):
        assert same_bits(a, b)
