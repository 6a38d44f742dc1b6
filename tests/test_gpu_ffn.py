"""Llama-3.1-8B-shaped decode FFN on the GPU, stream-ordered, no host round trip:
quantize(x) -> gate|up Q4_K GEMV -> SiLU(gate)*up + requantize -> down Q6_K GEMV.
The down product's input is the GPU's own h, re-quantised; the oracle checks
h against float64 SiLU*up, then quantises the GPU's h and must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import act_host, block_dots, check_y, dev, host, quantize, sample_rows, say

pytestmark = pytest.mark.gpu


def test_config2_ffn_chain():
    import block_quantized_gemv_w4a8_amd as qg
    c = synth.config2()
    Ngu, Kgu, Nd, Kd = c["N_gu"], c["K_gu"], c["N_down"], c["K_down"]
    say("config2 ffn chain")
    wgu, wdn = dev(c["w_gu"]), dev(c["w_down"])
    xd = dev(c["x"])
    q1, d1, s1 = qg.act_buffers(1, Kgu, "cuda:0")
    gu = torch.empty(Ngu, dtype=torch.float32, device="cuda:0")
    q2, d2, s2 = qg.act_buffers(1, Kd, "cuda:0")
    h = torch.empty(Kd, dtype=torch.float32, device="cuda:0")
    y = torch.empty(Nd, dtype=torch.float32, device="cuda:0")
    # the whole chain enqueued back to back on one stream
    qg.qgemv_quantize_act(xd, 1, Kgu, Kgu, q1, d1, s1)
    qg.qgemv_q4_k(wgu, Ngu, Kgu, q1, d1, s1, gu)
    qg.qgemv_silu_mul_quantize(gu, Kd, q2, d2, s2, h)
    qg.qgemv_q6_k(wdn, Nd, Kd, q2, d2, s2, y)
    torch.cuda.synchronize()

    qa, da, sa = act_host(q1, d1, s1)
    rq, rd, rs = oracle.quantize_act(c["x"])
    assert np.array_equal(qa, rq) and np.array_equal(da, rd) and np.array_equal(sa, rs)
    guh = host(gu)
    y_ref, T = oracle.gemv("q4_k", c["w_gu"], Ngu, Kgu, qa, da, sa)
    check_y(guh, y_ref, T, "gate|up")
    hh = host(h)
    href = oracle.silu_mul(guh)
    assert np.all(np.abs(hh - href) <= 1e-6 * np.abs(href) + 1e-30)
    qb, db, sb = act_host(q2, d2, s2)
    rq, rd, rs = oracle.quantize_act(hh[None], K=Kd)
    assert np.array_equal(qb, rq) and np.array_equal(db, rd) and np.array_equal(sb, rs)
    yh = host(y)
    y_ref, T = oracle.gemv("q6_k", c["w_down"], Nd, Kd, qb, db, sb)
    check_y(yh, y_ref, T, "down")
    # integer stages of both products, bit for bit, on sampled windows
    dots = block_dots(qg, "q4_k", wgu, Ngu, Kgu, q1, 14000, 600)
    assert np.array_equal(dots, oracle.block_dots("q4_k", c["w_gu"], Ngu, Kgu, qa, rows=(14000, 600)))
    dots = block_dots(qg, "q6_k", wdn, Nd, Kd, q2, 0, 256)
    assert np.array_equal(dots, oracle.block_dots("q6_k", c["w_down"], Nd, Kd, qb, rows=(0, 256)))
