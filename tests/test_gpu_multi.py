"""Several GEMVs on one activation row in one call (qgemv_multi,
qgemv_quantize_multi) on the GPU: each output equal, bit for bit, to the
format's GEMV of that matrix alone, and to the oracle within the tolerance;
with the activation quantised in the launch, equal to qgemv_quantize_act
followed by qgemv_multi."""
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


def same_bits(a, b):
    return np.array_equal(host(a).view(np.uint8), host(b).view(np.uint8))


def run_multi(qg, fmt, ns, K, seed, quantize_in_launch=False):
    g = np.random.default_rng(seed)
    ws = [synth.weights(fmt, g, n, K) if n > 0 else None for n in ns]
    x, _ = synth.activation(g, 1, K)
    act = quantize(qg, x)
    wds = [dev(w) if w is not None else None for w in ws]
    ys = [torch.full((max(n, 1),), float("nan"), device="cuda:0") for n in ns]
    say("multi", fmt, ns, K, "xq" if quantize_in_launch else "")
    if quantize_in_launch:
        xd = dev(np.ascontiguousarray(x.reshape(-1), dtype=np.float32))
        q2, d2, s2 = qg.act_buffers(1, K, "cuda:0")
        for t in (q2, d2, s2):
            t.view(torch.uint8).fill_(0x5A)
        qg.qgemv_quantize_multi(qg.FMT_ID[fmt], wds, ns, K, xd, q2, d2, s2, ys)
        for a, b in zip((q2, d2, s2), act):
            assert same_bits(a, b)
    else:
        qg.qgemv_multi(qg.FMT_ID[fmt], wds, ns, K, *act, ys)
    q, d, s = act_host(*act)
    for i, (w, n) in enumerate(zip(ws, ns)):
        if n == 0:
            assert np.isnan(host(ys[i])).all()     # untouched
            continue
        y1 = torch.empty(n, device="cuda:0")
        qg.GEMV[fmt](wds[i], n, K, *act, y1)
        assert same_bits(ys[i], y1), (fmt, ns, K, i)
        y_ref, T = oracle.gemv(fmt, w, n, K, q, d, s)
        check_y(host(ys[i]), y_ref, T, f"multi {fmt} matrix {i} n={n} K={K}")


@pytest.mark.parametrize("fmt,ns,K", [
    ("q4_k", [896, 128, 128], 896),          # q, k, v of the Qwen2.5-0.5B-shaped layer
    ("q4_k", [4864, 4864], 896),             # its gate and up, stored apart
    ("q6_k", [1, 7, 300], 1024),
    ("q4_0", [33, 0, 65], 96),               # an empty matrix in the middle
    ("q8_0", [100], 2048),                   # one matrix
    ("q4_k", [3, 5, 7, 11, 13, 17, 19, 23], 512),   # QGEMV_MULTI_MAX matrices
    ("q4_k", [300, 200], 4096),              # long rows: one launch per matrix
    ("q6_k", [64, 65], 14336),
    ("q4_k", [0, 300], 4096),                # long rows, empty first matrix
    ("q6_k", [0, 64], 14336),
    ("q4_0", [0, 0, 40], 2048),              # short rows, empty first matrices
])
@pytest.mark.parametrize("xq", [False, True])
def test_multi(qg, fmt, ns, K, xq):
    run_multi(qg, fmt, ns, K, seed=sum(ns) + K, quantize_in_launch=xq)


def test_multi_refusals_leave_outputs(qg):
    g = np.random.default_rng(3)
    K = 256
    w = dev(synth.q4_k_weights(g, 10, K))
    act = quantize(qg, synth.activation(g, 1, K)[0])
    ys = [torch.full((10,), 5.0, device="cuda:0") for _ in range(9)]
    with pytest.raises(qg.QgemvError):
        qg.qgemv_multi(qg.QGEMV_FMT_Q4_K, [w] * 9, [10] * 9, K, *act, ys)   # count > 8
    with pytest.raises(qg.QgemvError):
        qg.qgemv_multi(qg.QGEMV_FMT_Q4_K, [w, w], [10, -1], K, *act, ys[:2])
    torch.cuda.synchronize()
    assert all(np.all(host(y) == 5.0) for y in ys)
