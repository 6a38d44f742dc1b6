"""GPU activation quantisation and SwiGLU+quantisation against the oracle, bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import act_host, dev, host, quantize, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qg():
    import block_quantized_gemv_w4a8_amd as qg
    return qg


def _cmp(qg, x, K=None, what=""):
    say("quantize", what, x.shape, K)
    got = act_host(*quantize(qg, x, K))
    ref = oracle.quantize_act(x, K=K)
    for name, a, b in zip("qds", got, ref):
        assert np.array_equal(a, b), f"{what}: {name} differs at {np.argwhere(a != b)[:5].tolist()}"


@pytest.mark.parametrize("M,K,ldx", [(1, 32, 32), (1, 896, 896), (5, 96, 96), (3, 4096, 4100),
                                     (1, 4864, 4864), (2, 14336, 14336), (64, 4096, 4096),
                                     (8, 4096, 4096), (1, 32768, 32768), (7, 288, 301)])
def test_quantize_random(qg, M, K, ldx):
    g = np.random.default_rng(M * 1000 + K)
    x, _ = synth.activation(g, M, ldx)
    x = x * np.float32(g.uniform(0.01, 10))
    _cmp(qg, x, K, f"random M={M} K={K} ldx={ldx}")


def test_quantize_special_blocks(qg):
    g = np.random.default_rng(1)
    K = 1024
    x = np.zeros((4, K), np.float32)
    x[0, 5] = 3.7                       # one-hot
    x[1, :32] = 0.37                    # all equal
    x[1, 32] = 127.0                    # exact ties (d = 1)
    x[1, 33:43] = [0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 62.5, -62.5, 126.5, -126.5]
    x[2] = g.standard_normal(K).astype(np.float32) * 1e-3
    x[2, 64:96] = 0                     # a zero block inside
    # near-ties around (k + 1/2) d for each block's own d
    for b in range(K // 32):
        a = np.float32(g.uniform(0.05, 60))
        d32 = np.float32(a / np.float32(127))
        ks = g.integers(0, 127, 31)
        x0 = ((ks + 0.5) * np.float64(d32)).astype(np.float32)
        pick = g.integers(0, 3, 31)
        xv = np.where(pick == 0, x0, np.where(pick == 1, np.nextafter(x0, np.float32(np.inf)),
                                                np.nextafter(x0, np.float32(0))))
        x[3, 32 * b] = a
        x[3, 32 * b + 1:32 * b + 32] = xv * np.where(g.integers(0, 2, 31) == 0, 1, -1)
    _cmp(qg, x, None, "special blocks")
    # subnormal / tiny and large magnitudes
    y = np.concatenate([np.full(32, 1e-40, np.float32), np.full(32, -3e-39, np.float32),
                        g.standard_normal(64).astype(np.float32) * 1e4])[None]
    _cmp(qg, y, None, "tiny and large")


@pytest.mark.parametrize("seed", [0, 1])
def test_quantize_dense_near_ties(qg, seed):
    """Every value within 1..40 ulp of a rounding boundary (k + 1/2) d of its
    block, over scales from 1e-30 to 1e30: the codes must still be those of the
    correctly rounded quotient."""
    g = np.random.default_rng(100 + seed)
    M, K = 16, 4096
    nb = K // 32
    amax = (10.0 ** g.uniform(-30, 30, size=(M, nb, 1))).astype(np.float32)
    d32 = (amax / np.float32(127)).astype(np.float32)
    k = g.integers(-127, 127, size=(M, nb, 31)).astype(np.float32)
    xv = ((k + np.float32(0.5)) * d32).astype(np.float32)
    steps = g.integers(-40, 41, size=xv.shape)
    for s in range(40):
        move = np.abs(steps) > s
        xv = np.where(move, np.nextafter(xv, np.where(steps > 0, np.float32(np.inf),
                                                      np.float32(-np.inf))), xv)
    xv = np.clip(xv, -amax, amax).astype(np.float32)
    x = np.concatenate([amax * np.where(g.integers(0, 2, (M, nb, 1)) == 0, 1, -1), xv],
                       axis=2).astype(np.float32)
    perm = g.permuted(np.tile(np.arange(32), (M, nb, 1)), axis=2)
    x = np.take_along_axis(x, perm, axis=2).reshape(M, K)
    _cmp(qg, x, None, f"dense near-ties seed {seed}")


def test_quantize_padding_and_empty(qg):
    import torch
    x = np.ones((2, 96), np.float32)
    q, d, s = qg.act_buffers(2, 96, "cuda:0")
    for t in (q, d, s):
        t.fill_(-1)
    qg.qgemv_quantize_act(dev(x), 2, 96, 96, q, d, s)
    qh, dh, sh = act_host(q, d, s)
    assert np.all(qh[:, :96] == 127) and not qh[:, 96:].any()
    assert not dh[:, 3:].any() and not sh[:, 3:].any()
    # M == 0 is a no-op
    q.fill_(7)
    qg.qgemv_quantize_act(dev(x), 0, 96, 96, q, d, s)
    assert np.all(host(q) == 7)
    # a refused call leaves the outputs untouched
    with pytest.raises(qg.QgemvError):
        qg.qgemv_quantize_act(dev(x), 2, 48, 96, q, d, s)
    torch.cuda.synchronize()
    assert np.all(host(q) == 7)


def test_quantize_deterministic(qg):
    x, _ = synth.activation(np.random.default_rng(3), 16, 4096)
    a = act_host(*quantize(qg, x))
    b = act_host(*quantize(qg, x))
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("N", [32, 96, 1024, 14336])
def test_silu_mul_quantize(qg, N):
    import torch
    say("silu_mul_quantize", N)
    g = np.random.default_rng(N)
    gu = (g.standard_normal(2 * N) * 3).astype(np.float32)
    gu[:4] = [0.0, -100.0, 100.0, -20.0]
    gud = dev(gu)
    q, d, s = qg.act_buffers(1, N, "cuda:0")
    h = torch.empty(N, dtype=torch.float32, device="cuda:0")
    qg.qgemv_silu_mul_quantize(gud, N, q, d, s, h)
    hh = host(h)
    ref = oracle.silu_mul(gu)
    assert np.all(np.abs(hh - ref) <= 1e-6 * np.abs(ref) + 1e-30), "h outside tolerance"
    # the codes are exactly the quantisation of the GPU's own h
    rq, rd, rs = oracle.quantize_act(hh[None], K=N)
    gq, gd, gs = act_host(q, d, s)
    assert np.array_equal(gq, rq) and np.array_equal(gd, rd) and np.array_equal(gs, rs)
    # without h the same codes come out
    q2, d2, s2 = qg.act_buffers(1, N, "cuda:0")
    qg.qgemv_silu_mul_quantize(gud, N, q2, d2, s2, None)
    for a, b in zip(act_host(q2, d2, s2), (gq, gd, gs)):
        assert np.array_equal(a, b)
