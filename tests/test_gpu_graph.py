"""The decode step captured as one HIP graph (through torch.cuda.CUDAGraph):
every replay must give the eager result bit for bit, with eager work and
synchronisations between the replays.  The entries allocate nothing and
never synchronise, so their launches are capturable as they stand."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qg():
    import block_quantized_gemv_w4a8_amd as qg
    return qg


def bits(t):
    return host(t).view(np.uint8).copy()


def test_decode_step_graph_replays(qg):
    """x -> quantise + gate|up + SwiGLU + requantise -> down (repacked Q6_K)
    -> quantise + lm_head, at reduced sizes with the same structure (the
    lm_head rows exceed 256 per compute unit, so it takes the dynamic-row
    kernel as in the full-size step)."""
    dev = "cuda:0"
    g = np.random.default_rng(21)
    Kgu, Nff, Nh = 1024, 2048, 70000
    w_gu = torch.from_numpy(synth.q4_k_weights(g, 2 * Nff, Kgu)).to(dev)
    w_dn = torch.from_numpy(synth.q6_k_weights(g, Kgu, Nff)).to(dev)
    w_hd = torch.from_numpy(synth.q6_k_weights(g, Nh, Kgu)).to(dev)
    rep = []
    for wt, N, K in ((w_dn, Kgu, Nff), (w_hd, Nh, Kgu)):
        wr = torch.empty((N, qg.q6_k_r8_row_bytes(K)), dtype=torch.uint8, device=dev)
        qg.qgemv_q6_k_repack(wt, N, K, wr)
        rep.append(wr)
    w_dn_r, w_hd_r = rep
    x = torch.from_numpy(synth.activation(g, 1, Kgu)[0].reshape(-1)).to(dev)
    xh = torch.from_numpy(synth.activation(g, 1, Kgu)[0].reshape(-1)).to(dev)
    q1, d1, s1 = qg.act_buffers(1, Kgu, dev)
    q2, d2, s2 = qg.act_buffers(1, Nff, dev)
    q3, d3, s3 = qg.act_buffers(1, Kgu, dev)
    y = torch.empty(Kgu, device=dev)
    logits = torch.empty(Nh, device=dev)

    def step():
        sh = torch.cuda.current_stream().cuda_stream
        qg.qgemv_quantize_q4_k_swiglu(w_gu, Nff, Kgu, x, q1, d1, s1, q2, d2, s2, None, None,
                                      stream=sh)
        qg.qgemv_q6_k_r8(w_dn_r, Kgu, Nff, q2, d2, s2, y, stream=sh)
        qg.qgemv_quantize_gemv(qg.QGEMV_FMT_Q6_K_R8, w_hd_r, Nh, Kgu, xh, q3, d3, s3, logits,
                               stream=sh)

    say("graph: eager step")
    step()
    torch.cuda.synchronize()
    ref = [bits(t) for t in (q2, d2, s2, y, logits)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(5):
        say("graph: replay", r)
        for t in (y, logits):
            t.fill_(float("nan"))
        q2.fill_(7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [bits(t) for t in (q2, d2, s2, y, logits)]
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), f"replay {r}"
        # eager work between replays, on other buffers
        scratch = torch.randn(4096, device=dev)
        qg.qgemv_quantize_act(scratch, 1, 4096, 4096, *qg.act_buffers(1, 4096, dev))
        torch.cuda.synchronize()
