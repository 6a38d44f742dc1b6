"""Integer block dots through the loaders the streaming GEMV kernels run
(qgemv_block_dots_staged: split-K slices staged in 16-byte chunks, parked in
LDS, fields read back with the misaligned-field readers, the activation in
the kernels' registers), bit for bit against oracle.block_dots, for every
format and split-K width 1, 2, 4 -- including Q4_0/Q8_0 rows with an odd
number of blocks, Q4_K/Q6_K rows padded to whole super-blocks, and the
repacked Q6_K rows whose last slice of four lies past the row (K = 8448,
16640)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    ("q4_0", [32, 96, 1056, 4096, 4128]),
    ("q8_0", [32, 1056, 4096]),
    ("q4_k", [256, 896, 4096, 8192, 14336]),
    ("q6_k", [256, 896, 4096, 14336]),
    ("q6_k_r8", [256, 4096, 8448, 14336, 16640]),
]
PARAMS = [(f, K) for f, Ks in CASES for K in Ks]


def _production_wk(fmt, K):
    """The split-K width the streaming kernels take for this row length."""
    kp = (K + 255) // 256 * 256
    U = kp // 64 if fmt in ("q4_k", "q6_k", "q6_k_r8") else (K + 63) // 64
    return 4 if U > 128 else (2 if U > 64 else 1)


@pytest.mark.parametrize("fmt,K", PARAMS)
def test_staged_dots_equal_oracle(fmt, K):
    import block_quantized_gemv_w4a8_amd as qg
    N, row0, nrows = 41, 3, 35
    g = synth.rng(1000 + K)
    native = "q6_k" if fmt == "q6_k_r8" else fmt
    w = synth.weights(native, g, N, K)
    x, _ = synth.activation(g, 1, K)
    q, d, s = oracle.quantize_act(x)
    ref = oracle.block_dots(native, w, N, K, q, rows=(row0, nrows))
    wd = dev(w)
    if fmt == "q6_k_r8":
        wr = torch.empty((N, qg.q6_k_r8_row_bytes(K)), dtype=torch.uint8, device=DEV)
        qg.qgemv_q6_k_repack(wd, N, K, wr)
        wd = wr
    qd, dd, sd = dev(q), dev(d), dev(s)
    ran = []
    for wk in (1, 2, 4):
        out = torch.full(ref.shape, -(2**31), dtype=torch.int32, device=DEV)
        say(f"staged block dots {fmt} K={K} wk={wk}")
        try:
            qg.qgemv_block_dots_staged(qg.FMT_ID[fmt], wd, N, K, row0, nrows, qd, dd, sd, wk,
                                       out)
        except qg.QgemvError as e:
            assert e.status == qg.QGEMV_E_UNSUPPORTED, e
            assert wk != _production_wk(fmt, K), "the kernels' own split must be supported"
            continue
        got = host(out)
        assert np.array_equal(got, ref), (fmt, K, wk, np.argwhere(got != ref)[:5])
        ran.append(wk)
    assert _production_wk(fmt, K) in ran


def test_staged_dots_full_size_window():
    """The lm_head's repacked Q6_K rows (K = 4096) and the down product's
    (K = 14336): windows of real-size matrices through the staged loaders."""
    import block_quantized_gemv_w4a8_amd as qg
    for N, K, seed in ((2048, 4096, 3), (512, 14336, 2)):
        g = synth.rng(seed)
        w = synth.weights("q6_k", g, N, K)
        x, _ = synth.activation(g, 1, K)
        q, d, s = oracle.quantize_act(x)
        ref = oracle.block_dots("q6_k", w, N, K, q, rows=(N - 300, 300))
        wr = torch.empty((N, qg.q6_k_r8_row_bytes(K)), dtype=torch.uint8, device=DEV)
        qg.qgemv_q6_k_repack(dev(w), N, K, wr)
        out = torch.full(ref.shape, -(2**31), dtype=torch.int32, device=DEV)
        say(f"staged block dots r8 full window N={N} K={K}")
        qg.qgemv_block_dots_staged(qg.QGEMV_FMT_Q6_K_R8, wr, N, K, N - 300, 300, dev(q), dev(d),
                                   dev(s), _production_wk("q6_k_r8", K), out)
        assert np.array_equal(host(out), ref)
