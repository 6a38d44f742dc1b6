"""The integer stage of the small-M matrix-core products, bit for bit: the
raw int32 tile of every MFMA (qgemm_small_m_block_dots, which runs the kernel
a variant selects for the shape, with its operand unpack from the staged
bytes) against oracle.block_dots of each activation row, for Q4_K, Q6_K and
Q4_0 on wide and narrow matrices in every bucket of M, through the staged
and the register-resident kernels.  The raw tiles use unsigned codes: the
oracle's Q4_0 dot plus 8 * s, Q6_K 16-group dot plus 32 * (the group's code
sum).  The product written beside the tiles equals the small-M entry's."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import act_host, dev, host, quantize, say

pytestmark = pytest.mark.gpu

WEIGHTS = {"q4_k": synth.q4_k_weights, "q6_k": synth.q6_k_weights, "q4_0": synth.q4_0_weights}
FMT = {"q4_k": 1, "q6_k": 2, "q4_0": 0}

# wide matrices (at least 512 tiles of 16 rows) and narrow ones, M in each
# bucket of 16 (and for Q4_K both halves of the first: two-block tiles up to
# M = 8; above 32 some take 32 activation rows per workgroup, the rest on a
# second grid dimension); N = 24600 takes the register-resident kernel under
# MFMA (Q4_K)
CASES = [("q4_k", 8, 8200, 1024), ("q4_k", 20, 8200, 1024), ("q4_k", 40, 8200, 1024),
         ("q4_k", 64, 8200, 1024), ("q4_k", 8, 600, 4096), ("q4_k", 24, 300, 4096),
         ("q4_k", 48, 200, 2048), ("q4_k", 64, 130, 4096), ("q4_k", 5, 24600, 1024),
         ("q4_k", 1, 8200, 1024), ("q4_k", 3, 600, 4096),
         ("q6_k", 8, 8200, 1024), ("q6_k", 24, 8200, 1024), ("q6_k", 40, 8200, 1024),
         ("q6_k", 8, 600, 4096), ("q6_k", 24, 300, 4096), ("q6_k", 48, 200, 2048),
         ("q6_k", 64, 130, 4096), ("q4_0", 8, 8200, 1056), ("q4_0", 40, 8200, 1056),
         ("q4_0", 8, 600, 4128), ("q4_0", 24, 300, 4096), ("q4_0", 64, 130, 4096),
         ("q4_k", 50, 8200, 1024), ("q4_0", 64, 8200, 1056), ("q4_0", 50, 200, 2048)]


def _expected(fmt, w, N, K, q, s, M):
    """Raw unsigned-code dots [M][N][nb] from the oracle's block dots."""
    out = []
    for m in range(M):
        D = oracle.block_dots(fmt, w, N, K, q[m]).astype(np.int64)
        if fmt == "q4_0":
            D = D + 8 * s[m][: D.shape[1]].astype(np.int64)[None, :]
        elif fmt == "q6_k":
            g16 = q[m][: 16 * D.shape[1]].astype(np.int64).reshape(-1, 16).sum(axis=1)
            D = D + 32 * g16[None, :]
        out.append(D)
    return np.stack(out).astype(np.int32)


@pytest.mark.parametrize("fmt,M,N,K", CASES)
def test_small_m_mfma_dots_equal_oracle(fmt, M, N, K):
    import block_quantized_gemv_w4a8_amd as qg
    g = np.random.default_rng(M * 13 + N + K)
    w = WEIGHTS[fmt](g, N, K)
    x, _ = synth.activation(g, M, K)
    act = quantize(qg, x)
    qh, dh, sh = act_host(*act)
    ref = _expected(fmt, w, N, K, qh, sh, M)
    wd = dev(w)
    variants = [qg.QGEMV_VARIANT_MFMA, qg.QGEMV_VARIANT_MFMA_STAGED]
    if fmt == "q4_k" and M <= 16:
        variants.append(qg.QGEMV_VARIANT_MFMA_RESIDENT)
    ran = 0
    for v in variants:
        say("small_m dots", fmt, M, N, K, "variant", v)
        dots = torch.full(ref.shape, -(2**31), dtype=torch.int32, device="cuda:0")
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
        try:
            qg.qgemm_small_m_block_dots(FMT[fmt], wd, N, K, M, *act, y, v, dots)
        except qg.QgemvError as e:
            # only the wave-stream kernel (Q6_K from M = 17 under MFMA) has
            # no dots mode
            assert e.status == qg.QGEMV_E_UNSUPPORTED and fmt == "q6_k" and M > 16, e
            assert v == qg.QGEMV_VARIANT_MFMA
            continue
        got = host(dots)
        bad = np.argwhere(got != ref)
        assert bad.size == 0, (fmt, M, N, K, v, bad[:5], got[tuple(bad[0])], ref[tuple(bad[0])])
        y_prod = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda:0")
        qg.SMALL_M[fmt](wd, N, K, M, *act, y_prod, v)
        assert np.array_equal(host(y).view(np.uint32), host(y_prod).view(np.uint32)), v
        ran += 1
    assert ran >= 1
