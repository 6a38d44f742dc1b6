"""Host-side checks of the C-ABI library: it loads, exports every symbol the
header declares, and each argument gate returns its own status before any
device work (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")


def _lib():
    import block_quantized_gemv_w4a8_amd as qg
    return qg


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(qgemv_\w+|qgemm_\w+)\s*\(", text)))


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0


def test_header_declarations_match_binding():
    qg = _lib()
    assert _declared() == sorted(qg.EXPORTS)


def test_library_exports_every_declared_symbol():
    qg = _lib()
    lib = ctypes.CDLL(qg.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", qg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, re.M))
    assert set(_declared()) <= exported


def test_version_and_strings():
    qg = _lib()
    assert qg.qgemv_abi_version() == 1
    for code in range(0, 8):
        s = qg.qgemv_status_str(code)
        assert s.startswith("QGEMV_")
    assert qg.qgemv_status_str(-5).startswith("QGEMV_E_UNKNOWN")
    info = qg.qgemv_build_info()
    assert "gfx950" in info and "q6_k" in info


def test_time_next_launch_arms_and_disarms_without_a_device():
    # only a thread-local pair is stored: no HIP call, so no device needed
    qg = _lib()
    assert qg.qgemv_time_next_launch(0x1000, 0x2000) == 0
    assert qg.qgemv_time_next_launch(None, None) == 0


# Fake device addresses: only ever passed where an earlier gate must refuse.
A = 0x7F0000000000  # 256-byte aligned


def _status(fn, *args):
    qg = _lib()
    return getattr(qg._lib, fn)(*args)


def test_gates_null_shape_limits_align():
    qg = _lib()
    S = 0  # stream
    # NULL pointers
    assert _status("qgemv_q4_k", None, 10, 256, A, A, A, A, S) == qg.QGEMV_E_NULL
    assert _status("qgemv_q6_k", A, 10, 256, A, A, A, None, S) == qg.QGEMV_E_NULL
    assert "NULL" in qg.qgemv_last_error()
    assert _status("qgemv_quantize_act", None, 1, 32, 32, A, A, A, S) == qg.QGEMV_E_NULL
    assert _status("qgemv_silu_mul_quantize", A, 64, None, A, A, None, S) == qg.QGEMV_E_NULL
    assert _status("qgemv_block_dots", 1, A, 4, 256, 0, 4, A, None, S) == qg.QGEMV_E_NULL
    SW = "qgemv_q4_k_swiglu_quantize"   # w, N, K, q, d, s, q_out, d_out, s_out, gu, h, stream
    assert _status(SW, A, 64, 256, A, A, A, None, A, A, None, None, S) == qg.QGEMV_E_NULL
    assert _status(SW, None, 64, 256, A, A, A, A, A, A, None, None, S) == qg.QGEMV_E_NULL
    # shapes
    for K in (0, 16, 48, -32):
        assert _status("qgemv_q4_0", A, 10, K, A, A, A, A, S) == qg.QGEMV_E_SHAPE
    assert _status("qgemv_q4_k", A, -1, 256, A, A, A, A, S) == qg.QGEMV_E_SHAPE
    assert _status("qgemv_quantize_act", A, 2, 64, 32, A, A, A, S) == qg.QGEMV_E_SHAPE  # ldx < K
    assert _status("qgemv_silu_mul_quantize", A, 48, A, A, A, None, S) == qg.QGEMV_E_SHAPE
    assert _status("qgemv_block_dots", 1, A, 4, 256, 3, 2, A, A, S) == qg.QGEMV_E_SHAPE
    assert _status("qgemm_q4_k_small_m", A, 8, 256, -1, A, A, A, A, 1, S) == qg.QGEMV_E_SHAPE
    assert _status(SW, A, 48, 256, A, A, A, A, A, A, None, None, S) == qg.QGEMV_E_SHAPE
    assert _status(SW, A, 64, 48, A, A, A, A, A, A, None, None, S) == qg.QGEMV_E_SHAPE
    assert _status(SW, A, 1 << 30, 256, A, A, A, A, A, A, None, None, S) == qg.QGEMV_E_SHAPE
    # empty problems succeed without touching anything (NULLs allowed)
    assert _status("qgemv_q4_k", None, 0, 256, None, None, None, None, S) == qg.QGEMV_OK
    assert _status("qgemv_quantize_act", None, 0, 256, 256, None, None, None, S) == qg.QGEMV_OK
    assert _status("qgemm_q4_k_small_m", None, 5, 256, 0, None, None, None, None, 0, S) == qg.QGEMV_OK
    assert _status("qgemv_block_dots", 2, None, 4, 256, 4, 0, None, None, S) == qg.QGEMV_OK
    assert _status(SW, None, 0, 256, None, None, None, None, None, None, None, None, S) == qg.QGEMV_OK
    # limits of this library
    assert _status("qgemv_q6_k", A, 10, 65536, A, A, A, A, S) == qg.QGEMV_E_UNSUPPORTED
    assert _status("qgemm_q4_k_small_m", A, 8, 256, 65, A, A, A, A, 1, S) == qg.QGEMV_E_UNSUPPORTED
    assert _status("qgemm_q4_k_small_m", A, 8, 256, 4, A, A, A, A, 9, S) == qg.QGEMV_E_UNSUPPORTED
    assert _status("qgemv_q6_k_repack", A, 4, 256, None, S) == qg.QGEMV_E_NULL
    assert _status("qgemv_q6_k_repack", A, 4, 48, A, S) == qg.QGEMV_E_SHAPE
    assert _status("qgemv_q6_k_repack", A, 4, 65536, A, S) == qg.QGEMV_E_UNSUPPORTED
    assert _status("qgemv_q6_k_repack", A, 4, 256, A + 2, S) == qg.QGEMV_E_ALIGN
    assert _status("qgemv_q6_k_repack", None, 0, 256, None, S) == qg.QGEMV_OK
    assert _status("qgemv_q6_k_r8", A, 10, 256, A, A, A, None, S) == qg.QGEMV_E_NULL
    assert _status("qgemv_q6_k_r8", A + 8, 10, 256, A, A, A, A, S) == qg.QGEMV_E_ALIGN
    assert _status("qgemv_block_dots", 4, A, 4, 256, 0, 4, A, None, S) == qg.QGEMV_E_NULL
    assert _status("qgemv_block_dots", 5, A, 4, 256, 0, 4, A, A, S) == qg.QGEMV_E_UNSUPPORTED
    for fn in ("qgemm_q6_k_small_m", "qgemm_q4_0_small_m"):
        assert _status(fn, A, 8, 256, 65, A, A, A, A, 1, S) == qg.QGEMV_E_UNSUPPORTED
        assert _status(fn, A, 8, 256, 4, A, A, A, A, 7, S) == qg.QGEMV_E_UNSUPPORTED
        assert _status(fn, A, 8, 256, 4, A, None, A, A, 1, S) == qg.QGEMV_E_NULL
        assert _status(fn, A, 8, 48, 4, A, A, A, A, 1, S) == qg.QGEMV_E_SHAPE
        assert _status(fn, A + 2, 8, 256, 4, A, A, A, A, 1, S) == qg.QGEMV_E_ALIGN
        assert _status(fn, None, 8, 256, 0, None, None, None, None, 0, S) == qg.QGEMV_OK
    assert _status("qgemv_block_dots", 7, A, 4, 256, 0, 4, A, A, S) == qg.QGEMV_E_UNSUPPORTED
    assert _status(SW, A, 64, 65536, A, A, A, A, A, A, None, None, S) == qg.QGEMV_E_UNSUPPORTED
    # alignment
    assert _status("qgemv_q4_k", A + 8, 10, 256, A, A, A, A, S) == qg.QGEMV_E_ALIGN
    assert _status("qgemv_q4_k", A, 10, 256, A + 4, A, A, A, S) == qg.QGEMV_E_ALIGN
    assert _status("qgemv_q4_k", A, 10, 256, A, A + 1, A, A, S) == qg.QGEMV_E_ALIGN
    assert _status("qgemv_q4_k", A, 10, 256, A, A, A + 2, A, S) == qg.QGEMV_E_ALIGN
    assert _status("qgemv_q4_k", A, 10, 256, A, A, A, A + 2, S) == qg.QGEMV_E_ALIGN
    assert _status("qgemv_quantize_act", A + 2, 1, 32, 32, A, A, A, S) == qg.QGEMV_E_ALIGN
    assert _status("qgemv_silu_mul_quantize", A, 64, A, A, A, A + 1, S) == qg.QGEMV_E_ALIGN
    assert _status(SW, A + 8, 64, 256, A, A, A, A, A, A, None, None, S) == qg.QGEMV_E_ALIGN
    assert _status(SW, A, 64, 256, A, A, A, A + 4, A, A, None, None, S) == qg.QGEMV_E_ALIGN
    assert _status(SW, A, 64, 256, A, A, A, A, A + 1, A, None, None, S) == qg.QGEMV_E_ALIGN
    assert _status(SW, A, 64, 256, A, A, A, A, A, A + 2, None, None, S) == qg.QGEMV_E_ALIGN
    assert _status(SW, A, 64, 256, A, A, A, A, A, A, A + 2, None, S) == qg.QGEMV_E_ALIGN
    assert _status(SW, A, 64, 256, A, A, A, A, A, A, None, A + 1, S) == qg.QGEMV_E_ALIGN
    assert "aligned" in qg.qgemv_last_error()


def test_gates_quantize_fused_entries():
    """qgemv_quantize_gemv and qgemv_quantize_q4_k_swiglu: NULL, shape, limit,
    format and alignment gates (x must be 16-byte aligned), and empty calls."""
    qg = _lib()
    S = 0
    QG = "qgemv_quantize_gemv"          # fmt, w, N, K, x, q, d, s, y, stream
    for fmt in range(5):
        assert _status(QG, fmt, A, 10, 256, None, A, A, A, A, S) == qg.QGEMV_E_NULL
        assert _status(QG, fmt, A, 10, 256, A, A, A, A, None, S) == qg.QGEMV_E_NULL
        assert _status(QG, fmt, A, 10, 48, A, A, A, A, A, S) == qg.QGEMV_E_SHAPE
        assert _status(QG, fmt, A, 10, 65536, A, A, A, A, A, S) == qg.QGEMV_E_UNSUPPORTED
        assert _status(QG, fmt, A, 10, 256, A + 4, A, A, A, A, S) == qg.QGEMV_E_ALIGN
        assert _status(QG, fmt, A, 10, 256, A, A + 4, A, A, A, S) == qg.QGEMV_E_ALIGN
        assert _status(QG, fmt, A, 10, 256, A, A, A, A, A + 2, S) == qg.QGEMV_E_ALIGN
        assert _status(QG, fmt, None, 0, 256, None, None, None, None, None, S) == qg.QGEMV_OK
    assert _status(QG, 5, A, 10, 256, A, A, A, A, A, S) == qg.QGEMV_E_UNSUPPORTED
    assert _status(QG, -1, A, 10, 256, A, A, A, A, A, S) == qg.QGEMV_E_UNSUPPORTED
    assert _status(QG, 1, A, -1, 256, A, A, A, A, A, S) == qg.QGEMV_E_SHAPE
    XS = "qgemv_quantize_q4_k_swiglu"   # w, N, K, x, q, d, s, q_out, d_out, s_out, gu, h, stream
    assert _status(XS, A, 64, 256, None, A, A, A, A, A, A, None, None, S) == qg.QGEMV_E_NULL
    assert _status(XS, A, 64, 256, A, None, A, A, A, A, A, None, None, S) == qg.QGEMV_E_NULL
    assert _status(XS, A, 64, 256, A, A, A, A, None, A, A, None, None, S) == qg.QGEMV_E_NULL
    assert _status(XS, A, 48, 256, A, A, A, A, A, A, A, None, None, S) == qg.QGEMV_E_SHAPE
    assert _status(XS, A, 64, 48, A, A, A, A, A, A, A, None, None, S) == qg.QGEMV_E_SHAPE
    assert _status(XS, A, 64, 65536, A, A, A, A, A, A, A, None, None, S) == qg.QGEMV_E_UNSUPPORTED
    assert _status(XS, A, 64, 256, A + 8, A, A, A, A, A, A, None, None, S) == qg.QGEMV_E_ALIGN
    assert _status(XS, A, 64, 256, A, A + 4, A, A, A, A, A, None, None, S) == qg.QGEMV_E_ALIGN
    assert _status(XS, A, 64, 256, A, A, A, A, A, A, A, A + 2, None, S) == qg.QGEMV_E_ALIGN
    assert _status(XS, None, 0, 256, None, None, None, None, None, None, None, None, None,
                   S) == qg.QGEMV_OK


def test_gates_multi_entries():
    """qgemv_multi / qgemv_quantize_multi: count, NULL arrays and members,
    negative rows, format, limits and alignment, before any device work."""
    import ctypes
    qg = _lib()
    S = 0
    P = ctypes.c_void_p
    def arrays(ws, ns, ys):
        c = len(ws)
        return (c, (P * max(c, 1))(*ws), (ctypes.c_int64 * max(c, 1))(*ns), (P * max(c, 1))(*ys))
    c, w, n, y = arrays([A, A], [10, 20], [A, A])
    M = "qgemv_multi"          # fmt, count, w, n, K, q, d, s, y, stream
    assert _status(M, 1, c, w, n, 256, A, A, A, y, S) != qg.QGEMV_E_NULL
    assert _status(M, 1, -1, w, n, 256, A, A, A, y, S) == qg.QGEMV_E_SHAPE
    assert _status(M, 1, 0, None, None, 256, None, None, None, None, S) == qg.QGEMV_OK
    assert _status(M, 1, c, None, n, 256, A, A, A, y, S) == qg.QGEMV_E_NULL
    assert _status(M, 1, c, w, n, 256, None, A, A, y, S) == qg.QGEMV_E_NULL
    c2, w2, n2, y2 = arrays([A, None], [10, 20], [A, A])
    assert _status(M, 1, c2, w2, n2, 256, A, A, A, y2, S) == qg.QGEMV_E_NULL
    c3, w3, n3, y3 = arrays([A, None], [10, 0], [A, None])       # empty member: no pointers needed
    assert _status(M, 1, c3, w3, n3, 48, A, A, A, y3, S) == qg.QGEMV_E_SHAPE
    c4, w4, n4, y4 = arrays([A, A], [10, -2], [A, A])
    assert _status(M, 1, c4, w4, n4, 256, A, A, A, y4, S) == qg.QGEMV_E_SHAPE
    c5, w5, n5, y5 = arrays([A] * 9, [1] * 9, [A] * 9)
    assert _status(M, 1, c5, w5, n5, 256, A, A, A, y5, S) == qg.QGEMV_E_UNSUPPORTED
    assert _status(M, 9, c, w, n, 256, A, A, A, y, S) == qg.QGEMV_E_UNSUPPORTED
    assert _status(M, 1, c, w, n, 65536, A, A, A, y, S) == qg.QGEMV_E_UNSUPPORTED
    c6, w6, n6, y6 = arrays([A, A + 8], [10, 20], [A, A])
    assert _status(M, 1, c6, w6, n6, 256, A, A, A, y6, S) == qg.QGEMV_E_ALIGN
    c7, w7, n7, y7 = arrays([A, A], [10, 20], [A, A + 2])
    assert _status(M, 1, c7, w7, n7, 256, A, A, A, y7, S) == qg.QGEMV_E_ALIGN
    assert _status(M, 1, c, w, n, 256, A + 4, A, A, y, S) == qg.QGEMV_E_ALIGN
    XM = "qgemv_quantize_multi"   # fmt, count, w, n, K, x, q, d, s, y, stream
    assert _status(XM, 1, c, w, n, 256, None, A, A, A, y, S) == qg.QGEMV_E_NULL
    assert _status(XM, 1, c, w, n, 256, A + 4, A, A, A, y, S) == qg.QGEMV_E_ALIGN
    assert _status(XM, 1, 0, None, None, 256, None, None, None, None, None, S) == qg.QGEMV_OK


def test_gate_order_null_before_shape_before_align():
    qg = _lib()
    # a NULL pointer wins over a bad K and a misaligned pointer
    assert _status("qgemv_q4_k", None, 10, 48, A + 1, A, A, A, 0) == qg.QGEMV_E_NULL
    # a bad K wins over a misaligned pointer
    assert _status("qgemv_q4_k", A + 1, 10, 48, A, A, A, A, 0) == qg.QGEMV_E_SHAPE
    # the limits gate wins over alignment
    assert _status("qgemv_q4_k", A + 1, 10, 65536, A, A, A, A, 0) == qg.QGEMV_E_UNSUPPORTED


@pytest.mark.skipif(not _no_gpu(), reason="device gate refusal is only observable without a GPU")
def test_device_gate_without_gpu():
    qg = _lib()
    st = _status("qgemv_q4_k", A, 10, 256, A, A, A, A, 0)
    assert st == qg.QGEMV_E_DEVICE
    assert qg.qgemv_last_error()
    with pytest.raises(qg.QgemvError):
        qg.qgemv_q6_k(A, 10, 256, A, A, A, A, stream=0)


def test_gates_stream_read():
    """The streaming-read measurement aid: NULL, size, limit and alignment
    gates, before any device work."""
    qg = _lib()
    R = "qgemv_stream_read"   # buf, bytes, nontemporal, sink, wg_per_cu, stream
    assert _status(R, None, 1 << 20, 1, A, 4, 0) == qg.QGEMV_E_NULL
    assert _status(R, A, 1 << 20, 1, None, 4, 0) == qg.QGEMV_E_NULL
    assert _status(R, A, 0, 1, A, 4, 0) == qg.QGEMV_E_SHAPE
    assert _status(R, A, 24, 1, A, 4, 0) == qg.QGEMV_E_SHAPE
    assert _status(R, A, 1 << 20, 1, A, 0, 0) == qg.QGEMV_E_UNSUPPORTED
    assert _status(R, A, 1 << 20, 1, A, 33, 0) == qg.QGEMV_E_UNSUPPORTED
    assert _status(R, A + 8, 1 << 20, 1, A, 4, 0) == qg.QGEMV_E_ALIGN
    assert _status(R, A, 1 << 20, 1, A + 2, 4, 0) == qg.QGEMV_E_ALIGN


def test_gates_block_dots_staged():
    """The staged block-dots validation entry: NULL, shape, limits (split-K
    width, slice length) and alignment, before any device work."""
    qg = _lib()
    B = "qgemv_block_dots_staged"   # fmt, w, N, K, row0, nrows, q, d, s, wk, dots, stream
    Q4K, R8 = qg.QGEMV_FMT_Q4_K, qg.QGEMV_FMT_Q6_K_R8
    assert _status(B, Q4K, None, 4, 256, 0, 0, None, None, None, 1, None, 0) == qg.QGEMV_OK
    assert _status(B, Q4K, A, 4, 256, 3, 2, A, A, A, 1, A, 0) == qg.QGEMV_E_SHAPE
    assert _status(B, Q4K, A, 4, 256, 0, 4, A, None, A, 1, A, 0) == qg.QGEMV_E_NULL
    assert _status(B, Q4K, A, 4, 256, 0, 4, A, A, None, 1, A, 0) == qg.QGEMV_E_NULL
    assert _status(B, Q4K, A, 4, 48, 0, 4, A, A, A, 1, A, 0) == qg.QGEMV_E_SHAPE
    assert _status(B, 9, A, 4, 256, 0, 4, A, A, A, 1, A, 0) == qg.QGEMV_E_UNSUPPORTED
    assert _status(B, Q4K, A, 4, 256, 0, 4, A, A, A, 3, A, 0) == qg.QGEMV_E_UNSUPPORTED
    # 224 units in one slice: more than 128
    assert _status(B, R8, A, 4, 14336, 0, 4, A, A, A, 1, A, 0) == qg.QGEMV_E_UNSUPPORTED
    assert "split-K width" in qg.qgemv_last_error()
    assert _status(B, Q4K, A + 8, 4, 256, 0, 4, A, A, A, 1, A, 0) == qg.QGEMV_E_ALIGN
    assert _status(B, Q4K, A, 4, 256, 0, 4, A + 4, A, A, 1, A, 0) == qg.QGEMV_E_ALIGN
    assert _status(B, Q4K, A, 4, 256, 0, 4, A, A, A, 1, A + 2, 0) == qg.QGEMV_E_ALIGN
    if _no_gpu():
        assert _status(B, R8, A, 4, 14336, 0, 4, A, A, A, 4, A, 0) == qg.QGEMV_E_DEVICE


def test_gates_small_m_block_dots():
    qg = _lib()
    B = "qgemm_small_m_block_dots"   # fmt, w, N, K, M, q, d, s, y, variant, dots, stream
    Q4K, Q6K, MF = qg.QGEMV_FMT_Q4_K, qg.QGEMV_FMT_Q6_K, qg.QGEMV_VARIANT_MFMA
    assert _status(B, Q4K, None, 0, 256, 4, None, None, None, None, MF, None, 0) == qg.QGEMV_OK
    assert _status(B, Q4K, A, -1, 256, 4, A, A, A, A, MF, A, 0) == qg.QGEMV_E_SHAPE
    assert _status(B, Q4K, A, 8, 256, 4, A, A, A, A, MF, None, 0) == qg.QGEMV_E_NULL
    assert _status(B, Q4K, A, 8, 48, 4, A, A, A, A, MF, A, 0) == qg.QGEMV_E_SHAPE
    assert _status(B, qg.QGEMV_FMT_Q8_0, A, 8, 256, 4, A, A, A, A, MF, A, 0) == qg.QGEMV_E_UNSUPPORTED
    assert _status(B, Q4K, A, 8, 256, 65, A, A, A, A, MF, A, 0) == qg.QGEMV_E_UNSUPPORTED
    assert _status(B, Q4K, A, 8, 256, 4, A, A, A, A, qg.QGEMV_VARIANT_DOT4, A, 0) == qg.QGEMV_E_UNSUPPORTED
    assert _status(B, Q4K, A, 8, 256, 4, A, A, A, A, qg.QGEMV_VARIANT_MFMA_STREAM, A, 0) == qg.QGEMV_E_UNSUPPORTED
    # Q6_K at M = 64 under MFMA takes the wave-stream kernel: no dots mode
    assert _status(B, Q6K, A, 4096, 14336, 64, A, A, A, A, MF, A, 0) == qg.QGEMV_E_UNSUPPORTED
    assert _status(B, Q4K, A + 8, 8, 256, 4, A, A, A, A, MF, A, 0) == qg.QGEMV_E_ALIGN
    assert _status(B, Q4K, A, 8, 256, 4, A, A, A, A, MF, A + 2, 0) == qg.QGEMV_E_ALIGN
    if _no_gpu():
        assert _status(B, Q6K, A, 4096, 14336, 64, A, A, A, A, qg.QGEMV_VARIANT_MFMA_STAGED, A, 0) \
            == qg.QGEMV_E_DEVICE
