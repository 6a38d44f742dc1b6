"""Python binding of libqgemv (W4A8 block-quantized GEMV for AMD MI355X / gfx950).

Argument marshalling only: every function here has the name of a C-ABI entry
point in ``include/qgemv.h``, takes torch device tensors (or raw integer
device addresses) for its pointer arguments, passes them with the current
torch stream (unless ``stream`` is given) to the library, and raises
:class:`QgemvError` when the library returns a non-OK status.  All arithmetic
happens in the library's HIP kernels.  Importing this package fails loudly if
the library has not been built (``python -m block_quantized_gemv_w4a8_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libqgemv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libqgemv.so is not built ({LIB_PATH}); run "
        "`python -m block_quantized_gemv_w4a8_amd.build` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

QGEMV_OK = 0
QGEMV_E_NULL = 1
QGEMV_E_SHAPE = 2
QGEMV_E_UNSUPPORTED = 3
QGEMV_E_ALIGN = 4
QGEMV_E_DEVICE = 5
QGEMV_E_LAUNCH = 6

QGEMV_FMT_Q4_0, QGEMV_FMT_Q4_K, QGEMV_FMT_Q6_K, QGEMV_FMT_Q8_0 = 0, 1, 2, 3
QGEMV_FMT_Q6_K_R8 = 4
QGEMV_VARIANT_AUTO, QGEMV_VARIANT_DOT4, QGEMV_VARIANT_MFMA = 0, 1, 2
QGEMV_VARIANT_MFMA_STAGED, QGEMV_VARIANT_MFMA_STREAM, QGEMV_VARIANT_MFMA_RESIDENT = 3, 4, 5
QGEMV_K_MAX = 32768
QGEMV_MULTI_MAX = 8
QGEMV_M_MAX = 64

# Every extern "C" symbol that include/qgemv.h declares.
EXPORTS = [
    "qgemv_abi_version", "qgemv_status_str", "qgemv_build_info", "qgemv_last_error",
    "qgemv_time_next_launch", "qgemv_stream_read",
    "qgemv_quantize_act", "qgemv_q4_0", "qgemv_q4_k", "qgemv_q6_k", "qgemv_q8_0",
    "qgemv_q6_k_repack", "qgemv_q6_k_r8",
    "qgemm_q4_k_small_m", "qgemm_q6_k_small_m", "qgemm_q4_0_small_m",
    "qgemv_silu_mul_quantize", "qgemv_q4_k_swiglu_quantize",
    "qgemv_quantize_gemv", "qgemv_quantize_q4_k_swiglu", "qgemv_multi", "qgemv_quantize_multi",
    "qgemv_block_dots", "qgemv_block_dots_staged", "qgemm_small_m_block_dots",
]

_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_lib.qgemv_abi_version.restype = _I
_lib.qgemv_abi_version.argtypes = []
_lib.qgemv_status_str.restype = ctypes.c_char_p
_lib.qgemv_status_str.argtypes = [_I]
_lib.qgemv_build_info.restype = ctypes.c_char_p
_lib.qgemv_build_info.argtypes = []
_lib.qgemv_last_error.restype = ctypes.c_char_p
_lib.qgemv_last_error.argtypes = []
_lib.qgemv_time_next_launch.argtypes = [_P, _P]
_lib.qgemv_quantize_act.restype = _I
_lib.qgemv_quantize_act.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P]
for _n in ("qgemv_q4_0", "qgemv_q4_k", "qgemv_q6_k", "qgemv_q8_0", "qgemv_q6_k_r8"):
    getattr(_lib, _n).restype = _I
    getattr(_lib, _n).argtypes = [_P, _I64, _I64, _P, _P, _P, _P, _P]
for _n in ("qgemm_q4_k_small_m", "qgemm_q6_k_small_m", "qgemm_q4_0_small_m"):
    getattr(_lib, _n).restype = _I
    getattr(_lib, _n).argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P, _I, _P]
_lib.qgemv_silu_mul_quantize.restype = _I
_lib.qgemv_silu_mul_quantize.argtypes = [_P, _I64, _P, _P, _P, _P, _P]
_lib.qgemv_q4_k_swiglu_quantize.restype = _I
_lib.qgemv_q4_k_swiglu_quantize.argtypes = [_P, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.qgemv_quantize_q4_k_swiglu.restype = _I
_lib.qgemv_quantize_q4_k_swiglu.argtypes = [_P, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                            _P]
_lib.qgemv_quantize_gemv.restype = _I
_lib.qgemv_quantize_gemv.argtypes = [_I, _P, _I64, _I64, _P, _P, _P, _P, _P, _P]
_lib.qgemv_multi.restype = _I
_lib.qgemv_multi.argtypes = [_I, _I, _P, _P, _I64, _P, _P, _P, _P, _P]
_lib.qgemv_quantize_multi.restype = _I
_lib.qgemv_quantize_multi.argtypes = [_I, _I, _P, _P, _I64, _P, _P, _P, _P, _P, _P]
_lib.qgemv_block_dots.restype = _I
_lib.qgemv_block_dots.argtypes = [_I, _P, _I64, _I64, _I64, _I64, _P, _P, _P]
_lib.qgemv_block_dots_staged.restype = _I
_lib.qgemv_block_dots_staged.argtypes = [_I, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _I, _P, _P]
_lib.qgemm_small_m_block_dots.restype = _I
_lib.qgemm_small_m_block_dots.argtypes = [_I, _P, _I64, _I64, _I64, _P, _P, _P, _P, _I, _P, _P]

if _lib.qgemv_abi_version() != 1:
    raise ImportError("libqgemv ABI generation mismatch (expected 1)")


class QgemvError(RuntimeError):
    def __init__(self, status: int, func: str):
        self.status = status
        reason = qgemv_last_error()
        super().__init__(f"{func}: {qgemv_status_str(status)} ({reason})")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


_current_raw_stream = None


def _stream(stream) -> int | None:
    """The hipStream_t of `stream`; None means torch's current stream, read
    through torch's raw-handle getter where it has one (it skips building a
    Stream object, a few microseconds per call)."""
    global _current_raw_stream
    if stream is None:
        if _current_raw_stream is None:
            import torch
            raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
            get_dev = getattr(torch._C, "_cuda_getDevice", None)
            if raw is not None and get_dev is not None:
                _current_raw_stream = lambda: raw(get_dev())
            else:
                _current_raw_stream = lambda: torch.cuda.current_stream().cuda_stream
        return _current_raw_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, func: str) -> int:
    if status != QGEMV_OK:
        raise QgemvError(status, func)
    return status


# ---------------------------------------------------------- C-ABI names ----

def qgemv_abi_version() -> int:
    return _lib.qgemv_abi_version()


def qgemv_status_str(status: int) -> str:
    return _lib.qgemv_status_str(status).decode()


def qgemv_build_info() -> str:
    return _lib.qgemv_build_info().decode()


def qgemv_last_error() -> str:
    return _lib.qgemv_last_error().decode()


def _handle(e):
    return e.value if isinstance(e, ctypes.c_void_p) else e


def qgemv_time_next_launch(start=None, stop=None):
    """start, stop: hipEvent_t handles (int or ctypes.c_void_p) or None."""
    return _check(_lib.qgemv_time_next_launch(_handle(start), _handle(stop)),
                  "qgemv_time_next_launch")


_lib.qgemv_stream_read.restype = _I
_lib.qgemv_stream_read.argtypes = [_P, _I64, _I, _P, _I, _P]


def qgemv_stream_read(buf, nbytes, nontemporal, sink, wg_per_cu=4, stream=None):
    """Measurement aid: one streaming read of nbytes of buf (see the header)."""
    return _check(_lib.qgemv_stream_read(_ptr(buf), nbytes, int(nontemporal), _ptr(sink),
                                         wg_per_cu, _stream(stream)), "qgemv_stream_read")


def qgemv_quantize_act(x, M, K, ldx, q, d, s, stream=None):
    return _check(_lib.qgemv_quantize_act(_ptr(x), M, K, ldx, _ptr(q), _ptr(d), _ptr(s),
                                          _stream(stream)), "qgemv_quantize_act")


def _gemv(name, w, N, K, q, d, s, y, stream):
    return _check(getattr(_lib, name)(_ptr(w), N, K, _ptr(q), _ptr(d), _ptr(s), _ptr(y),
                                      _stream(stream)), name)


def qgemv_q4_0(w, N, K, q, d, s, y, stream=None):
    return _gemv("qgemv_q4_0", w, N, K, q, d, s, y, stream)


def qgemv_q4_k(w, N, K, q, d, s, y, stream=None):
    return _gemv("qgemv_q4_k", w, N, K, q, d, s, y, stream)


def qgemv_q6_k(w, N, K, q, d, s, y, stream=None):
    return _gemv("qgemv_q6_k", w, N, K, q, d, s, y, stream)


def qgemv_q6_k_r8(w_r, N, K, q, d, s, y, stream=None):
    return _gemv("qgemv_q6_k_r8", w_r, N, K, q, d, s, y, stream)


_lib.qgemv_q6_k_repack.restype = _I
_lib.qgemv_q6_k_repack.argtypes = [_P, _I64, _I64, _P, _P]


def qgemv_q6_k_repack(w, N, K, w_r, stream=None):
    return _check(_lib.qgemv_q6_k_repack(_ptr(w), N, K, _ptr(w_r), _stream(stream)),
                  "qgemv_q6_k_repack")


def q6_k_r8_row_bytes(K: int) -> int:
    """Bytes of one row of Q6_K weights repacked by qgemv_q6_k_repack."""
    nsb = (K + 255) // 256
    return (nsb + 7) // 8 * 1680


def qgemv_q8_0(w, N, K, q, d, s, y, stream=None):
    return _gemv("qgemv_q8_0", w, N, K, q, d, s, y, stream)


def qgemm_q4_k_small_m(w, N, K, M, q, d, s, y, variant=QGEMV_VARIANT_AUTO, stream=None):
    return _check(_lib.qgemm_q4_k_small_m(_ptr(w), N, K, M, _ptr(q), _ptr(d), _ptr(s), _ptr(y),
                                          variant, _stream(stream)), "qgemm_q4_k_small_m")


def qgemm_q6_k_small_m(w, N, K, M, q, d, s, y, variant=QGEMV_VARIANT_AUTO, stream=None):
    return _check(_lib.qgemm_q6_k_small_m(_ptr(w), N, K, M, _ptr(q), _ptr(d), _ptr(s), _ptr(y),
                                          variant, _stream(stream)), "qgemm_q6_k_small_m")


def qgemm_q4_0_small_m(w, N, K, M, q, d, s, y, variant=QGEMV_VARIANT_AUTO, stream=None):
    return _check(_lib.qgemm_q4_0_small_m(_ptr(w), N, K, M, _ptr(q), _ptr(d), _ptr(s), _ptr(y),
                                          variant, _stream(stream)), "qgemm_q4_0_small_m")


SMALL_M = {"q4_k": qgemm_q4_k_small_m, "q6_k": qgemm_q6_k_small_m,
           "q4_0": qgemm_q4_0_small_m}


def qgemv_silu_mul_quantize(gu, N, q, d, s, h=None, stream=None):
    return _check(_lib.qgemv_silu_mul_quantize(_ptr(gu), N, _ptr(q), _ptr(d), _ptr(s), _ptr(h),
                                               _stream(stream)), "qgemv_silu_mul_quantize")


def qgemv_q4_k_swiglu_quantize(w, N, K, q, d, s, q_out, d_out, s_out, gu=None, h=None,
                               stream=None):
    return _check(_lib.qgemv_q4_k_swiglu_quantize(_ptr(w), N, K, _ptr(q), _ptr(d), _ptr(s),
                                                  _ptr(q_out), _ptr(d_out), _ptr(s_out), _ptr(gu),
                                                  _ptr(h), _stream(stream)),
                  "qgemv_q4_k_swiglu_quantize")


def qgemv_quantize_q4_k_swiglu(w, N, K, x, q, d, s, q_out, d_out, s_out, gu=None, h=None,
                               stream=None):
    return _check(_lib.qgemv_quantize_q4_k_swiglu(_ptr(w), N, K, _ptr(x), _ptr(q), _ptr(d),
                                                  _ptr(s), _ptr(q_out), _ptr(d_out), _ptr(s_out),
                                                  _ptr(gu), _ptr(h), _stream(stream)),
                  "qgemv_quantize_q4_k_swiglu")


def qgemv_quantize_gemv(fmt, w, N, K, x, q, d, s, y, stream=None):
    return _check(_lib.qgemv_quantize_gemv(fmt, _ptr(w), N, K, _ptr(x), _ptr(q), _ptr(d), _ptr(s),
                                           _ptr(y), _stream(stream)), "qgemv_quantize_gemv")


def _multi_arrays(ws, ns, ys):
    if not (len(ws) == len(ns) == len(ys)):
        raise ValueError("ws, ns and ys must have the same length")
    c = len(ws)
    wa = (ctypes.c_void_p * max(c, 1))(*[_ptr(t) for t in ws])
    na = (ctypes.c_int64 * max(c, 1))(*[int(v) for v in ns])
    ya = (ctypes.c_void_p * max(c, 1))(*[_ptr(t) for t in ys])
    return c, wa, na, ya


def qgemv_multi(fmt, ws, ns, K, q, d, s, ys, stream=None):
    """Several GEMVs (lists ws, ns, ys of one length) on one activation."""
    c, wa, na, ya = _multi_arrays(ws, ns, ys)
    return _check(_lib.qgemv_multi(fmt, c, wa, na, K, _ptr(q), _ptr(d), _ptr(s), ya,
                                   _stream(stream)), "qgemv_multi")


def qgemv_quantize_multi(fmt, ws, ns, K, x, q, d, s, ys, stream=None):
    c, wa, na, ya = _multi_arrays(ws, ns, ys)
    return _check(_lib.qgemv_quantize_multi(fmt, c, wa, na, K, _ptr(x), _ptr(q), _ptr(d),
                                            _ptr(s), ya, _stream(stream)),
                  "qgemv_quantize_multi")


def qgemv_block_dots(fmt, w, N, K, row0, nrows, q, dots, stream=None):
    return _check(_lib.qgemv_block_dots(fmt, _ptr(w), N, K, row0, nrows, _ptr(q), _ptr(dots),
                                        _stream(stream)), "qgemv_block_dots")


def qgemv_block_dots_staged(fmt, w, N, K, row0, nrows, q, d, s, wk, dots, stream=None):
    return _check(_lib.qgemv_block_dots_staged(fmt, _ptr(w), N, K, row0, nrows, _ptr(q), _ptr(d),
                                               _ptr(s), wk, _ptr(dots), _stream(stream)),
                  "qgemv_block_dots_staged")


def qgemm_small_m_block_dots(fmt, w, N, K, M, q, d, s, y, variant, dots, stream=None):
    return _check(_lib.qgemm_small_m_block_dots(fmt, _ptr(w), N, K, M, _ptr(q), _ptr(d), _ptr(s),
                                                _ptr(y), variant, _ptr(dots), _stream(stream)),
                  "qgemm_small_m_block_dots")


GEMV = {"q4_0": qgemv_q4_0, "q4_k": qgemv_q4_k, "q6_k": qgemv_q6_k, "q8_0": qgemv_q8_0,
        "q6_k_r8": qgemv_q6_k_r8}
FMT_ID = {"q4_0": QGEMV_FMT_Q4_0, "q4_k": QGEMV_FMT_Q4_K, "q6_k": QGEMV_FMT_Q6_K,
          "q8_0": QGEMV_FMT_Q8_0, "q6_k_r8": QGEMV_FMT_Q6_K_R8}


def act_buffers(M: int, K: int, device="cuda"):
    """Empty activation buffers (q, d, s) of the library's layout for M rows of K."""
    import torch
    Kp = (K + 255) // 256 * 256
    q = torch.empty((M, Kp), dtype=torch.int8, device=device)
    d = torch.empty((M, Kp // 32), dtype=torch.int16, device=device)
    s = torch.empty((M, Kp // 32), dtype=torch.int32, device=device)
    return q, d, s
