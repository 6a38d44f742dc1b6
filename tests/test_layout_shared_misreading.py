"""A misreading of a block layout made the same way in the packer (synth) and
in the oracle's unpacker is invisible to the pack/unpack round trip.  For each
such shared misreading below, the oracle is rebuilt with it, synth's packer is
replaced by one with the same misreading, and then:
  * the round-trip pin still passes (it cannot tell), and
  * the literal-block pin fails (its expected fields are written out from the
    layout descriptions, not produced by either side).
The layouts are the GGUF ones ("llambda.lisp" README, Features &
Architecture: Q4_K_M and Q6_K tensors read straight from .gguf files)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import pins
import synth


def _u16(v):
    return np.ascontiguousarray(v, dtype=np.uint16).view(np.uint8).reshape(v.shape + (2,))


def pack_q6_k_qh_swapped(d, sc, codes):
    """Q6_K with the high bits of quadrants 1 and 2 in each other's qh bits."""
    N, S = d.shape
    c = codes.reshape(N, S, 2, 4, 32).astype(np.uint8)
    out = np.empty((N, S, 210), dtype=np.uint8)
    ql = np.empty((N, S, 2, 2, 32), np.uint8)
    ql[:, :, :, 0, :] = (c[:, :, :, 0, :] & 15) | ((c[:, :, :, 2, :] & 15) << 4)
    ql[:, :, :, 1, :] = (c[:, :, :, 1, :] & 15) | ((c[:, :, :, 3, :] & 15) << 4)
    out[:, :, 0:128] = ql.reshape(N, S, 128)
    qh = ((c[:, :, :, 0, :] >> 4) | ((c[:, :, :, 2, :] >> 4) << 2) |
          ((c[:, :, :, 1, :] >> 4) << 4) | ((c[:, :, :, 3, :] >> 4) << 6))
    out[:, :, 128:192] = qh.reshape(N, S, 64)
    out[:, :, 192:208] = np.asarray(sc, dtype=np.int8).view(np.uint8)
    out[:, :, 208:210] = _u16(d)
    return out.reshape(N, S * 210)


def _pack_q4_k(d, dmin, sc, mn, codes, hi_swap=False, nib_swap=False):
    N, S = d.shape
    sc = sc.astype(np.uint8) & 63
    mn = mn.astype(np.uint8) & 63
    out = np.empty((N, S, 144), dtype=np.uint8)
    out[:, :, 0:2] = _u16(d)
    out[:, :, 2:4] = _u16(dmin)
    hs, hm = ((mn, sc) if hi_swap else (sc, mn))
    out[:, :, 4:8] = sc[:, :, 0:4] | ((hs[:, :, 4:8] >> 4) << 6)
    out[:, :, 8:12] = mn[:, :, 0:4] | ((hm[:, :, 4:8] >> 4) << 6)
    out[:, :, 12:16] = (sc[:, :, 4:8] & 15) | ((mn[:, :, 4:8] & 15) << 4)
    c = codes.reshape(N, S, 4, 2, 32).astype(np.uint8)
    lo, hi = (c[:, :, :, 1, :], c[:, :, :, 0, :]) if nib_swap else (c[:, :, :, 0, :],
                                                                   c[:, :, :, 1, :])
    out[:, :, 16:144] = ((lo & 15) | ((hi & 15) << 4)).reshape(N, S, 128)
    return out.reshape(N, S * 144)


# name: (oracle source replacements applied in order, synth attribute, packer)
SHARED = {
    "q6k_qh_quadrants_1_2": (
        [("(((H[l] >> 2) & 3) << 4)", "@@A@@"), ("(((H[l] >> 4) & 3) << 4)", "(((H[l] >> 2) & 3) << 4)"),
         ("@@A@@", "(((H[l] >> 4) & 3) << 4)")],
        "pack_q6_k", pack_q6_k_qh_swapped),
    "q4k_high_bits_scale_min_swapped": (
        [("((b[j - 4] >> 6) << 4)", "@@A@@"), ("((b[j] >> 6) << 4)", "((b[j - 4] >> 6) << 4)"),
         ("@@A@@", "((b[j] >> 6) << 4)")],
        "pack_q4_k", lambda *a: _pack_q4_k(*a, hi_swap=True)),
    "q4k_nibble_halves_swapped": (
        [("codes[64 * c + l] = qs[32 * c + l] & 0x0f;", "codes[64 * c + l] = qs[32 * c + l] >> 4;"),
         ("codes[64 * c + 32 + l] = qs[32 * c + l] >> 4;",
          "codes[64 * c + 32 + l] = qs[32 * c + l] & 0x0f;")],
        "pack_q4_k", lambda *a: _pack_q4_k(*a, nib_swap=True)),
}


@pytest.mark.parametrize("name", sorted(SHARED))
def test_shared_misreading_needs_the_literal_pin(name, tmp_path, monkeypatch):
    repl, attr, packer = SHARED[name]
    src_dir = os.path.dirname(oracle._SRC)
    text = open(oracle._SRC).read()
    for old, new in repl:
        assert text.count(old) == 1, f"mutation site not unique/present: {old!r}"
        text = text.replace(old, new)
    shutil.copy(os.path.join(src_dir, "qgemv_oracle.h"), tmp_path / "qgemv_oracle.h")
    (tmp_path / "qgemv_oracle.c").write_text(text)
    out = str(tmp_path / "libshared.so")
    subprocess.run(["gcc", *oracle.CFLAGS, "-w", "-o", out, str(tmp_path / "qgemv_oracle.c"),
                    "-lm"], check=True)
    lib = oracle._load(out)
    monkeypatch.setattr(synth, attr, packer)
    pins.pin_unpack_roundtrip(lib)          # blind to the shared misreading
    with pytest.raises(AssertionError):
        pins.pin_layout_literal_blocks(lib)
