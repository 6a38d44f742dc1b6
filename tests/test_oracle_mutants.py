"""Planted mistakes in the oracle must each fail at least one pin.

Every case below copies ``oracle/qgemv_oracle.c`` into a temporary directory,
applies one textual mutation (a dropped term, a wrong sign, index or offset, a
different rounding rule), compiles it on the CPU and runs the pins against the
mutant.  A mutant that passes every pin would mean the pins cannot tell that
mistake from the definition.
"""
import os
import shutil

import pytest

import oracle
import pins

MUTANTS = {
    "q4k_drop_min_term": ("y += t1 - t2;", "y += t1;"),
    "q4k_min_sign": ("y += t1 - t2;", "y += t1 + t2;"),
    "q4k_T_net": ("T += fabs(t1) + fabs(t2);", "T += fabs(t1 - t2);"),
    "q4_0_offset": ("((int32_t)codes[i] - 8)", "((int32_t)codes[i] - 7)"),
    "q6k_no_offset": ("((int32_t)codes[16 * g + i] - 32)", "((int32_t)codes[16 * g + i])"),
    "q6k_act_block": ("int64_t b = 8 * S + g / 2;", "int64_t b = 8 * S + (g % 8);"),
    "q4k_scale_hi_bits": ("((b[j - 4] >> 6) << 4)", "((b[j] >> 6) << 4)"),
    "q4k_min_lo_bits": ("mn[j] = b[j + 4] & 63;", "mn[j] = b[j] & 63;"),
    "q4k_nibble_swap": ("codes[64 * c + l] = qs[32 * c + l] & 0x0f;",
                        "codes[64 * c + l] = qs[32 * c + l] >> 4;"),
    "q6k_qh_bits": ("(((H[l] >> 2) & 3) << 4)", "(((H[l] >> 4) & 3) << 4)"),
    "q6k_scale_unsigned": ("sc[i] = (int8_t)sb[192 + i];", "sc[i] = (int8_t)(sb[192 + i] & 0x7f);"),
    "q6k_d_offset": ("*d = rd16(sb + 208);", "*d = rd16(sb + 192);"),
    "quant_round_half_even": ("roundf(x[i] / d32)", "rintf(x[i] / d32)"),
    "quant_reciprocal": ("roundf(x[i] / d32)", "roundf(x[i] * (1.0f / d32))"),
    "quant_fp16_divisor": ("roundf(x[i] / d32)",
                           "roundf(x[i] / (float)orc_fp16_to_f64(orc_f32_to_fp16(d32)))"),
    "quant_signed_amax": ("float a = fabsf(x[i]);", "float a = x[i];"),
    "quant_d_251": ("float d32 = amax / 127.0f;", "float d32 = amax / 128.0f;"),
    "fp16_truncate": ("double n = nearbyint(ldexp(a, 10 - e));",
                      "double n = floor(ldexp(a, 10 - e));"),
    "fp16_subnormal_scale": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "gemm_row_stride": ("orc_gemv(fmt, w, N, K, row0, nrows, q + m * Kp,",
                        "orc_gemv(fmt, w, N, K, row0, nrows, q + m * K,"),
    "silu_sign": ("h[i] = g / (1.0 + exp(-g)) * u;", "h[i] = g / (1.0 + exp(g)) * u;"),
    "q8_0_block_bytes": ("int64_t bb = (fmt == ORC_Q4_0) ? 18 : 34;",
                         "int64_t bb = (fmt == ORC_Q4_0) ? 18 : 32;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src_dir = os.path.dirname(oracle._SRC)
    text = open(oracle._SRC).read()
    assert text.count(old) == 1, f"mutation site not unique/present: {old!r}"
    shutil.copy(os.path.join(src_dir, "qgemv_oracle.h"), tmp_path / "qgemv_oracle.h")
    mut_src = tmp_path / "qgemv_oracle.c"
    mut_src.write_text(text.replace(old, new))
    out = str(tmp_path / "libmutant.so")
    import subprocess
    subprocess.run(["gcc", *oracle.CFLAGS, "-w", "-o", out, str(mut_src), "-lm"], check=True)
    lib = oracle._load(out)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
            break
    assert failed, f"mutant {name} passed every pin"
