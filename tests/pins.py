"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` function takes a loaded oracle library (``lib``) and raises
AssertionError when the oracle disagrees with what the definitions and the
mathematics fix.  ``test_oracle_pins.py`` runs them against the real oracle;
``test_oracle_mutants.py`` runs them against deliberately broken copies of the
oracle and requires each copy to fail at least one pin.

Independent references used here (none calls the oracle's own arithmetic):
  * numpy's binary16 conversion (a library routine) for fp16 encode/decode;
  * a numpy float32 re-derivation of the activation rule (IEEE division in
    float32, then half-away rounding done exactly in float64);
  * integer brute force over the raw codes the generator drew (not unpacked
    from the packed bytes by the oracle);
  * float64 dequantise-then-dot with the per-format weight formulas
      Q4_0 w = d (code - 8)          Q8_0 w = d code
      Q4_K w = d sc_j code - dmin m_j Q6_K w = d sc (code - 32)
    against x_hat = f(dx) q;
  * closed forms: all-equal codes, zero scales, one-hot activations.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth


# ------------------------------------------------------------------ fp16 ---

def pin_fp16_decode_exhaustive(lib):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.fp16_to_f64(h, lib=lib)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _fp16_encode_cases(seed=0):
    g = np.random.default_rng(seed)
    # every finite fp16 value, the midpoints between neighbours, and the
    # float32 neighbours of each midpoint (the RNE decision points)
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2
    mids = np.concatenate([mids, [65520.0]])
    m32 = mids.astype(np.float32)
    near = np.concatenate([m32, np.nextafter(m32, np.float32(np.inf)),
                           np.nextafter(m32, np.float32(0)),
                           v.astype(np.float32)])
    rand = g.uniform(-70000, 70000, 200000).astype(np.float32)
    small = (g.uniform(-1, 1, 200000) * 2.0 ** g.integers(-30, -10, 200000)).astype(np.float32)
    bits = g.integers(0, 2**32, 200000, dtype=np.uint32).view(np.float32)
    bits = bits[np.isfinite(bits)]
    allv = np.concatenate([near, -near, rand, small, bits,
                           np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e30, -1e30],
                                    dtype=np.float32)])
    return allv.astype(np.float32)


def pin_fp16_encode_rne(lib):
    f = _fp16_encode_cases()
    got = oracle.f32_to_fp16(f, lib=lib)
    with np.errstate(over="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"fp16 encode mismatch at {f[bad[:5]]}: {got[bad[:5]]} vs {ref[bad[:5]]}"


# -------------------------------------------------------- quantisation -----

def ref_quantize(x: np.ndarray, K: int):
    """Independent numpy statement of the activation rule (float32 IEEE)."""
    x = np.asarray(x, dtype=np.float32)
    M = x.shape[0]
    Kp = oracle.kp(K)
    xp = np.zeros((M, Kp), dtype=np.float32)
    xp[:, :K] = x[:, :K]
    blk = xp.reshape(M, Kp // 32, 32)
    amax = np.max(np.abs(blk), axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        d32 = (amax / np.float32(127.0)).astype(np.float32)
        v = (blk / d32[:, :, None]).astype(np.float32)
    r = np.sign(v.astype(np.float64)) * np.floor(np.abs(v.astype(np.float64)) + 0.5)
    r = np.clip(r, -127, 127)
    zero = amax == 0
    r[zero] = 0
    q = r.astype(np.int8).reshape(M, Kp)
    d = d32.astype(np.float16).view(np.uint16)
    d[zero] = 0
    s = r.sum(axis=2).astype(np.int32)
    return q, d, s


def pin_quantize_random(lib):
    g = np.random.default_rng(11)
    for M, K, ldx in [(1, 32, 32), (2, 96, 100), (1, 896, 896), (3, 4096, 4096),
                      (1, 4864, 4864), (2, 1056, 1060)]:
        x = g.standard_normal((M, ldx)).astype(np.float32) * np.float32(g.uniform(0.01, 30))
        x[:, g.choice(ldx, size=max(1, ldx // 100), replace=False)] *= 20
        if K >= 64:
            x[:, 32:64] = 0.0  # an all-zero block
        q, d, s = oracle.quantize_act(x, K=K, lib=lib)
        rq, rd, rs = ref_quantize(x, K)
        assert np.array_equal(q, rq), "codes differ"
        assert np.array_equal(d, rd), "scales differ"
        assert np.array_equal(s, rs), "sums differ"
    # near-ties: x within an ulp of (k + 1/2) d for the block's own d, where a
    # reciprocal multiply or a different rounding rule picks another code
    rows = []
    for t in range(64):
        a = np.float32(g.uniform(0.05, 60))
        d32 = np.float32(a / np.float32(127))
        ks = g.integers(0, 127, 31)
        x0 = ((ks + 0.5) * np.float64(d32)).astype(np.float32)
        pick = g.integers(0, 3, 31)
        x = np.where(pick == 0, x0, np.where(pick == 1, np.nextafter(x0, np.float32(np.inf)),
                                               np.nextafter(x0, np.float32(0))))
        x = x * np.where(g.integers(0, 2, 31) == 0, 1, -1).astype(np.float32)
        rows.append(np.concatenate([[a], x]).astype(np.float32))
    x = np.concatenate(rows)[None, :]
    q, d, s = oracle.quantize_act(x, lib=lib)
    rq, rd, rs = ref_quantize(x, x.shape[1])
    assert np.array_equal(q, rq) and np.array_equal(d, rd) and np.array_equal(s, rs), "near-ties"


def pin_quantize_closed_forms(lib):
    K = 256
    # one-hot: x = a e_k
    for a, k in [(3.7, 5), (-0.03, 40), (250.0, 255), (1e-3, 128)]:
        x = np.zeros((1, K), np.float32)
        x[0, k] = a
        q, d, s = oracle.quantize_act(x, lib=lib)
        b = k // 32
        exp_q = np.zeros(K, np.int8)
        exp_q[k] = 127 if a > 0 else -127
        assert np.array_equal(q[0], exp_q)
        d_exp = np.float16(np.float32(abs(np.float32(a))) / np.float32(127)).view(np.uint16)
        assert d[0, b] == d_exp
        assert s[0, b] == exp_q[k]
        others = [i for i in range(K // 32) if i != b]
        assert np.all(d[0, others] == 0) and np.all(s[0, others] == 0)
    # all-equal positive block: every code 127, sum 32 * 127
    x = np.full((1, K), 0.37, np.float32)
    q, d, s = oracle.quantize_act(x, lib=lib)
    assert np.all(q == 127) and np.all(s == 4064)
    # exact ties x/d = k + 0.5 round away from zero (amax 127 gives d = 1)
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 127.0
    halves = np.array([0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 62.5, -62.5, 126.5, -126.5],
                      np.float32)
    x[0, 1:1 + halves.size] = halves
    q, d, s = oracle.quantize_act(x, lib=lib)
    exp = np.sign(halves) * (np.abs(halves) + 0.5)
    assert np.array_equal(q[0, 1:1 + halves.size].astype(np.float32), exp)
    assert d[0, 0] == np.float16(1.0).view(np.uint16)
    # all-zero input and padding past K
    q, d, s = oracle.quantize_act(np.zeros((1, 96), np.float32), lib=lib)
    assert q.shape == (1, 256) and not q.any() and not d.any() and not s.any()
    x = np.ones((1, 96), np.float32)
    q, d, s = oracle.quantize_act(x, lib=lib)
    assert np.all(q[0, :96] == 127) and not q[0, 96:].any()
    assert np.all(s[0, :3] == 4064) and not s[0, 3:].any() and not d[0, 3:].any()


# ---------------------------------------------------------- pack/unpack ----

def pin_unpack_roundtrip(lib):
    g = np.random.default_rng(5)
    # Q4_0
    w, raw = synth.q4_0_weights(g, 2, 64, raw=True)
    for r in range(2):
        for b in range(2):
            codes, d = oracle.unpack_q4_0(w[r, 18 * b:18 * b + 18], lib=lib)
            assert np.array_equal(codes, raw["codes"][r, 32 * b:32 * b + 32])
            assert d == raw["d"][r, b]
    # Q8_0
    w, raw = synth.q8_0_weights(g, 2, 64, raw=True)
    for r in range(2):
        for b in range(2):
            codes, d = oracle.unpack_q8_0(w[r, 34 * b:34 * b + 34], lib=lib)
            assert np.array_equal(codes, raw["codes"][r, 32 * b:32 * b + 32])
            assert d == raw["d"][r, b]
    # Q4_K: every value 0..63 in every one of the 8 scale and 8 min slots
    S = 64
    sc = np.empty((1, S, 8), np.uint8)
    mn = np.empty((1, S, 8), np.uint8)
    for v in range(64):
        sc[0, v] = (v + 7 * np.arange(8)) % 64
        mn[0, v] = (63 - v + 11 * np.arange(8)) % 64
    d = g.integers(0, 0x7C00, (1, S)).astype(np.uint16)
    dmin = g.integers(0, 0x7C00, (1, S)).astype(np.uint16)
    codes = g.integers(0, 16, (1, S * 256)).astype(np.uint8)
    w = synth.pack_q4_k(d, dmin, sc, mn, codes)
    for t in range(S):
        c, s_, m_, dd, dm = oracle.unpack_q4_k(w[0, 144 * t:144 * t + 144], lib=lib)
        assert np.array_equal(c, codes[0, 256 * t:256 * t + 256])
        assert np.array_equal(s_, sc[0, t]) and np.array_equal(m_, mn[0, t])
        assert dd == d[0, t] and dm == dmin[0, t]
    # Q6_K: every code 0..63 at every position, every scale value
    S = 64
    codes = ((np.arange(256)[None, :] + np.arange(S)[:, None]) % 64).astype(np.uint8)
    codes = codes.reshape(1, S * 256)
    sc = (((np.arange(16)[None, :] * 9 + np.arange(S)[:, None] * 2) % 128) - 64).astype(np.int8)
    sc = sc.reshape(1, S, 16)
    d = g.integers(0, 0x7C00, (1, S)).astype(np.uint16)
    w = synth.pack_q6_k(d, sc, codes)
    for t in range(S):
        c, s_, dd = oracle.unpack_q6_k(w[0, 210 * t:210 * t + 210], lib=lib)
        assert np.array_equal(c, codes[0, 256 * t:256 * t + 256])
        assert np.array_equal(s_, sc[0, t])
        assert dd == d[0, t]


# ------------------------------------------------------------- helpers -----

def dequant_rows(fmt: str, raw: dict, K: int) -> np.ndarray:
    """Float64 dequantised weights [N][K] from the raw draws (not the packed bytes)."""
    f = lambda h: np.asarray(h, np.uint16).view(np.float16).astype(np.float64)
    if fmt == "q4_0":
        d = np.repeat(f(raw["d"]), 32, axis=1)
        return d * (raw["codes"].astype(np.float64) - 8)
    if fmt == "q8_0":
        d = np.repeat(f(raw["d"]), 32, axis=1)
        return d * raw["codes"].astype(np.float64)
    if fmt == "q4_k":
        N = raw["codes"].shape[0]
        d = f(raw["d"])[:, :, None]
        dm = f(raw["dmin"])[:, :, None]
        scale = d * raw["sc"].astype(np.float64)      # [N][S][8]
        mins = dm * raw["mn"].astype(np.float64)
        c = raw["codes"].astype(np.float64).reshape(N, -1, 8, 32)
        w = scale[..., None] * c - mins[..., None]
        return w.reshape(N, -1)[:, :K]
    if fmt == "q6_k":
        N = raw["codes"].shape[0]
        d = f(raw["d"])[:, :, None]
        scale = d * raw["sc"].astype(np.float64)      # [N][S][16]
        c = raw["codes"].astype(np.float64).reshape(N, -1, 16, 16) - 32
        return (scale[..., None] * c).reshape(N, -1)[:, :K]
    raise ValueError(fmt)


def xhat(q, d, K):
    """Dequantised activation f(dx) * q over the first K columns."""
    dx = np.repeat(np.asarray(d, np.uint16).view(np.float16).astype(np.float64), 32)
    return (dx * np.asarray(q, np.float64).reshape(-1))[:K]


def brute_dots(fmt: str, raw: dict, q: np.ndarray, K: int):
    """Integer block dots from the raw codes with plain Python ints."""
    q = [int(v) for v in np.asarray(q).reshape(-1)]
    out = []
    for row in raw["codes"]:
        row = [int(v) for v in row]
        if fmt in ("q4_0", "q8_0"):
            off = 8 if fmt == "q4_0" else 0
            out.append([sum((row[32 * b + i] - off) * q[32 * b + i] for i in range(32))
                        for b in range(K // 32)])
        elif fmt == "q4_k":
            out.append([sum(row[32 * b + i] * q[32 * b + i] for i in range(32))
                        for b in range(len(row) // 32)])
        else:
            out.append([sum((row[16 * gi + i] - 32) * q[16 * gi + i] for i in range(16))
                        for gi in range(len(row) // 16)])
    return np.array(out, dtype=np.int64)


# --------------------------------------------------------------- dots ------

def pin_block_dots_brute(lib):
    g = np.random.default_rng(7)
    for fmt, K in [("q4_0", 32), ("q4_0", 160), ("q8_0", 96), ("q4_k", 256),
                   ("q4_k", 288), ("q4_k", 512), ("q6_k", 256), ("q6_k", 480)]:
        N = 5
        w, raw = synth.weights(fmt, g, N, K, raw=True)
        x, _ = synth.activation(g, 1, K)
        q, d, s = oracle.quantize_act(x, lib=lib)
        got = oracle.block_dots(fmt, w, N, K, q, lib=lib)
        ref = brute_dots(fmt, raw, q, K)
        assert np.array_equal(got.astype(np.int64), ref), f"{fmt} K={K}"
        # a row subset returns the same rows
        sub = oracle.block_dots(fmt, w, N, K, q, rows=(2, 2), lib=lib)
        assert np.array_equal(sub, got[2:4])


def pin_block_dots_closed_forms(lib):
    g = np.random.default_rng(8)
    K = 512
    x, _ = synth.activation(g, 1, K)
    q, d, s = oracle.quantize_act(x, lib=lib)
    q16 = q.reshape(-1).astype(np.int64).reshape(-1, 16).sum(axis=1)
    for c in (0, 5, 15):
        w = synth.pack_q4_0(np.full((1, K // 32), 0x3C00, np.uint16),
                            np.full((1, K), c, np.uint8))
        D = oracle.block_dots("q4_0", w, 1, K, q, lib=lib)[0]
        assert np.array_equal(D, (c - 8) * s[0, :K // 32])
        w = synth.pack_q4_k(np.full((1, 2), 0x3C00, np.uint16), np.zeros((1, 2), np.uint16),
                            np.ones((1, 2, 8), np.uint8), np.zeros((1, 2, 8), np.uint8),
                            np.full((1, K), c, np.uint8))
        D = oracle.block_dots("q4_k", w, 1, K, q, lib=lib)[0]
        assert np.array_equal(D, c * s[0])
    for c in (0, 32, 63):
        w = synth.pack_q6_k(np.full((1, 2), 0x3C00, np.uint16), np.ones((1, 2, 16), np.int8),
                            np.full((1, K), c, np.uint8))
        D = oracle.block_dots("q6_k", w, 1, K, q, lib=lib)[0]
        assert np.array_equal(D, (c - 32) * q16)


# ------------------------------------------------------------- outputs -----

def pin_gemv_dequant_brute(lib):
    g = np.random.default_rng(9)
    for fmt, K in [("q4_0", 64), ("q4_0", 224), ("q8_0", 128), ("q4_k", 256),
                   ("q4_k", 416), ("q4_k", 768), ("q6_k", 256), ("q6_k", 352),
                   ("q6_k", 512)]:
        N = 6
        w, raw = synth.weights(fmt, g, N, K, raw=True)
        x, _ = synth.activation(g, 1, K)
        q, d, s = oracle.quantize_act(x, lib=lib)
        y, T = oracle.gemv(fmt, w, N, K, q, d, s, lib=lib)
        W = dequant_rows(fmt, raw, K)
        ref = W @ xhat(q, d, K)
        assert np.all(np.abs(y - ref) <= 1e-12 * T + 1e-300), f"{fmt} K={K}"
        # T must be the sum of magnitudes of the separately scaled terms: it
        # bounds |y| and is no larger than sum |w_k x_hat_k| plus the
        # min-term magnitudes, which for one-sign formats is an equality
        assert np.all(np.abs(y) <= T * (1 + 1e-12))
        # the row subset path gives the same numbers
        y2, T2 = oracle.gemv(fmt, w, N, K, q, d, s, rows=(1, 3), lib=lib)
        assert np.array_equal(y2, y[1:4]) and np.array_equal(T2, T[1:4])


def pin_gemv_closed_forms(lib):
    g = np.random.default_rng(10)
    K = 512
    x, _ = synth.activation(g, 1, K)
    q, d, s = oracle.quantize_act(x, lib=lib)
    fdx = np.asarray(d, np.uint16).view(np.float16).astype(np.float64).reshape(-1)
    s1 = s.reshape(-1).astype(np.float64)
    # zero weight scales give exactly zero
    w = synth.pack_q4_0(np.zeros((2, K // 32), np.uint16), g.integers(0, 16, (2, K)).astype(np.uint8))
    y, T = oracle.gemv("q4_0", w, 2, K, q, d, s, lib=lib)
    assert np.all(y == 0) and np.all(T == 0)
    w = synth.pack_q6_k(np.full((2, 2), 0x3C00, np.uint16), np.zeros((2, 2, 16), np.int8),
                        g.integers(0, 64, (2, K)).astype(np.uint8))
    y, T = oracle.gemv("q6_k", w, 2, K, q, d, s, lib=lib)
    assert np.all(y == 0)
    # Q4_K with every scale 0 leaves only the min term: y = -sum f(dmin) m f(dx) s
    dmin = np.array([[0x1A00, 0x2C01]], np.uint16)
    mn = g.integers(0, 64, (1, 2, 8)).astype(np.uint8)
    w = synth.pack_q4_k(np.full((1, 2), 0x3C00, np.uint16), dmin,
                        np.zeros((1, 2, 8), np.uint8), mn,
                        g.integers(0, 16, (1, K)).astype(np.uint8))
    y, T = oracle.gemv("q4_k", w, 1, K, q, d, s, lib=lib)
    fdm = dmin.view(np.float16).astype(np.float64).reshape(-1)
    ref = -sum(fdm[b // 8] * mn[0, b // 8, b % 8] * fdx[b] * s1[b] for b in range(K // 32))
    assert abs(y[0] - ref) <= 1e-13 * T[0]
    # one-hot activation: y_r = f(dw) f(dx) (+-127) (code_k - 8) for Q4_0, etc.
    for sign in (1, -1):
        k = 77
        xo = np.zeros((1, K), np.float32)
        xo[0, k] = sign * 2.5
        qo, do, so = oracle.quantize_act(xo, lib=lib)
        fd = float(np.asarray(do[0, k // 32], np.uint16).view(np.float16))
        w, raw = synth.q4_0_weights(g, 3, K, raw=True)
        y, _ = oracle.gemv("q4_0", w, 3, K, qo, do, so, lib=lib)
        fdw = raw["d"][:, k // 32].view(np.float16).astype(np.float64)
        ref = fdw * fd * sign * 127 * (raw["codes"][:, k].astype(np.float64) - 8)
        assert np.array_equal(y, ref)
        w, raw = synth.q4_k_weights(g, 3, K, raw=True)
        y, _ = oracle.gemv("q4_k", w, 3, K, qo, do, so, lib=lib)
        S, j = k // 256, (k % 256) // 32
        fdd = raw["d"][:, S].view(np.float16).astype(np.float64)
        fdm = raw["dmin"][:, S].view(np.float16).astype(np.float64)
        ref = (fdd * raw["sc"][:, S, j] * fd * sign * 127 * raw["codes"][:, k]
               - fdm * raw["mn"][:, S, j] * fd * sign * 127)
        assert np.allclose(y, ref, rtol=1e-15, atol=0)
        w, raw = synth.q6_k_weights(g, 3, K, raw=True)
        y, _ = oracle.gemv("q6_k", w, 3, K, qo, do, so, lib=lib)
        gi = (k % 256) // 16
        fdd = raw["d"][:, S].view(np.float16).astype(np.float64)
        ref = fdd * raw["sc"][:, S, gi] * fd * sign * 127 * (raw["codes"][:, k].astype(np.float64) - 32)
        assert np.array_equal(y, ref)


def pin_quantization_error_bound(lib):
    """W4A8 vs the unquantised activation: |y - W x| <= sum_k |w_k| f(dx_b)/2
    plus the error of storing d in fp16 (relative 2^-11 per block)."""
    g = np.random.default_rng(12)
    for fmt, K in [("q4_0", 896), ("q4_k", 1024), ("q6_k", 1024)]:
        N = 8
        w, raw = synth.weights(fmt, g, N, K, raw=True)
        x, _ = synth.activation(g, 1, K)
        q, d, s = oracle.quantize_act(x, lib=lib)
        y, _ = oracle.gemv(fmt, w, N, K, q, d, s, lib=lib)
        W = dequant_rows(fmt, raw, K)
        exact = W @ x[0].astype(np.float64)
        fdx = np.repeat(np.asarray(d, np.uint16).view(np.float16).astype(np.float64).reshape(-1), 32)[:K]
        bound = np.abs(W) @ (fdx / 2 + np.abs(x[0]) * 2.0 ** -10) + 1e-12
        assert np.all(np.abs(y - exact) <= bound), fmt


def pin_gemm_rows(lib):
    g = np.random.default_rng(13)
    K, N, M = 416, 7, 4     # K not a multiple of 256: activation rows are padded
    w = synth.q4_k_weights(g, N, K)
    x, _ = synth.activation(g, M, K)
    q, d, s = oracle.quantize_act(x, lib=lib)
    Y, TT = oracle.gemm("q4_k", w, N, K, q, d, s, lib=lib)
    for m in range(M):
        y, T = oracle.gemv("q4_k", w, N, K, q[m], d[m], s[m], lib=lib)
        assert np.array_equal(Y[m], y) and np.array_equal(TT[m], T)
    # M rows of the same vector give M equal rows
    qq, dd, ss = (np.repeat(a[:1], 3, axis=0) for a in (q, d, s))
    Y, _ = oracle.gemm("q4_k", w, N, K, qq, dd, ss, lib=lib)
    assert np.array_equal(Y[0], Y[1]) and np.array_equal(Y[1], Y[2])


def pin_silu_mul(lib):
    import math
    gate = np.array([0.0, 1.0, -1.0, 20.0, -20.0, 0.5, -100.0, 3.25], np.float32)
    up = np.array([3.0, 2.0, 2.0, 1.0, 1.0, -4.0, 5.0, 0.0], np.float32)
    h = oracle.silu_mul(np.concatenate([gate, up]), lib=lib)
    # logistic(g) = 1 / (1 + e^-g); silu(g) = g * logistic(g)
    ref = np.array([float(gg) / (1.0 + math.exp(-float(gg))) * float(uu)
                    for gg, uu in zip(gate, up)])
    assert np.allclose(h, ref, rtol=1e-14, atol=0)
    assert h[0] == 0.0 and h[7] == 0.0
    assert abs(h[1] - 2 * 0.7310585786300049) < 1e-15   # 2 * logistic(1)


def pin_gemv_term_sums(lib):
    """T is the sum of |every separately scaled fp term|, from the raw draws."""
    g = np.random.default_rng(14)
    f = lambda h: np.asarray(h, np.uint16).view(np.float16).astype(np.float64)
    for fmt, K in [("q4_0", 192), ("q8_0", 96), ("q4_k", 288), ("q6_k", 288)]:
        N = 4
        w, raw = synth.weights(fmt, g, N, K, raw=True)
        x, _ = synth.activation(g, 1, K)
        q, d, s = oracle.quantize_act(x, lib=lib)
        _, T = oracle.gemv(fmt, w, N, K, q, d, s, lib=lib)
        D = brute_dots(fmt, raw, q, K).astype(np.float64)
        fdx = f(d).reshape(-1)
        s1 = s.reshape(-1).astype(np.float64)
        for r in range(N):
            if fmt in ("q4_0", "q8_0"):
                nb = K // 32
                ref = np.sum(np.abs(f(raw["d"][r]) * fdx[:nb] * D[r]))
            elif fmt == "q4_k":
                nb = (K + 31) // 32
                S_of = np.arange(nb) // 8
                j_of = np.arange(nb) % 8
                t1 = f(raw["d"][r])[S_of] * raw["sc"][r][S_of, j_of] * fdx[:nb] * D[r][:nb]
                t2 = f(raw["dmin"][r])[S_of] * raw["mn"][r][S_of, j_of] * fdx[:nb] * s1[:nb]
                ref = np.sum(np.abs(t1)) + np.sum(np.abs(t2))
            else:
                ng = K // 16
                S_of = np.arange(ng) // 16
                g_of = np.arange(ng) % 16
                t = (f(raw["d"][r])[S_of] * raw["sc"][r][S_of, g_of].astype(np.float64)
                     * fdx[np.arange(ng) // 2] * D[r][:ng])
                ref = np.sum(np.abs(t))
            assert abs(T[r] - ref) <= 1e-12 * ref, (fmt, r, T[r], ref)


ALL_PINS = [pin_fp16_decode_exhaustive, pin_fp16_encode_rne, pin_quantize_random,
            pin_quantize_closed_forms, pin_unpack_roundtrip, pin_block_dots_brute,
            pin_block_dots_closed_forms, pin_gemv_dequant_brute, pin_gemv_closed_forms,
            pin_quantization_error_bound, pin_gemv_term_sums, pin_gemm_rows, pin_silu_mul]


# ------------------------------------------------- literal block layouts ---
#
# Blocks built byte by byte, without synth's packers, with the expected fields
# written out as literals from the layout descriptions of the formats (GGUF
# block layouts, the reading of "llambda.lisp" README, Features &
# Architecture: Q4_K_M and Q6_K tensors are read straight from .gguf files).
# Every byte not named in a probe is zero, so every code not named in the
# expected map is zero.  Each placement rule (which byte and which bits feed
# which element) is exercised by at least one probe, so a misreading shared by
# the packer and the oracle -- which the round-trip pin cannot see -- fails
# here.

def _block(nbytes, assign):
    b = np.zeros(nbytes, np.uint8)
    for k, v in assign.items():
        b[k] = v
    return b


def _codes(n, nonzero, dtype=np.int64):
    c = np.zeros(n, dtype)
    for k, v in nonzero.items():
        c[k] = v
    return c


# (byte assignments, expected nonzero codes) per format
Q4_0_PROBES = [
    ({2 + 3: 0x0B}, {3: 11}),               # qs[3] low nibble -> element 3
    ({2 + 3: 0x60}, {19: 6}),               # qs[3] high nibble -> element 19
    ({17: 0xF1}, {15: 1, 31: 15}),          # qs[15] -> elements 15 and 31
    ({2: 0x7A}, {0: 10, 16: 7}),
]
Q8_0_PROBES = [
    ({2 + 5: 0xFE}, {5: -2}),
    ({33: 0x7F, 2: 0x81}, {31: 127, 0: -127}),
]
Q4_K_PROBES = [
    ({16: 0x03}, {0: 3}),                   # chunk 0, l = 0, low -> element 0
    ({16: 0x50}, {32: 5}),                  # chunk 0, l = 0, high -> element 32
    ({16 + 39: 0x0E}, {71: 14}),            # chunk 1, l = 7, low -> 64 + 7
    ({16 + 39: 0xB0}, {103: 11}),           # chunk 1, l = 7, high -> 64 + 32 + 7
    ({16 + 127: 0xF0}, {255: 15}),          # chunk 3, l = 31, high -> 192 + 32 + 31
    ({16 + 127: 0x09}, {223: 9}),           # chunk 3, l = 31, low -> 192 + 31
    ({16 + 80: 0x4D}, {144: 13, 176: 4}),   # chunk 2, l = 16
]
Q6_K_PROBES = [
    ({5: 0x0A}, {5: 10}),                   # ql[5] low -> element 5
    ({5: 0xA0}, {69: 10}),                  # ql[5] high -> element 5 + 64
    ({37: 0x07}, {37: 7}),                  # ql[37] low -> element 5 + 32
    ({37: 0x70}, {101: 7}),                 # ql[37] high -> element 5 + 96
    ({67: 0x0C}, {131: 12}),                # second half: ql[64 + 3] low -> 128 + 3
    ({99: 0xC0}, {227: 12}),                # ql[64 + 35] high -> 128 + 3 + 96
    ({128 + 9: 0x02}, {9: 32}),             # qh[9] bits 0-1 -> element 9, code bits 4-5
    ({128 + 9: 0x0C}, {41: 48}),            # qh[9] bits 2-3 -> element 9 + 32
    ({128 + 9: 0x10}, {73: 16}),            # qh[9] bits 4-5 -> element 9 + 64
    ({128 + 9: 0x80}, {105: 32}),           # qh[9] bits 6-7 -> element 9 + 96
    ({128 + 63: 0x40}, {255: 16}),          # qh[32 + 31] bits 6-7 -> 128 + 31 + 96
    ({128 + 32: 0x03}, {128: 48}),          # qh[32] bits 0-1 -> element 128
    ({0: 0x21, 128: 0xE4}, {0: 1, 32: 16, 64: 34, 96: 48}),
]
# Q4_K header: d = 0x3555, dmin = 0x2AAA, then the 12 scale bytes of
#   scales 5, 17, 33, 62, 45, 28, 51, 12 and mins 9, 40, 3, 63, 22, 57, 36, 1:
#   bytes 0-3: scale j (bits 0-5) | top two bits of scale j+4 (bits 6-7)
#   bytes 4-7: min j (bits 0-5) | top two bits of min j+4 (bits 6-7)
#   bytes 8-11: low 4 bits of scale j+4 | low 4 bits of min j+4 << 4
Q4_K_HEADERS = [
    ({0: 0x55, 1: 0x35, 2: 0xAA, 3: 0x2A, 4: 0x85, 5: 0x51, 6: 0xE1, 7: 0x3E, 8: 0x49, 9: 0xE8,
      10: 0x83, 11: 0x3F, 12: 0x6D, 13: 0x9C, 14: 0x43, 15: 0x1C},
     0x3555, 0x2AAA, [5, 17, 33, 62, 45, 28, 51, 12], [9, 40, 3, 63, 22, 57, 36, 1]),
    ({4: 0xC0}, 0, 0, [0, 0, 0, 0, 48, 0, 0, 0], [0] * 8),    # top bits of scale 4 only
    ({11: 0x80}, 0, 0, [0] * 8, [0, 0, 0, 0, 0, 0, 0, 32]),   # top bits of min 7 only
    ({14: 0x5A}, 0, 0, [0, 0, 0, 0, 0, 0, 10, 0], [0, 0, 0, 0, 0, 0, 5, 0]),
    ({6: 0x7F}, 0, 0, [0, 0, 63, 0, 0, 0, 16, 0], [0] * 8),   # scale 2 | top bit of scale 6
]
Q6_K_SCALES = [0xC0, 0x3F, 0xFF, 0x00, 0x11, 0xDF, 0x05, 0xF8,
               0x80, 0x7F, 0x01, 0x02, 0xFE, 0x40, 0x9C, 0x2A]
Q6_K_SCALE_VALUES = [-64, 63, -1, 0, 17, -33, 5, -8, -128, 127, 1, 2, -2, 64, -100, 42]


def pin_layout_literal_blocks(lib):
    for assign, exp in Q4_0_PROBES:
        codes, d = oracle.unpack_q4_0(_block(18, assign), lib=lib)
        assert np.array_equal(codes.astype(np.int64), _codes(32, exp)), ("q4_0", assign)
        assert d == 0
    codes, d = oracle.unpack_q4_0(_block(18, {0: 0x34, 1: 0x12}), lib=lib)
    assert d == 0x1234 and not codes.any()
    for assign, exp in Q8_0_PROBES:
        codes, d = oracle.unpack_q8_0(_block(34, assign), lib=lib)
        assert np.array_equal(codes.astype(np.int64), _codes(32, exp)), ("q8_0", assign)
    codes, d = oracle.unpack_q8_0(_block(34, {0: 0x00, 1: 0x3C}), lib=lib)
    assert d == 0x3C00 and not codes.any()
    for assign, exp in Q4_K_PROBES:
        codes, sc, mn, d, dmin = oracle.unpack_q4_k(_block(144, assign), lib=lib)
        assert np.array_equal(codes.astype(np.int64), _codes(256, exp)), ("q4_k", assign)
        assert not sc.any() and not mn.any() and d == 0 and dmin == 0
    for assign, d_e, dmin_e, sc_e, mn_e in Q4_K_HEADERS:
        codes, sc, mn, d, dmin = oracle.unpack_q4_k(_block(144, assign), lib=lib)
        assert not codes.any()
        assert d == d_e and dmin == dmin_e, ("q4_k header", assign)
        assert list(sc) == sc_e and list(mn) == mn_e, ("q4_k scales/mins", assign, sc, mn)
    for assign, exp in Q6_K_PROBES:
        codes, sc, d = oracle.unpack_q6_k(_block(210, assign), lib=lib)
        assert np.array_equal(codes.astype(np.int64), _codes(256, exp)), ("q6_k", assign)
        assert not sc.any() and d == 0
    hdr = {192 + i: v for i, v in enumerate(Q6_K_SCALES)}
    hdr.update({208: 0x34, 209: 0x12})
    codes, sc, d = oracle.unpack_q6_k(_block(210, hdr), lib=lib)
    assert not codes.any() and d == 0x1234
    assert list(sc.astype(int)) == Q6_K_SCALE_VALUES


ALL_PINS.append(pin_layout_literal_blocks)
