"""The seeded input generator: determinism, value ranges, padding and sizes."""
import numpy as np

import oracle
import synth


def test_deterministic_and_seeded():
    a = synth.q6_k_weights(synth.rng(3), 17, 512)
    b = synth.q6_k_weights(synth.rng(3), 17, 512)
    c = synth.q6_k_weights(synth.rng(4), 17, 512)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    x1, ch1 = synth.activation(synth.rng(0), 2, 896)
    x2, ch2 = synth.activation(synth.rng(0), 2, 896)
    assert np.array_equal(x1, x2) and np.array_equal(ch1, ch2)


def test_value_ranges():
    g = synth.rng(1)
    f16 = lambda h: np.asarray(h, np.uint16).view(np.float16).astype(np.float64)
    _, raw = synth.q4_0_weights(g, 64, 256, raw=True)
    assert raw["codes"].max() <= 15 and raw["codes"].min() >= 0
    assert f16(raw["d"]).min() >= 1e-3 * (1 - 2**-10) and f16(raw["d"]).max() <= 4e-3 * (1 + 2**-10)
    _, raw = synth.q4_k_weights(g, 64, 512, raw=True)
    assert raw["sc"].max() <= 63 and raw["mn"].max() <= 63 and raw["codes"].max() <= 15
    assert f16(raw["d"]).min() >= 1e-4 * (1 - 2**-10) and f16(raw["dmin"]).max() <= 1e-3 * (1 + 2**-10)
    _, raw = synth.q6_k_weights(g, 256, 512, raw=True)
    assert raw["codes"].max() == 63 and raw["codes"].min() == 0
    assert raw["sc"].min() == -64 and raw["sc"].max() == 63
    dv = f16(raw["d"])
    assert dv.min() >= 1e-5 * (1 - 2**-9) and dv.max() <= 1e-4 * (1 + 2**-10)
    sub = np.mean((raw["d"] & 0x7C00) == 0)  # binary16 subnormal encodings
    assert 0.5 < sub < 0.65       # (2^-14 - 1e-5) / 9e-5 ~ 0.567


def test_padding_is_zero():
    g = synth.rng(2)
    _, raw = synth.q4_k_weights(g, 8, 896, raw=True)
    assert not raw["codes"][:, 896:].any()
    assert not raw["sc"][:, 3, 4:].any() and not raw["mn"][:, 3, 4:].any()
    assert raw["sc"][:, 3, :4].any()
    _, raw = synth.q6_k_weights(g, 8, 288, raw=True)
    assert not raw["codes"][:, 288:].any() and not raw["sc"][:, 1, 2:].any()


def test_outlier_channels():
    for K, n in [(896, 9), (4096, 41), (4864, 49), (14336, 143)]:
        x, ch = synth.activation(synth.rng(5), 3, K)
        assert len(ch) == n and len(set(ch.tolist())) == n
        assert x.dtype == np.float32 and x.shape == (3, K)


def test_config_sizes():
    """Stored and logical weight bytes of the five workloads."""
    assert synth.row_bytes("q4_0", 896) == 504
    assert synth.row_bytes("q4_k", 896) == 576 and synth.row_bytes("q4_k", 4864) == 2736
    assert synth.row_bytes("q4_k", 4096) == 2304
    assert synth.row_bytes("q6_k", 14336) == 11760 and synth.row_bytes("q6_k", 4096) == 3360
    assert synth.logical_bytes("q6_k", 128256, 4096) == 430_940_160
    assert synth.logical_bytes("q4_k", 28672, 4096) == 66_060_288
    assert synth.logical_bytes("q6_k", 4096, 14336) == 48_168_960
    assert synth.logical_bytes("q4_k", 14336, 4096) == 33_030_144
    layer = sum(synth.logical_bytes("q4_k", N, K) for _, N, K in synth.CONFIG1_SHAPES)
    assert layer == 8_386_560
    for fmt, K in [("q4_0", 96), ("q4_k", 896), ("q6_k", 4096), ("q8_0", 64)]:
        assert synth.row_bytes(fmt, K) == oracle.row_bytes(fmt, K)


def test_config0_and_config1_shapes():
    c0 = synth.config0()
    assert c0["w"].shape == (896, 504) and c0["x"].shape == (1, 896)
    c1 = synth.config1()
    assert c1["mats"]["k"]["w"].shape == (128, 576)
    assert c1["mats"]["down"]["w"].shape == (896, 2736)
    assert np.array_equal(c1["mats"]["q"]["x"], c1["mats"]["up"]["x"])
    assert not np.array_equal(c1["mats"]["q"]["x"], c1["mats"]["o"]["x"])
