"""Pins of the oracle's binary16 window buffer (k and v stored as IEEE half
precision).  CPU only.

The arXiv abstract ("Abstract (arXiv)" section, mlsanity.com paper page) asks
for high-precision buffered updates; the binary16 buffer is the compact
reading of that.  The rounding is checked against numpy's independent float16
conversion (every finite half value, every midpoint between neighbours,
random fp32 inputs), against the format's anchor values, and the windowed run
against the plain FP64 recurrence of the rounded tokens.
"""
import numpy as np
import pytest


def _finite_halves():
    h = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
    return h[np.isfinite(h)].astype(np.float32)


def test_representable_values_are_kept(orc):
    h = _finite_halves()
    out = orc.fp16_round(h)
    assert np.array_equal(out.view(np.uint32), h.view(np.uint32))  # signed zeros included


def test_midpoints_and_neighbours_match_numpy(orc):
    h = np.unique(_finite_halves())
    mids = ((h[:-1].astype(np.float64) + h[1:]) / 2).astype(np.float32)  # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (h[:-1].astype(np.float64) + h[1:]) / 2)
    x = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))])
    x = x[np.abs(x) <= 65504]
    ref = x.astype(np.float16).astype(np.float32)
    assert np.array_equal(orc.fp16_round(x), ref)


def test_random_fp32_match_numpy(orc):
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(20000) * 1e-5,
                        np.exp(rng.uniform(np.log(1e-9), np.log(65000), 20000)) * rng.choice([-1, 1], 20000),
                        rng.standard_t(3, 20000) * 50]).astype(np.float32)
    ref = x.astype(np.float16).astype(np.float32)
    assert np.array_equal(orc.fp16_round(x), ref)


def test_anchors_saturation_and_nan(orc):
    f = lambda v: float(orc.fp16_round(np.array([v], np.float32))[0])
    assert f(65504.0) == 65504.0 and f(65519.0) == 65504.0 and f(65520.0) == 65504.0
    assert f(1e30) == 65504.0 and f(-1e30) == -65504.0 and f(np.inf) == 65504.0
    assert np.isnan(f(np.nan))
    assert f(2.0 ** -24) == 2.0 ** -24  # smallest subnormal
    assert f(2.0 ** -25) == 0.0  # tie between 0 and 2^-24: even
    assert f(3 * 2.0 ** -25) == 2.0 ** -23  # tie between 1 and 2 units: even
    assert f(2.0 ** -14) == 2.0 ** -14  # smallest normal
    assert f(1.0 + 2.0 ** -11) == 1.0  # tie: even mantissa
    assert f(1.0 + 3 * 2.0 ** -11) == 1.0 + 2.0 ** -9
    assert f(2049.0) == 2048.0 and f(2051.0) == 2052.0  # spacing 2 above 2048


@pytest.mark.parametrize("kda", [False, True])
def test_fp16_window_is_the_windowed_run_of_rounded_tokens(orc, kda):
    """With no quantization boundary inside the run (W > T, n_c = d_v + d_k so the
    quantizer keeps every line exactly up to fp32), the fp16-buffer run is the
    plain recurrence of the binary16-rounded keys and values."""
    rng = np.random.default_rng(31)
    U, d, T = 3, 8, 20
    S0 = rng.standard_normal((U, d, d)).astype(np.float32).astype(np.float64)
    k = rng.standard_normal((T, U, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((T, U, d))
    v = rng.standard_normal((T, U, d)) * 3
    b = rng.uniform(0, 1, (T, U))
    g = rng.uniform(0.8, 1, (T, U, d) if kda else (T, U))
    o = orc.windowed_run(S0, q, k, v, b, g, T + 1, 2 * d, buffer="fp16")
    kr = orc.fp16_round(k.astype(np.float32))
    vr = orc.fp16_round(v.astype(np.float32))
    assert not np.array_equal(kr, k.astype(np.float32))  # the rounding does something
    _, o_ref = orc.recurrence(S0, q, kr, vr, b, g)
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    _, o_raw = orc.recurrence(S0, q, k, v, b, g)
    assert np.abs(o - o_raw).max() > 1e-6
