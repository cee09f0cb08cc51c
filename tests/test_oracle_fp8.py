"""Pins of the oracle's 8-bit floating-point (E4M3) code format.  CPU only.

The arXiv abstract ("Abstract (arXiv)" section, mlsanity.com paper page) keeps
the state in 8 bits, the bedrocknews.com review says INT8; the E4M3 variant is
the floating-point reading of "8-bit" (OCP 8-bit floating point, E4M3 without
infinities: bias 7, three mantissa bits, largest finite magnitude 448).  These
tests check the oracle's E4M3 value table against torch's independent
float8_e4m3fn implementation and against the format's fixed anchor values,
its rounding against brute force over every finite code, and its quantizer
against the reconstruction bound the format implies -- not against a retyped
copy of the oracle's own arithmetic.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def _table(orc):
    return np.array([orc.e4m3_value(c) for c in range(256)])


def test_value_table_matches_torch(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = _table(orc)
    for c in range(256):
        if math.isnan(ref[c]):
            assert math.isnan(mine[c]), c
        else:
            assert mine[c] == ref[c], (c, mine[c], ref[c])


def test_anchor_values_and_order(orc):
    v = _table(orc)
    assert v[0x00] == 0.0 and v[0x80] == 0.0
    assert v[0x38] == 1.0 and v[0xB8] == -1.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0  # largest finite magnitude
    assert v[0x08] == 2.0 ** -6  # smallest normal
    assert v[0x01] == 2.0 ** -9  # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9
    assert math.isnan(v[0x7F]) and math.isnan(v[0xFF])
    pos = v[:0x7F]
    assert (np.diff(pos) > 0).all()  # codes 0..126 are strictly increasing
    assert np.array_equal(v[0x80:0xFF], -pos)
    assert len(set(pos.tolist())) == 127


def _nearest_even(table, x):
    """Brute force: the finite code nearest to x; on an exact tie the even code."""
    a = min(abs(x), 448.0)
    best = None
    for c in range(0x7F):
        d = abs(table[c] - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    c = best[1]
    return c | (0x80 if (x < 0 and c != 0) else 0)


def test_encode_is_nearest_with_even_ties(orc):
    table = _table(orc)
    pos = table[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(8)
    xs = list(pos) + list(mids) + list(mids * (1 + 2.0 ** -30)) + list(mids * (1 - 2.0 ** -30))
    xs += list(np.exp(rng.uniform(math.log(2.0 ** -12), math.log(460.0), 3000)))
    xs += list(rng.uniform(0, 2.0 ** -5, 500))
    for x in xs:
        for sx in (x, -x):
            assert orc.e4m3_encode(sx) == _nearest_even(table, sx), sx


def test_encode_matches_torch_on_fp32_inputs(orc):
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(4000) * 50, rng.uniform(-448, 448, 4000),
                        rng.standard_normal(2000) * 2.0 ** -7]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([orc.e4m3_encode(float(t)) for t in x])
    # torch keeps the sign of a value that rounds to zero; the oracle stores +0
    ref = np.where(ref == 0x80, 0, ref)
    assert np.array_equal(mine, ref)


def test_encode_saturates_and_zero(orc):
    assert orc.e4m3_encode(448.0) == 0x7E
    assert orc.e4m3_encode(464.0) == 0x7E
    assert orc.e4m3_encode(1e9) == 0x7E and orc.e4m3_encode(-1e9) == 0xFE
    assert orc.e4m3_encode(0.0) == 0 and orc.e4m3_encode(-0.0) == 0
    assert orc.e4m3_encode(-2.0 ** -11) == 0  # rounds to zero: +0
    assert orc.e4m3_encode(2.0 ** -10) == 0  # tie between 0 and 2^-9: the even code 0
    assert orc.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie between codes 1 and 2: code 2
    assert orc.e4m3_encode(17.0) == orc.e4m3_encode(16.0)  # 17 ties 16 (m=0) and 18 (m=1)


def _spacing(x):
    a = abs(x)
    E = max(math.floor(math.log2(a)), -6) if a > 0 else -6
    return 2.0 ** (E - 3)


@pytest.mark.parametrize("dv,dk,n_c", [(8, 8, 2), (16, 12, 5), (32, 32, 4)])
def test_e4m3_reconstruction_bound(orc, dv, dk, n_c):
    rng = np.random.default_rng(13)
    S = rng.standard_normal((5, dv, dk)) * rng.uniform(0.1, 10, (5, 1, 1))
    S[:, 1, :] *= 30.0
    S[:, :, 2] *= 25.0
    blob, x, _ = orc.qz(S, n_c, fmt="e4m3")
    ref, _, _ = orc.qz(S, n_c)  # INT8: same selection and smoothing
    assert np.array_equal(blob.comp_idx, ref.comp_idx)
    assert np.array_equal(blob.smooth, ref.smooth)
    Sh = orc.dequant(blob)
    vals = orc.code_values(blob.codes, "e4m3")
    table = _table(orc)
    for u in range(S.shape[0]):
        rows = {c for c in blob.comp_idx[u] if c < dv}
        cols = {c - dv for c in blob.comp_idx[u] if c >= dv}
        for i in range(dv):
            if i in rows:
                assert blob.sigma[u, i] == 0 and not blob.codes[u, i].any()
                continue
            # every kept row reaches the format's largest magnitude
            assert np.abs(vals[u, i]).max() == 448.0
            for j in range(dk):
                if j in cols:
                    continue
                c = int(blob.codes[u, i, j]) & 0xFF
                assert c not in (0x7F, 0xFF)
                assert c == _nearest_even(table, x[u, i, j])
                # half a code spacing at x, in units of sigma_i s_j
                bound = 0.5 * _spacing(x[u, i, j]) * float(blob.sigma[u, i]) * float(blob.smooth[u, j])
                assert abs(Sh[u, i, j] - S[u, i, j]) <= bound * (1 + 1e-12) + 1e-300
        # scales: sigma_i = row absmax of R/s over 448, rounded to fp32
        R = S[u].copy()
        for i in rows:
            R[i, :] = 0
        for j in cols:
            R[:, j] = 0
        m = np.abs(R / blob.smooth[u].astype(np.float64)).max(axis=1)
        for i in range(dv):
            if i not in rows:
                assert blob.sigma[u, i] == np.float32(m[i] / 448.0)


def test_e4m3_replay_equals_definitional_window(orc):
    """O3 (buffered replay) equals O2 (FP64 state advanced token by token) from
    an E4M3 window-start state, as it does for INT8."""
    rng = np.random.default_rng(21)
    U, d, n = 3, 16, 9
    S = rng.standard_normal((U, d, d))
    blob, _, _ = orc.qz(S, 2, fmt="e4m3")
    S_hat = orc.dequant(blob)
    k = rng.standard_normal((n, U, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((n, U, d))
    v = rng.standard_normal((n, U, d))
    b = rng.uniform(0, 1, (n, U))
    g = rng.uniform(0.9, 1, (n, U))
    _, o_ref = orc.recurrence(S_hat, q, k, v, b, g)
    bk, bv = np.transpose(k, (1, 0, 2)), np.transpose(v, (1, 0, 2))
    o = orc.replay_output(blob, bk, bv, b.T, g.T, q[-1])
    np.testing.assert_allclose(o, o_ref[-1], rtol=1e-12, atol=1e-12)


def test_e4m3_windowed_run_beats_naive_and_tracks_int8(orc):
    rng = np.random.default_rng(22)
    U, d, T = 6, 32, 96
    S0 = rng.standard_normal((U, d, d))
    k = rng.standard_normal((T, U, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((T, U, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, U, d))
    b = rng.uniform(0, 1, (T, U))
    g = rng.uniform(0.9, 1, (T, U))
    _, o_ref = orc.recurrence(S0, q, k, v, b, g)
    err = lambda o: np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref)
    e8 = err(orc.windowed_run(S0, q, k, v, b, g, 32, 2, fmt="e4m3"))
    ei = err(orc.windowed_run(S0, q, k, v, b, g, 32, 2))
    naive = err(orc.windowed_run(S0, q, k, v, b, g, 1, 0, smooth=False, fmt="e4m3"))
    assert e8 < naive
    assert 0.2 < e8 / ei < 20  # same order as INT8 (3 mantissa bits vs 7 bits of range)
