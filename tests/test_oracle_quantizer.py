"""Pins of the oracle's quantizer Qz (compensator extraction, smoothing, INT8
requantization) and of its dequantization.  CPU only.

The pages (arXiv 2609.38166 abstract, "Abstract (arXiv)" section; bedrocknews
review) say the largest outlier rows and columns are kept as high-precision
Compensator Tokens and the smoothed residual is quantized to 8 bits; the
formulas are readings.  These tests check the oracle against brute force
(every candidate subset, every one of the 255 codes), closed-form bounds and
a hand-worked example -- not against a retyped copy of its own loops.
"""
import itertools
from fractions import Fraction as F

import numpy as np
import pytest

from oracle import exact
from tests.test_oracle_recurrence import parse_golden


def _dyadic_state(rng, dv, dk, scale=64):
    return rng.integers(-scale, scale + 1, (dv, dk)) / 8.0


@pytest.mark.parametrize("n_c", range(0, 9))
def test_selection_is_best_subset_4x4(orc, n_c):
    rng = np.random.default_rng(100 + n_c)
    states = [_dyadic_state(rng, 4, 4) for _ in range(12)]
    # planted exact ties between lines: equal squared norms
    t = np.array([[1, 2, 0, 0], [2, 1, 0, 0], [0, 0, 2, 1], [0, 0, 1, 2]], float)
    states.append(t)
    states.append(np.zeros((4, 4)))
    states.append(np.ones((4, 4)))
    for S in states:
        blob, _, scores = orc.qz(S[None], n_c)
        fS = exact.frac_matrix(S)
        want = exact.best_subset(exact.line_scores(fS), n_c)
        assert list(blob.comp_idx[0]) == want, (S, want, blob.comp_idx)
        np.testing.assert_array_equal(scores[0], [float(x) for x in exact.line_scores(fS)])


def test_codes_are_nearest_with_even_ties(orc):
    rng = np.random.default_rng(11)
    # random dyadic states: every code is the argmin over all 255 codes of |x - c|
    for _ in range(20):
        S = _dyadic_state(rng, 4, 4)
        blob, x, _ = orc.qz(S[None], 1)
        Sf = exact.frac_matrix(S)
        for i in range(4):
            for j in range(4):
                if blob.sigma[0, i] == 0:
                    assert blob.codes[0, i, j] == 0
                    continue
                on_line = (i in blob.comp_idx[0]) or (4 + j in blob.comp_idx[0])
                R = F(0) if on_line else Sf[i][j]
                xe = R / (F(float(blob.sigma[0, i])) * F(float(blob.smooth[0, j])))
                assert blob.codes[0, i, j] == exact.nearest_code(xe)
    # planted exact half-integer x: sigma_0 = 1 exactly (row max 127 * s_0 with
    # s_0 = 127), s = 8 elsewhere, entries (n + 1/2) * 8
    S = np.zeros((2, 4))
    S[0] = [16129.0, 2.5 * 8, 3.5 * 8, -0.5 * 8]
    S[1] = [1.0, 64.0, -64.0, 64.0]
    blob, x, _ = orc.qz(S[None], 0)
    assert blob.smooth[0].tolist() == [127.0, 8.0, 8.0, 8.0]
    assert blob.sigma[0, 0] == 1.0
    assert x[0, 0].tolist() == [127.0, 2.5, 3.5, -0.5]
    assert blob.codes[0, 0].tolist() == [127, 2, 4, 0]


@pytest.mark.parametrize("dv,dk,n_c", [(8, 8, 2), (16, 12, 5), (12, 16, 0), (32, 32, 4)])
def test_reconstruction_bound_and_code_range(orc, dv, dk, n_c):
    rng = np.random.default_rng(12)
    S = rng.standard_normal((6, dv, dk)) * rng.uniform(0.1, 10, (6, 1, 1))
    S[:, 1, :] *= 30.0  # an outlier row
    S[:, :, 2] *= 25.0  # an outlier column
    blob, x, scores = orc.qz(S, n_c)
    Sh = orc.dequant(blob)
    for u in range(S.shape[0]):
        rows = {c for c in blob.comp_idx[u] if c < dv}
        cols = {c - dv for c in blob.comp_idx[u] if c >= dv}
        assert len(rows) + len(cols) == n_c
        for i in range(dv):
            for j in range(dk):
                if i in rows or j in cols:
                    # compensator lines hold S exactly up to one fp32 rounding
                    assert abs(Sh[u, i, j] - S[u, i, j]) <= 2 ** -24 * abs(S[u, i, j]) * 1.0000001
                else:
                    bound = 0.5 * float(blob.sigma[u, i]) * float(blob.smooth[u, j])
                    assert abs(Sh[u, i, j] - S[u, i, j]) <= bound * (1 + 1e-12) + 1e-300
        assert np.abs(blob.codes[u].astype(int)).max() <= 127
        for i in range(dv):
            if i in rows:
                assert blob.sigma[u, i] == 0 and not blob.codes[u, i].any()
            else:
                assert np.abs(blob.codes[u, i].astype(int)).max() == 127
        # smoothing: s_j^2 is the residual column absmax, to fp32 rounding
        R = S[u].copy()
        for i in rows:
            R[i, :] = 0
        for j in cols:
            R[:, j] = 0
        a = np.abs(R).max(axis=0)
        for j in range(dk):
            if a[j] == 0:
                assert blob.smooth[u, j] == 1.0
            else:
                assert abs(float(blob.smooth[u, j]) ** 2 - a[j]) <= 2.5 * 2 ** -24 * a[j]


def test_degenerate_states(orc):
    # zero state: no outliers to keep, codes 0, sigma 0, s 1; the first n_c rows
    # win the all-zero tie and hold zero vectors
    blob, _, _ = orc.qz(np.zeros((2, 5, 6)), 3)
    assert not blob.codes.any() and not blob.sigma.any()
    assert (blob.smooth == 1).all()
    assert blob.comp_idx.tolist() == [[0, 1, 2], [0, 1, 2]]
    assert not blob.comp_vec.any()
    assert not orc.dequant(blob).any()
    # a zero row gets sigma 0; a zero column gets s 1
    S = np.arange(1, 26, dtype=float).reshape(1, 5, 5)
    S[0, 3, :] = 0
    S[0, :, 1] = 0
    blob, _, _ = orc.qz(S, 0)
    assert blob.sigma[0, 3] == 0 and not blob.codes[0, 3].any()
    assert blob.smooth[0, 1] == 1.0 and not blob.codes[0, :, 1].any()
    # n_c = d_v + d_k keeps everything in the compensators: the residual is 0
    S = np.random.default_rng(3).standard_normal((1, 3, 4))
    blob, _, _ = orc.qz(S, 7)
    assert not blob.codes.any()
    np.testing.assert_allclose(orc.dequant(blob), S.astype(np.float32), rtol=0, atol=0)


def test_forced_selection(orc):
    rng = np.random.default_rng(5)
    S = rng.standard_normal((3, 6, 6))
    blob, _, _ = orc.qz(S, 2)
    forced = np.array([[0, 7], [1, 2], [6, 11]], np.int32)
    blob2, _, _ = orc.qz(S, 2, force_sel=forced)
    assert blob2.comp_idx.tolist() == forced.tolist()
    same = orc.qz(S, 2, force_sel=blob.comp_idx)[0]
    assert np.array_equal(same.codes, blob.codes)


@pytest.mark.parametrize("n_c", [1, 2, 3])
def test_golden_3x3_worked_example(orc, n_c):
    g = parse_golden("quantizer_3x3.txt")
    S = np.array(g["S"], float).reshape(1, 3, 3)
    blob, _, _ = orc.qz(S, n_c)
    p = f"nc{n_c}."
    assert blob.comp_idx[0].tolist() == [int(x) for x in g[p + "comp_idx"]]
    np.testing.assert_array_equal(blob.comp_vec[0].ravel(), np.array(g[p + "comp_vec"], np.float32))
    np.testing.assert_array_equal(blob.smooth[0], np.array(g[p + "smooth"], np.float32))
    sig = [np.float32(int(a) / int(b)) for a, b in (r.split("/") for r in g[p + "sigma_ratio"])]
    np.testing.assert_array_equal(blob.sigma[0], np.array(sig, np.float32))
    assert blob.codes[0].ravel().tolist() == [int(x) for x in g[p + "codes"]]


def test_golden_3x3_naive_ablation(orc):
    # the naive per-token ablation's quantizer (no compensators, no smoothing)
    # against the hand-worked values: s = 1, sigma = row absmax / 127
    g = parse_golden("quantizer_3x3.txt")
    S = np.array(g["S"], float).reshape(1, 3, 3)
    blob, _, _ = orc.qz(S, 0, smooth=False)
    assert blob.comp_idx.shape == (1, 0)
    np.testing.assert_array_equal(blob.smooth[0], np.array(g["naive.smooth"], np.float32))
    sig = [np.float32(int(a) / int(b)) for a, b in (r.split("/") for r in g["naive.sigma_ratio"])]
    np.testing.assert_array_equal(blob.sigma[0], np.array(sig, np.float32))
    assert blob.codes[0].ravel().tolist() == [int(x) for x in g["naive.codes"]]
    # the same state with smoothing on differs (the ablation switch is live)
    smoothed, _, _ = orc.qz(S, 0, smooth=True)
    assert not np.array_equal(smoothed.smooth[0], blob.smooth[0])
