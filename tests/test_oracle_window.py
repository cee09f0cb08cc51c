"""Pins of the oracle's windowed forms.  CPU only.

O3 (output from the fixed low-bit state plus the buffered window, by a reverse
pass over the buffer) and O2 (the definitional windowed run) follow the arXiv
2609.38166 abstract ("Abstract (arXiv)" section of the mlsanity.com paper
page): a token inside a window reads the 8-bit state, unchanged since the
window began, plus the window's full-precision tokens, and the state is
requantized a single time, when the window closes.  With quantization out of the picture the windowed form must
reproduce the plain recurrence; that, an exact closed-form sum, and the
linearity of compensator tokens pin them.
"""
from fractions import Fraction as F

import numpy as np
import pytest

from oracle import exact
from tests.test_oracle_recurrence import parse_golden, rand_tokens


def exact_blob(orc, S_int, comps=()):
    """A stored state that represents an integer matrix exactly: codes = S,
    sigma = 1, s = 1; optional compensator slots (index, fp32 vector)."""
    U, dv, dk = S_int.shape
    D = max(dv, dk)
    ci = np.array([[c for c, _ in comps]] * U, np.int32).reshape(U, len(comps))
    cv = np.zeros((U, len(comps), D), np.float32)
    for s, (_, vec) in enumerate(comps):
        cv[:, s, :len(vec)] = vec
    return orc.Blob(S_int.astype(np.int8), np.ones((U, dv), np.float32),
                    np.ones((U, dk), np.float32), ci, cv)


def entries_from_tokens(q, k, v, b, g):
    """Token-major [n, U, ...] -> unit-major buffer [U, n, ...]."""
    return (np.ascontiguousarray(k.swapaxes(0, 1)), np.ascontiguousarray(v.swapaxes(0, 1)),
            np.ascontiguousarray(b.swapaxes(0, 1)), np.ascontiguousarray(g.swapaxes(0, 1)))


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("n", [1, 2, 7, 33])
def test_replay_equals_plain_recurrence(orc, kda, n):
    rng = np.random.default_rng(20 + n + 100 * kda)
    U, dv, dk = 5, 12, 16
    S_int = rng.integers(-127, 128, (U, dv, dk))
    blob = exact_blob(orc, S_int)
    q, k, v, b, g = rand_tokens(rng, n, U, dk, dv, kda)
    _, o = orc.recurrence(S_int.astype(np.float64), q, k, v, b, g)
    bk, bv, bb, bg = entries_from_tokens(q, k, v, b, g)
    o3 = orc.replay_output(blob, bk, bv, bb, bg, q[-1])
    np.testing.assert_allclose(o3, o[-1], rtol=1e-12, atol=1e-12 * np.abs(o[-1]).max())


@pytest.mark.parametrize("kda", [False, True])
def test_replay_with_compensators_is_linear(orc, kda):
    # compensator tokens share the update path: slots == the same lines folded
    # into the state
    rng = np.random.default_rng(31 + kda)
    U, dv, dk, n = 3, 8, 8, 9
    S_int = rng.integers(-100, 101, (U, dv, dk))
    row = rng.standard_normal(dk).astype(np.float32)
    col = rng.standard_normal(dv).astype(np.float32)
    blob = exact_blob(orc, S_int, comps=[(2, row), (dv + 5, col)])
    dense = S_int.astype(np.float64)
    dense[:, 2, :] += row
    dense[:, :, 5] += col
    np.testing.assert_array_equal(orc.dequant(blob), dense)
    q, k, v, b, g = rand_tokens(rng, n, U, dk, dv, kda)
    _, o = orc.recurrence(dense, q, k, v, b, g)
    o3 = orc.replay_output(blob, *entries_from_tokens(q, k, v, b, g), q[-1])
    np.testing.assert_allclose(o3, o[-1], rtol=1e-12, atol=1e-12 * np.abs(o[-1]).max())


@pytest.mark.parametrize("kda", [False, True])
def test_window_closed_form_exact(orc, kda):
    # exact arithmetic: S_n q from the explicit sum of matrix products equals
    # the step-by-step explicit-matrix run; the oracle's reverse replay agrees
    rng = np.random.default_rng(40 + kda)
    d, n = 4, 4
    S0 = rng.integers(-6, 7, (d, d))
    toks = []
    for _ in range(n):
        q = rng.integers(-8, 9, d) / 4.0
        k = rng.integers(-2, 3, d) / 2.0
        v = rng.integers(-8, 9, d) / 4.0
        beta = rng.integers(0, 5) / 4.0
        gg = rng.integers(1, 5, d) / 4.0 if kda else rng.integers(1, 5) / 4.0
        toks.append((q, k, v, beta, gg))
    ft = [(exact.frac_vector(q), exact.frac_vector(k), exact.frac_vector(v), F(bt),
           exact.frac_vector(gg) if kda else F(gg)) for (q, k, v, bt, gg) in toks]
    _, outs = exact.dense_product_run(exact.frac_matrix(S0), ft)
    closed = exact.explicit_window_output(exact.frac_matrix(S0), ft, ft[-1][0])
    assert closed == outs[-1]
    blob = exact_blob(orc, S0[None])
    arr = lambda i: np.array([t[i] for t in toks], np.float32)[None]
    bg = arr(4)
    o3 = orc.replay_output(blob, arr(1), arr(2), arr(3), bg, np.array(toks[-1][0], np.float32)[None])
    np.testing.assert_allclose(o3[0], [float(x) for x in closed], rtol=0, atol=1e-12)


def test_golden_2x2_replay(orc):
    g = parse_golden("delta_rule_2x2.txt")
    blob = exact_blob(orc, np.array(g["S0"], float).reshape(1, 2, 2))
    get = lambda key, t: np.array(g[f"t{t}.{key}"], np.float32)
    bk = np.stack([get("k", t) for t in (1, 2, 3)])[None]
    bv = np.stack([get("v", t) for t in (1, 2, 3)])[None]
    bb = np.array([get("beta", t)[0] for t in (1, 2, 3)], np.float32)[None]
    ba = np.stack([get("a", t) for t in (1, 2, 3)])[None]
    o = orc.replay_output(blob, bk, bv, bb, ba, get("q", 3)[None])
    np.testing.assert_allclose(o[0], np.array(g["t3.o"], float), atol=1e-6)


@pytest.mark.parametrize("kda", [False, True])
def test_windowed_run_without_boundaries_is_plain_recurrence(orc, kda):
    # with no boundary inside the run and a start state the stored form holds
    # exactly (zero), the windowed form reproduces the plain recurrence bitwise
    rng = np.random.default_rng(50 + kda)
    U, d, T = 4, 8, 20
    q, k, v, b, g = rand_tokens(rng, T, U, d, d, kda)
    _, o1 = orc.recurrence(np.zeros((U, d, d)), q, k, v, b, g)
    o2 = orc.windowed_run(np.zeros((U, d, d)), q, k, v, b, g, W=T + 1, n_c=2)
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("kda", [False, True])
def test_windowed_run_is_the_composition(orc, kda):
    # O2 = quantize at start, run W tokens unquantized, requantize, ... with a
    # forced partial flush for one unit
    rng = np.random.default_rng(60 + kda)
    U, d, T, W, n_c = 3, 8, 23, 6, 2
    S0 = rng.standard_normal((U, d, d))
    q, k, v, b, g = rand_tokens(rng, T, U, d, d, kda)
    force_at = np.array([-1, 3, -1], np.int32)
    o2 = orc.windowed_run(S0, q, k, v, b, g, W=W, n_c=n_c, force_at=force_at)
    for u in range(U):
        S = orc.dequant(orc.qz(S0[u:u + 1], n_c)[0])
        fill = 0
        for t in range(T):
            S, o = orc.recurrence(S, q[t:t + 1, u:u + 1], k[t:t + 1, u:u + 1], v[t:t + 1, u:u + 1],
                                  b[t:t + 1, u:u + 1], g[t:t + 1, u:u + 1])
            np.testing.assert_array_equal(o[0, 0], o2[t, u])
            fill += 1
            if fill == W or force_at[u] == t:
                S = orc.dequant(orc.qz(S, n_c)[0])
                fill = 0


def test_windowing_beats_per_token_quantization(orc):
    # not a pin of the pages' numbers (they print none): the per-token
    # ablation accumulates rounding error, one requantization per window less
    rng = np.random.default_rng(70)
    U, d, T = 8, 32, 128
    S0 = np.zeros((U, d, d))
    q, k, v, b, g = rand_tokens(rng, T, U, d, d, False)
    g[:] = rng.uniform(0.97, 1.0, g.shape)
    _, ref = orc.recurrence(S0, q, k, v, b, g)
    lq = orc.windowed_run(S0, q, k, v, b, g, W=32, n_c=2)
    naive = orc.windowed_run(S0, q, k, v, b, g, W=1, n_c=0, smooth=False)
    err = lambda o: np.linalg.norm(o - ref) / np.linalg.norm(ref)
    assert err(lq) < err(naive)


def test_golden_naive_per_token_2x2(orc):
    # the naive per-token ablation (W = 1, no compensators, no smoothing) over
    # two tokens, against the hand-worked run in the golden file
    g = parse_golden("naive_per_token_2x2.txt")
    S0 = np.array(g["S0"], float).reshape(1, 2, 2)
    tok = lambda key, t, n: np.array(g[f"t{t}.{key}"], np.float32).reshape(n)
    q = np.stack([tok("q", t, (1, 2)) for t in (1, 2)])
    k = np.stack([tok("k", t, (1, 2)) for t in (1, 2)])
    v = np.stack([tok("v", t, (1, 2)) for t in (1, 2)])
    b = np.stack([tok("beta", t, (1,)) for t in (1, 2)])
    a = np.stack([tok("alpha", t, (1,)) for t in (1, 2)])
    o, S_end = orc.windowed_run(S0, q, k, v, b, a, W=1, n_c=0, smooth=False, want_state=True)
    assert o[0, 0].tolist() == [float(x) for x in g["t1.o"]]
    sig = [np.float32(float(x) / float(y)) for x, y in (r.split("/") for r in g["t1.sigma_ratio"])]
    codes = [int(x) for x in g["t1.codes"]]
    want_S1 = np.array([[codes[0] * float(sig[0]), codes[1] * float(sig[0])],
                        [codes[2] * float(sig[1]), codes[3] * float(sig[1])]])
    np.testing.assert_array_equal(S_end[0], want_S1)  # token 2 leaves the requantized state as is
    c2 = [int(x) for x in g["t2.o_codes"]]
    assert o[1, 0].tolist() == [c2[0] * float(sig[0]), c2[1] * float(sig[1])]
