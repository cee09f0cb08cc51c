"""Pins of the oracle's plain recurrence (O1) against closed forms, invariants,
an explicit dense-matrix formulation in exact arithmetic and a hand-derived
worked example.  CPU only.

The recurrence is the gated delta rule named (not printed) on the arXiv
2609.38166 abstract page; its orientation and gate placement are the readings
these invariants fix.
"""
import os
from fractions import Fraction as F

import numpy as np
import pytest

from oracle import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def parse_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = val.split()
    return out


def rand_tokens(rng, T, U, dk, dv, kda, unit_k=True, beta=None, gate=None):
    q = rng.standard_normal((T, U, dk)).astype(np.float32)
    k = rng.standard_normal((T, U, dk))
    if unit_k:
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    k = k.astype(np.float32)
    v = rng.standard_normal((T, U, dv)).astype(np.float32)
    b = rng.uniform(0, 1, (T, U)).astype(np.float32) if beta is None else np.full((T, U), beta, np.float32)
    gshape = (T, U, dk) if kda else (T, U)
    g = rng.uniform(0.8, 1.0, gshape).astype(np.float32) if gate is None else np.full(gshape, gate, np.float32)
    return q, k, v, b, g


@pytest.mark.parametrize("kda", [False, True])
def test_beta0_gate1_keeps_state_bitwise(orc, kda):
    rng = np.random.default_rng(1)
    S = rng.standard_normal((3, 8, 6))
    q, k, v, b, g = rand_tokens(rng, 5, 3, 6, 8, kda, beta=0.0, gate=1.0)
    S1, o = orc.recurrence(S, q, k, v, b, g)
    assert np.array_equal(S1, S)
    # o_t = S q_t exactly: the same sums in the same order as a plain matvec loop
    ref = np.einsum("uij,tuj->tui", S, q.astype(np.float64))
    np.testing.assert_allclose(o, ref, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("kda", [False, True])
def test_beta1_unit_key_writes_value(orc, kda):
    # S_t k_t = v_t after the update, for any gate (gate != 1 so that a gate
    # applied after the correction would fail this)
    rng = np.random.default_rng(2)
    for _ in range(5):
        S = rng.standard_normal((4, 7, 9)) * 3
        q, k, v, b, g = rand_tokens(rng, 1, 4, 9, 7, kda, beta=1.0)
        k = exact_unit_keys(rng, 1, 4, 9)
        g = (g * 0 + rng.uniform(0.3, 0.9, g.shape)).astype(np.float32)
        S1, _ = orc.recurrence(S, q, k, v, b, g)
        Sk = np.einsum("uij,uj->ui", S1, k[0].astype(np.float64))
        np.testing.assert_allclose(Sk, v[0], rtol=0, atol=1e-13 * np.abs(S).max())


def test_beta0_pure_decay(orc):
    rng = np.random.default_rng(3)
    S = rng.standard_normal((2, 5, 6))
    # GDN: S_n = (prod alpha) S_0
    q, k, v, b, g = rand_tokens(rng, 7, 2, 6, 5, False, beta=0.0)
    Sn, _ = orc.recurrence(S, q, k, v, b, g)
    gam = np.prod(g.astype(np.float64), axis=0)
    np.testing.assert_allclose(Sn, S * gam[:, None, None], rtol=1e-14)
    # KDA: S_n = S_0 Diag(prod a) -- the gate scales key channels (columns)
    q, k, v, b, g = rand_tokens(rng, 7, 2, 6, 5, True, beta=0.0)
    Sn, _ = orc.recurrence(S, q, k, v, b, g)
    Gam = np.prod(g.astype(np.float64), axis=0)  # [U, dk]
    np.testing.assert_allclose(Sn, S * Gam[:, None, :], rtol=1e-14)


@pytest.mark.parametrize("kda", [False, True])
def test_first_token_from_zero(orc, kda):
    # S_1 = beta v k^T and o_1 = beta v (k . q): the output sees its own token
    rng = np.random.default_rng(4)
    q, k, v, b, g = rand_tokens(rng, 1, 3, 5, 4, kda, unit_k=False)
    S1, o = orc.recurrence(np.zeros((3, 4, 5)), q, k, v, b, g)
    b64 = b[0].astype(np.float64)
    ref = b64[:, None, None] * v[0].astype(np.float64)[:, :, None] * k[0].astype(np.float64)[:, None, :]
    np.testing.assert_allclose(S1, ref, rtol=1e-15, atol=0)
    kq = np.einsum("uj,uj->u", k[0].astype(np.float64), q[0].astype(np.float64))
    np.testing.assert_allclose(o[0], b64[:, None] * v[0] * kq[:, None], rtol=1e-13, atol=1e-15)


def test_householder_beta2_preserves_row_norms(orc):
    rng = np.random.default_rng(5)
    S = rng.standard_normal((3, 6, 8))
    q, k, v, b, g = rand_tokens(rng, 9, 3, 8, 6, False, beta=2.0, gate=1.0)
    k = exact_unit_keys(rng, 9, 3, 8)
    v[:] = 0
    Sn, _ = orc.recurrence(S, q, k, v, b, g)
    np.testing.assert_allclose(np.linalg.norm(Sn, axis=2), np.linalg.norm(S, axis=2), rtol=1e-13)


def test_channel_gate_uniform_equals_scalar_gate(orc):
    rng = np.random.default_rng(6)
    S = rng.standard_normal((3, 6, 7))
    q, k, v, b, g = rand_tokens(rng, 11, 3, 7, 6, False)
    gc = np.repeat(g[:, :, None], 7, axis=2)
    S1, o1 = orc.recurrence(S, q, k, v, b, g)
    S2, o2 = orc.recurrence(S, q, k, v, b, gc)
    assert np.array_equal(S1, S2) and np.array_equal(o1, o2)


def exact_unit_keys(rng, T, U, dk):
    """Keys with |k| = 1 exactly in binary: +-1/2 on 4 channels or +-1/4 on 16."""
    k = np.zeros((T, U, dk), np.float32)
    for t in range(T):
        for u in range(U):
            m = 16 if dk >= 16 and rng.integers(0, 2) else 4
            pos = rng.choice(dk, m, replace=False)
            k[t, u, pos] = rng.choice([-1.0, 1.0], m) / np.sqrt(m)
    return k


def _dyadic(rng, shape, scale=8):
    return rng.integers(-scale * 4, scale * 4 + 1, shape) / 4.0


@pytest.mark.parametrize("kda", [False, True])
def test_matches_explicit_dense_products_exactly(orc, kda):
    # dyadic inputs, no rounding anywhere in exact arithmetic; the fp64 oracle
    # must agree to rounding error
    rng = np.random.default_rng(7 + kda)
    d, T = 4, 5
    S0 = _dyadic(rng, (d, d))
    toks = []
    for _ in range(T):
        q = _dyadic(rng, d)
        k = _dyadic(rng, d, 1)
        v = _dyadic(rng, d)
        beta = rng.integers(0, 5) / 4.0
        g = (rng.integers(1, 5, d) / 4.0) if kda else rng.integers(1, 5) / 4.0
        toks.append((q, k, v, beta, g))
    ftoks = [(exact.frac_vector(q), exact.frac_vector(k), exact.frac_vector(v), F(beta),
              exact.frac_vector(g) if kda else F(g)) for (q, k, v, beta, g) in toks]
    S_ex, o_ex = exact.dense_product_run(exact.frac_matrix(S0), ftoks)
    qa = np.array([t[0] for t in toks], np.float32)[:, None]
    ka = np.array([t[1] for t in toks], np.float32)[:, None]
    va = np.array([t[2] for t in toks], np.float32)[:, None]
    ba = np.array([t[3] for t in toks], np.float32)[:, None]
    ga = (np.array([t[4] for t in toks], np.float32)[:, None] if kda
          else np.array([t[4] for t in toks], np.float32)[:, None])
    S1, o = orc.recurrence(S0[None], qa, ka, va, ba, ga)
    S_ex_f = np.array([[float(x) for x in row] for row in S_ex])
    scale = max(1.0, np.abs(S_ex_f).max())
    np.testing.assert_allclose(S1[0], S_ex_f, rtol=0, atol=1e-12 * scale)
    for t in range(T):
        np.testing.assert_allclose(o[t, 0], [float(x) for x in o_ex[t]], rtol=0, atol=1e-12 * scale)


def test_golden_2x2_worked_example(orc):
    g = parse_golden("delta_rule_2x2.txt")
    S = np.array(g["S0"], np.float64).reshape(1, 2, 2)
    for t in (1, 2, 3):
        p = f"t{t}."
        q = np.array(g[p + "q"], np.float32).reshape(1, 1, 2)
        k = np.array(g[p + "k"], np.float32).reshape(1, 1, 2)
        v = np.array(g[p + "v"], np.float32).reshape(1, 1, 2)
        b = np.array(g[p + "beta"], np.float32).reshape(1, 1)
        a = np.array(g[p + "a"], np.float32).reshape(1, 1, 2)
        S, o = orc.recurrence(S, q, k, v, b, a)
        np.testing.assert_allclose(S[0].ravel(), np.array(g[p + "S"], float), atol=1e-6)
        np.testing.assert_allclose(o[0, 0], np.array(g[p + "o"], float), atol=1e-6)
