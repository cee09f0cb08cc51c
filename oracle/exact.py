"""Exact rational-arithmetic checks for tiny states (test infrastructure only).

These are independent formulations used to pin ``lq_oracle.c``, not copies of
it:

* ``dense_product_run`` builds every transition A_t = Diag(g_t)(I - beta_t k_t k_t^T)
  as an explicit matrix and multiplies, S_t = S_{t-1} A_t + beta_t v_t k_t^T,
  o_t = S_t q_t -- the matrix form of the gated delta rule that the pages name
  for GDN and KDA (arXiv 2609.38166 abstract, "Abstract (arXiv)" section of the
  mlsanity.com paper page), with the orientation fixed by the invariants
  "beta = 0 with gate = 1 keeps S" and "beta = 1 with a unit key gives S k = v".
* ``explicit_window_output`` writes the state after a window as the closed sum
  S_n = S_0 A_1...A_n + sum_i beta_i v_i k_i^T A_{i+1}...A_n (matrix products of
  the explicit A_i) and returns S_n q -- the "fixed state plus buffered updates"
  reading of the abstract, without any reverse pass.
* ``qz_bruteforce`` chooses compensator lines by enumerating every subset of
  the d_v + d_k candidate lines and each code by scanning all 255 codes.

Everything is ``fractions.Fraction``; inputs are dyadic so that no step rounds.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction as F

import numpy as np


def frac_matrix(a):
    a = np.asarray(a)
    return [[F(float(x)) for x in row] for row in a]


def frac_vector(a):
    return [F(float(x)) for x in np.asarray(a).ravel()]


def matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][t] * B[t][j] for t in range(m)), F(0)) for j in range(p)] for i in range(n)]


def matvec(A, x):
    return [sum((A[i][j] * x[j] for j in range(len(x))), F(0)) for i in range(len(A))]


def outer(a, b):
    return [[x * y for y in b] for x in a]


def add(A, B):
    return [[A[i][j] + B[i][j] for j in range(len(A[0]))] for i in range(len(A))]


def scale(A, c):
    return [[c * x for x in row] for row in A]


def identity(n):
    return [[F(int(i == j)) for j in range(n)] for i in range(n)]


def transition(k, beta, g):
    """A = Diag(g) (I - beta k k^T) as an explicit d_k x d_k matrix."""
    d = len(k)
    g = g if isinstance(g, list) else [g] * d
    B = add(identity(d), scale(outer(k, k), -beta))
    return [[g[i] * B[i][j] for j in range(d)] for i in range(d)]


def dense_product_run(S0, toks):
    """S_t = S_{t-1} A_t + beta v k^T with explicit A_t; returns (S_T, [o_t])."""
    S = [row[:] for row in S0]
    outs = []
    for (q, k, v, beta, g) in toks:
        S = add(matmul(S, transition(k, beta, g)), scale(outer(v, k), beta))
        outs.append(matvec(S, q))
    return S, outs


def explicit_window_output(S0, toks, q):
    """S_n q with S_n = S0 A_1..A_n + sum_i beta_i v_i k_i^T A_{i+1}..A_n."""
    n = len(toks)
    d = len(S0[0])
    A = [transition(k, beta, g) for (_, k, _, beta, g) in toks]

    def prod(a, b):  # A_a ... A_b (1-based, inclusive), identity if empty
        P = identity(d)
        for i in range(a, b + 1):
            P = matmul(P, A[i - 1])
        return P

    S = matmul(S0, prod(1, n))
    for i in range(1, n + 1):
        _, k, v, beta, _ = toks[i - 1]
        S = add(S, scale(matmul(outer(v, k), prod(i + 1, n)), beta))
    return matvec(S, q)


# ---------------------------------------------------------------------------
# Brute-force quantizer checks
# ---------------------------------------------------------------------------

def best_subset(scores, n_c):
    """Subset of n_c candidate indices with the largest score sum; among equal
    sums the lexicographically smallest ascending index tuple."""
    best = None
    for sub in itertools.combinations(range(len(scores)), n_c):
        s = sum((scores[i] for i in sub), F(0))
        if best is None or s > best[0]:
            best = (s, sub)
    return list(best[1])


def line_scores(S):
    dv, dk = len(S), len(S[0])
    rows = [sum((S[i][j] * S[i][j] for j in range(dk)), F(0)) for i in range(dv)]
    cols = [sum((S[i][j] * S[i][j] for i in range(dv)), F(0)) for j in range(dk)]
    return rows + cols


def nearest_code(x):
    """argmin over c in [-127, 127] of |x - c|; an exact half goes to the even code."""
    best = None
    for c in range(-127, 128):
        d = abs(x - c)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]


def f32(x) -> float:
    return float(np.float32(x))


def sqrt_f32(a: F) -> float:
    """fp32 rounding of the fp64 square root of a (a is an fp64 value here)."""
    return f32(math.sqrt(float(a)))
