"""The chain-free (WY) window buffer is an exact rewriting of the scalar-gate
delta rule: checked in FP64 against the oracle's plain recurrence.  CPU only.

Within a window that starts from S_hat, with g_t the product of the gates up
to token t (the current one included),
    n_t = beta_t (v_t - g_t S_hat k_t - sum_{i<t} (g_t/g_i) n_i (k_i . k_t)),
    S_t = g_t S_hat + sum_{i<=t} (g_t/g_i) n_i k_i^T,
    o_t = S_t q_t.
The ratios g_t/g_i are formed as the decode forms them: 2 to the sum of log2
of the gates after entry i, each floored at 2^-126, summed newest first.  A
plausible mistake in that reading (the ratio inverted, the current gate left
out, beta applied twice, the sum over i <= t in n_t) fails these checks.
"""
import numpy as np
import pytest

import oracle as orc

FLOOR = -126.0


def _ratios(gates_newest_first_log2, lt):
    """Exclusive running sums of the floored log2 gates, newest first, plus the
    current token's: exponent of g_t / g_i for the m-th newest entry."""
    ex = np.concatenate([[0.0], np.cumsum(gates_newest_first_log2)[:-1]])
    return ex + lt


def nform_window(S_hat, q, k, v, beta, gate):
    """One unit, one window of T tokens: n_t, o_t and the window-end state."""
    T, d = k.shape
    with np.errstate(divide="ignore"):  # log2(0) = -inf, floored like any gate below 2^-126
        lg = np.maximum(np.log2(gate.astype(np.float64)), FLOOR)
    ns, outs = [], []
    for t in range(T):
        # exponents of g_t / g_i for i = t-1, t-2, ..., 0 (newest first), and log2 g_t
        newest_first = lg[:t][::-1]
        exps = _ratios(newest_first, lg[t]) if t > 0 else np.zeros(0)
        log_gt = lg[: t + 1].sum()
        gt = 2.0 ** log_gt
        ratio = (2.0 ** exps)[::-1] if t > 0 else np.zeros(0)  # back to entry order
        kt, qt = k[t].astype(np.float64), q[t].astype(np.float64)
        acc_k = gt * (S_hat @ kt)
        acc_q = gt * (S_hat @ qt)
        for i in range(t):
            ki = k[i].astype(np.float64)
            acc_k = acc_k + ratio[i] * ns[i] * (ki @ kt)
            acc_q = acc_q + ratio[i] * ns[i] * (ki @ qt)
        n_t = float(beta[t]) * (v[t].astype(np.float64) - acc_k)
        ns.append(n_t)
        outs.append(acc_q + n_t * (kt @ qt))
    # window end: T <- g_W S_hat + sum_i (g_W / g_i) n_i k_i^T
    lW = lg.sum()
    S_end = 2.0 ** lW * S_hat
    suffix = np.concatenate([np.cumsum(lg[::-1])[::-1][1:], [0.0]])  # sum of log2 gates after i
    for i in range(T):
        S_end = S_end + 2.0 ** suffix[i] * np.outer(ns[i], k[i].astype(np.float64))
    return np.array(ns), np.array(outs), S_end


def _window(rng, T, d, gate_lo=0.9, gate_hi=1.0):
    q = rng.standard_normal((T, d))
    k = rng.standard_normal((T, d))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, d))
    beta = rng.uniform(0.0, 1.0, T)
    gate = rng.uniform(gate_lo, gate_hi, T)
    S_hat = rng.standard_normal((d, d))
    return [x.astype(np.float32) for x in (q, k, v, beta, gate)] + [S_hat]


def _oracle(S_hat, q, k, v, beta, gate):
    S, o = orc.recurrence(S_hat[None], q[:, None], k[:, None], v[:, None], beta[:, None], gate[:, None])
    return S[0], o[:, 0]


@pytest.mark.parametrize("seed,T,d", [(0, 12, 8), (1, 64, 16), (2, 1, 4), (3, 40, 32)])
def test_nform_matches_the_recurrence(seed, T, d):
    q, k, v, beta, gate, S_hat = _window(np.random.default_rng(seed), T, d)
    _, o, S_end = nform_window(S_hat, q, k, v, beta, gate)
    S_ref, o_ref = _oracle(S_hat, q, k, v, beta, gate)
    assert np.abs(o - o_ref).max() <= 1e-12 * max(1.0, np.abs(o_ref).max())
    assert np.abs(S_end - S_ref).max() <= 1e-12 * max(1.0, np.abs(S_ref).max())


def test_nform_state_at_every_token():
    # S_t from the stored entries alone, at every t, against the recurrence cut there
    rng = np.random.default_rng(7)
    q, k, v, beta, gate, S_hat = _window(rng, 9, 6)
    for t in range(1, 10):
        _, _, S_t = nform_window(S_hat, q[:t], k[:t], v[:t], beta[:t], gate[:t])
        S_ref, _ = _oracle(S_hat, q[:t], k[:t], v[:t], beta[:t], gate[:t])
        assert np.abs(S_t - S_ref).max() <= 1e-12 * max(1.0, np.abs(S_ref).max()), t


def test_nform_extreme_gates():
    # gates of 0 and far below the floor: the floored ratios differ from the
    # exact ones only by terms below 2^-126 of the state, and a zero gate
    # leaves nothing of the entries before it
    rng = np.random.default_rng(11)
    q, k, v, beta, gate, S_hat = _window(rng, 20, 8)
    gate = gate.copy()
    gate[3], gate[4] = 1e-20, 1e-30
    gate[9] = 0.0
    gate[15] = 1e-30
    _, o, S_end = nform_window(S_hat, q, k, v, beta, gate)
    S_ref, o_ref = _oracle(S_hat, q, k, v, beta, gate)
    scale = max(1.0, np.abs(S_ref).max())
    assert np.abs(S_end - S_ref).max() <= 1e-12 * scale
    assert np.abs(o - o_ref).max() <= 1e-12 * max(1.0, np.abs(o_ref).max())


def test_nform_beta_zero_gate_one_leaves_the_state():
    rng = np.random.default_rng(5)
    q, k, v, beta, gate, S_hat = _window(rng, 6, 5)
    beta[:] = 0.0
    gate[:] = 1.0
    ns, o, S_end = nform_window(S_hat, q, k, v, beta, gate)
    assert np.all(ns == 0.0)
    assert np.allclose(S_end, S_hat, rtol=0, atol=0)
    assert np.allclose(o, q.astype(np.float64) @ S_hat.T, rtol=1e-14, atol=1e-14)
