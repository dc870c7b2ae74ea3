"""Pins of oracle.transition, the prefill's final state as an affine map P S + Q of its initial
state S.  Each pin is a fact that does not come from the oracle's own code path: the state the
recurrence reaches from a random S, the explicit product of the per-row factors
(I - beta k k^T) diag(alpha), the matrix determinant lemma, the composition of two segments, and
the closed form at beta = 0.  A slip in P (decay on the wrong side, a dropped beta, a transposed
factor, the wrong row order) or in Q fails at least one of them."""
import numpy as np

import oracle


def _inputs(B, T, H, D, seed, gate_lo=-2.0, beta_hi=1.0, key_norm=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, H, D))
    k *= key_norm / np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, D))
    gate = rng.uniform(gate_lo, 0.0, (B, T, H, D))
    beta = rng.uniform(0.0, beta_hi, (B, T, H))
    f = lambda a: a.astype(np.float32)
    return f(q), f(k), f(v), f(gate), f(beta)


def test_affine_in_the_initial_state():
    q, k, v, gate, beta = _inputs(2, 37, 3, 16, seed=1)
    P, Q = oracle.transition(q, k, v, gate, beta)
    rng = np.random.default_rng(2)
    for _ in range(3):
        S = rng.standard_normal((2, 3, 16, 16))
        _, st, _, _ = oracle.serial(q, k, v, gate, beta, S)
        np.testing.assert_allclose(oracle.apply_transition(P, Q, S), st, rtol=0, atol=1e-12)


def test_product_of_row_factors():
    # P = A_T ... A_1 with A_t = (I - beta_t k_t k_t^T) diag(exp(gate_t)), later rows on the left
    B, T, H, D = 1, 9, 2, 8
    q, k, v, gate, beta = _inputs(B, T, H, D, seed=3, beta_hi=1.5)
    P, _ = oracle.transition(q, k, v, gate, beta)
    for h in range(H):
        M = np.eye(D)
        for t in range(T):
            kk = k[0, t, h].astype(np.float64)
            A = (np.eye(D) - float(beta[0, t, h]) * np.outer(kk, kk)) @ np.diag(np.exp(gate[0, t, h].astype(np.float64)))
            M = A @ M
        np.testing.assert_allclose(P[0, h], M, rtol=0, atol=1e-13)


def test_determinant_lemma():
    # det(I - beta k k^T) = 1 - beta |k|^2, det diag(alpha) = prod alpha: det P is their product
    B, T, H, D = 2, 12, 2, 6
    q, k, v, gate, beta = _inputs(B, T, H, D, seed=4, gate_lo=-0.5, beta_hi=0.9)
    P, _ = oracle.transition(q, k, v, gate, beta)
    kk = k.astype(np.float64)
    expect = np.prod(1.0 - beta.astype(np.float64) * np.sum(kk * kk, axis=-1), axis=1) * \
        np.exp(np.sum(gate.astype(np.float64), axis=(1, 3)))
    np.testing.assert_allclose(np.linalg.det(P), expect, rtol=1e-11, atol=0)


def test_segments_compose():
    q, k, v, gate, beta = _inputs(1, 50, 2, 12, seed=5)
    P, Q = oracle.transition(q, k, v, gate, beta)
    cut = 19
    P1, Q1 = oracle.transition(*(a[:, :cut] for a in (q, k, v, gate, beta)))
    P2, Q2 = oracle.transition(*(a[:, cut:] for a in (q, k, v, gate, beta)))
    np.testing.assert_allclose(oracle.apply_transition(P2, None, P1), P, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.apply_transition(P2, Q2, Q1), Q, rtol=0, atol=1e-12)


def test_beta0_is_pure_decay():
    # no updates: every key row decays by the product of its alphas and the values never enter
    q, k, v, gate, beta = _inputs(2, 15, 2, 10, seed=6)
    beta[:] = 0.0
    P, Q = oracle.transition(q, k, v, gate, beta)
    decay = np.exp(np.sum(gate.astype(np.float64), axis=1))  # [B][H][D]
    for b in range(2):
        for h in range(2):
            np.testing.assert_allclose(P[b, h], np.diag(decay[b, h]), rtol=1e-13, atol=0)
    np.testing.assert_array_equal(Q, 0.0)


def test_values_enter_only_q():
    q, k, v, gate, beta = _inputs(1, 20, 2, 8, seed=7)
    P, Q = oracle.transition(q, k, v, gate, beta)
    P2, Q2 = oracle.transition(q, k, 2.0 * v, gate, beta)
    np.testing.assert_array_equal(P2, P)
    np.testing.assert_allclose(Q2, 2.0 * Q, rtol=0, atol=1e-13)
