"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

The pages print no numeric example, so each pin is a closed form, an exact
rational brute force in a different (matrix) formulation, a hand-worked case,
or an invariant of the gated delta rule.  Each is chosen to fail on a
plausible slip: a dropped beta, a sign, the decay on the wrong axis or after
the update, a transposed read-out, the pre-update state in the output, an
off-by-one chunk, pad rows leaking into the result.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import kda_inputs as ki
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def _inputs(B, T, H, D, gate_lo=-5.0, state_std=0.02, seed=0, unit_k=True, rows=None):
    rng = np.random.default_rng(seed)
    rows = T if rows is None else rows
    q = rng.standard_normal((B, rows, H, D))
    k = rng.standard_normal((B, rows, H, D))
    if unit_k:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, rows, H, D))
    gate = rng.uniform(gate_lo, 0.0, (B, rows, H, D))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, rows, H))))
    state = state_std * rng.standard_normal((B, H, D, D))
    f = lambda a: a.astype(np.float32)
    return f(q), f(k), f(v), f(gate), f(beta), state


def test_hand_worked_d2():
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_d2.json")))
    D = g["D"]
    arr = lambda key: np.array(g[key], dtype=np.float32).reshape(1, -1, 1, D)
    beta = np.array(g["beta"], dtype=np.float32).reshape(1, -1, 1)
    st0 = np.array(g["state0"], dtype=np.float64).reshape(1, 1, D, D)
    out, st, _, _ = oracle.serial(arr("q"), arr("k"), arr("v"), arr("gate"), beta, st0)
    np.testing.assert_array_equal(out[0, :, 0, :], np.array(g["expected_out"]))
    np.testing.assert_array_equal(st[0, 0], np.array(g["expected_state"]))


def test_beta0_gate0_leaves_state_and_reads_out():
    q, k, v, gate, beta, st0 = _inputs(2, 5, 3, 128)
    gate[:] = 0.0
    beta[:] = 0.0
    out, st, _, _ = oracle.serial(q, k, v, gate, beta, st0)
    np.testing.assert_array_equal(st, st0)  # exactly unchanged
    expect = np.einsum("bthi,bhij->bthj", q.astype(np.float64), st0)
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-14)


def _exact_unit_keys(rng, B, T, H, D):
    """Keys with 16 entries of +-1/4: the squared norm is exactly 1 in binary."""
    k = np.zeros((B, T, H, D), dtype=np.float32)
    for idx in np.ndindex(B, T, H):
        pos = rng.choice(D, 16, replace=False)
        k[idx][pos] = rng.choice([-0.25, 0.25], 16)
    return k


def test_beta1_unit_key_fixed_point():
    """beta = 1, |k| = 1: after every update S^T k = v; with q = k the output is v."""
    rng = np.random.default_rng(7)
    B, T, H, D = 1, 6, 2, 128
    _, _, v, gate, beta, st0 = _inputs(B, T, H, D, seed=3)
    k = _exact_unit_keys(rng, B, T, H, D)
    beta[:] = 1.0
    out, st, snaps, _ = oracle.serial(k, k, v, gate, beta, st0, n_snap=T)
    for t in range(T):
        for h in range(H):
            np.testing.assert_allclose(snaps[t, 0, h].T @ k[0, t, h].astype(np.float64), v[0, t, h], rtol=0,
                                       atol=1e-12)
    np.testing.assert_allclose(out, v.astype(np.float64), rtol=0, atol=1e-12)


def test_zero_state_single_token_closed_form():
    """S0 = 0, T = 1: S = beta k v^T and out = beta (q.k) v (no scale, post-update)."""
    q, k, v, gate, beta, _ = _inputs(2, 1, 3, 128, seed=11)
    st0 = np.zeros((2, 3, 128, 128))
    out, st, _, _ = oracle.serial(q, k, v, gate, beta, st0)
    q64, k64, v64, b64 = (a.astype(np.float64) for a in (q, k, v, beta))
    for b in range(2):
        for h in range(3):
            S = b64[b, 0, h] * np.outer(k64[b, 0, h], v64[b, 0, h])
            np.testing.assert_allclose(st[b, h], S, rtol=0, atol=1e-15)
            o = b64[b, 0, h] * (q64[b, 0, h] @ k64[b, 0, h]) * v64[b, 0, h]
            np.testing.assert_allclose(out[b, 0, h], o, rtol=0, atol=1e-14)


def test_basis_keys_row_ema():
    """k = e_i: row i becomes (1-beta) alpha_i S_i + beta v; other rows only decay by their own alpha."""
    B, T, H, D = 1, 4, 1, 128
    q, _, v, gate, beta, st0 = _inputs(B, T, H, D, seed=5)
    rows = [3, 77, 3, 127]
    k = np.zeros((B, T, H, D), dtype=np.float32)
    for t, i in enumerate(rows):
        k[0, t, 0, i] = 1.0
    out, st, snaps, _ = oracle.serial(q, k, v, gate, beta, st0, n_snap=T)
    S = st0[0, 0].copy()
    for t, i in enumerate(rows):
        alpha = np.array([math.exp(float(g)) for g in gate[0, t, 0]])
        b = float(beta[0, t, 0])
        new = alpha[:, None] * S
        new[i] = (1.0 - b) * alpha[i] * S[i] + b * v[0, t, 0].astype(np.float64)
        np.testing.assert_allclose(snaps[t, 0, 0], new, rtol=1e-13, atol=1e-15)
        S = snaps[t, 0, 0]


def test_scalar_head_decay_before_update():
    """D = 1: S' = alpha S (1 - beta k^2) + beta k v, out = q S'.  Decay-after-update or
    a pre-update read-out give different numbers for these inputs."""
    rng = np.random.default_rng(9)
    T = 7
    q = rng.uniform(-1, 1, (1, T, 1, 1)).astype(np.float32)
    k = rng.uniform(-1, 1, (1, T, 1, 1)).astype(np.float32)
    v = rng.uniform(-1, 1, (1, T, 1, 1)).astype(np.float32)
    gate = rng.uniform(-2, 0, (1, T, 1, 1)).astype(np.float32)
    beta = rng.uniform(0, 1, (1, T, 1)).astype(np.float32)
    s0 = np.array([[[[0.7]]]])
    out, st, _, _ = oracle.serial(q, k, v, gate, beta, s0)
    S = 0.7
    for t in range(T):
        a = math.exp(float(gate[0, t, 0, 0]))
        kk, vv, bb, qq = (float(x) for x in (k[0, t, 0, 0], v[0, t, 0, 0], beta[0, t, 0], q[0, t, 0, 0]))
        S = a * S * (1.0 - bb * kk * kk) + bb * kk * vv
        assert abs(out[0, t, 0, 0] - qq * S) < 1e-14
    assert abs(st[0, 0, 0, 0] - S) < 1e-14


def test_exact_rational_matrix_form():
    """Brute force in exact rationals with the matrix form
    S_t = (I - beta k k^T) diag(a) S_{t-1} + beta k v^T, out_t = S_t^T q_t, D = 3."""
    rng = np.random.default_rng(21)
    D, T = 3, 4
    q, k, v, gate, beta, _ = _inputs(1, T, 1, D, seed=4)
    s0 = (0.5 * rng.standard_normal((1, 1, D, D)))
    out, st, _, _ = oracle.serial(q, k, v, gate, beta, s0)
    F = Fraction
    S = [[F(float(s0[0, 0, i, j])) for j in range(D)] for i in range(D)]
    for t in range(T):
        kt = [F(float(x)) for x in k[0, t, 0]]
        vt = [F(float(x)) for x in v[0, t, 0]]
        qt = [F(float(x)) for x in q[0, t, 0]]
        a = [F(math.exp(float(g))) for g in gate[0, t, 0]]
        bt = F(float(beta[0, t, 0]))
        P = [[(1 if i == m else 0) - bt * kt[i] * kt[m] for m in range(D)] for i in range(D)]
        DS = [[a[m] * S[m][j] for j in range(D)] for m in range(D)]
        S = [[sum(P[i][m] * DS[m][j] for m in range(D)) + bt * kt[i] * vt[j] for j in range(D)]
             for i in range(D)]
        o = [sum(S[i][j] * qt[i] for i in range(D)) for j in range(D)]
        for j in range(D):
            assert abs(out[0, t, 0, j] - float(o[j])) <= 1e-14 * max(1.0, abs(float(o[j])))
    for i in range(D):
        for j in range(D):
            assert abs(st[0, 0, i, j] - float(S[i][j])) <= 1e-14 * max(1.0, abs(float(S[i][j])))


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 100])
def test_chunked_equals_serial(C, T):
    q, k, v, gate, beta, st0 = _inputs(1, T, 2, 128, seed=T * 7 + C)
    out_s, st_s, _, _ = oracle.serial(q, k, v, gate, beta, st0)
    out_c, st_c, _ = oracle.chunked(q, k, v, gate, beta, st0, C)
    assert np.abs(out_c - out_s).max() <= 1e-12 * max(1.0, np.abs(out_s).max())
    assert np.abs(st_c - st_s).max() <= 1e-12 * max(1.0, np.abs(st_s).max())


@pytest.mark.parametrize("pad", [0.0, 1e4, np.inf, -np.inf, np.nan])
def test_pad_rows_are_ignored(pad):
    T, rows = 37, 64
    q, k, v, gate, beta, st0 = _inputs(2, T, 2, 128, seed=2, rows=rows)
    ref = None
    for arr in (q, k, v, gate):
        arr[:, T:] = pad
    beta[:, T:] = pad
    out_s, st_s, _, _ = oracle.serial(q, k, v, gate, beta, st0, T=T)
    out_c, st_c, _ = oracle.chunked(q, k, v, gate, beta, st0, 16, T=T)
    q2, k2, v2, g2, b2 = (a[:, :T].copy() for a in (q, k, v, gate, beta))
    ref_o, ref_s, _, _ = oracle.serial(q2, k2, v2, g2, b2, st0)
    ref_oc, ref_sc, _ = oracle.chunked(q2, k2, v2, g2, b2, st0, 16)
    np.testing.assert_array_equal(out_s, ref_o)
    np.testing.assert_array_equal(st_s, ref_s)
    np.testing.assert_array_equal(out_c, ref_oc)
    np.testing.assert_array_equal(st_c, ref_sc)
    assert ref is None


def test_linear_in_state_and_values():
    """The map is affine with no constant term in (S0, V): F(S0+2S0', V+2V') = F(S0,V) + 2 F(S0',V')."""
    rng = np.random.default_rng(31)
    q, k, _, gate, beta, _ = _inputs(1, 20, 2, 128, seed=8)
    # values on a 2^-10 grid so that V + 2V' is exact in fp32
    V1 = (rng.integers(-2048, 2048, q.shape) / 1024.0).astype(np.float32)
    V2 = (rng.integers(-2048, 2048, q.shape) / 1024.0).astype(np.float32)
    S1 = rng.standard_normal((1, 2, 128, 128)) * 0.02
    S2 = rng.standard_normal((1, 2, 128, 128)) * 0.02
    o1, s1, _, _ = oracle.serial(q, k, V1, gate, beta, S1)
    o2, s2, _, _ = oracle.serial(q, k, V2, gate, beta, S2)
    o3, s3, _, _ = oracle.serial(q, k, (V1 + 2 * V2).astype(np.float32), gate, beta, S1 + 2 * S2)
    np.testing.assert_allclose(o3, o1 + 2 * o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(s3, s1 + 2 * s2, rtol=0, atol=1e-12)


def test_value_column_head_and_sequence_permutation():
    q, k, v, gate, beta, st0 = _inputs(3, 9, 4, 128, seed=13)
    out, st, _, _ = oracle.serial(q, k, v, gate, beta, st0)
    perm = RNG.permutation(128)
    out_p, st_p, _, _ = oracle.serial(q, k, v[..., perm].copy(), gate, beta, st0[..., perm].copy())
    np.testing.assert_array_equal(out_p, out[..., perm])
    np.testing.assert_array_equal(st_p, st[..., perm])
    hp, bp = RNG.permutation(4), RNG.permutation(3)
    sel = lambda a: a[bp][:, :, hp].copy()
    out_h, st_h, _, _ = oracle.serial(sel(q), sel(k), sel(v), sel(gate), beta[bp][:, :, hp].copy(),
                                      st0[bp][:, hp].copy())
    np.testing.assert_array_equal(out_h, out[bp][:, :, hp])
    np.testing.assert_array_equal(st_h, st[bp][:, hp])


def test_continuation_and_snapshots():
    T1, T2 = 23, 41
    q, k, v, gate, beta, st0 = _inputs(2, T1 + T2, 2, 128, seed=17)
    out, st, snaps, _ = oracle.serial(q, k, v, gate, beta, st0, n_snap=5)
    a = lambda x: x[:, :T1].copy()
    b = lambda x: x[:, T1:].copy()
    o1, s1, _, _ = oracle.serial(a(q), a(k), a(v), a(gate), a(beta), st0)
    o2, s2, _, _ = oracle.serial(b(q), b(k), b(v), b(gate), b(beta), s1)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), out)
    np.testing.assert_array_equal(s2, st)
    for t in range(5):
        _, s_t, _, _ = oracle.serial(q[:, :t + 1].copy(), k[:, :t + 1].copy(), v[:, :t + 1].copy(),
                                     gate[:, :t + 1].copy(), beta[:, :t + 1].copy(), st0)
        np.testing.assert_array_equal(snaps[t], s_t)
    # chunked across the same split agrees with serial to rounding
    c1, cs1, _ = oracle.chunked(a(q), a(k), a(v), a(gate), a(beta), st0, 16)
    c2, cs2, _ = oracle.chunked(b(q), b(k), b(v), b(gate), b(beta), cs1, 32)
    assert np.abs(np.concatenate([c1, c2], axis=1) - out).max() < 1e-12
    assert np.abs(cs2 - st).max() < 1e-12


def test_state_norm_bound_long_run():
    """|k| = 1, beta in [0,1], gate <= 0: ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||."""
    T = 300
    q, k, v, gate, beta, st0 = _inputs(1, T, 1, 128, gate_lo=-0.05, seed=19)
    k = _exact_unit_keys(np.random.default_rng(3), 1, T, 1, 128)
    _, _, snaps, _ = oracle.serial(q, k, v, gate, beta, st0, n_snap=T)
    prev = np.linalg.norm(st0[0, 0])
    for t in range(T):
        cur = np.linalg.norm(snaps[t, 0, 0])
        assert cur <= prev + float(beta[0, t, 0]) * np.linalg.norm(v[0, t, 0].astype(np.float64)) + 1e-12
        prev = cur


def test_chunk_stages_match_serial_deltas():
    """Delta of the chunked form equals the per-token delta of the serial map,
    recovered from consecutive serial snapshots as (S_r - diag(a_r) S_{r-1})^T k_r / |k_r|^2."""
    T, C = 40, 32
    q, k, v, gate, beta, st0 = _inputs(1, T, 1, 128, seed=23)
    _, _, snaps, _ = oracle.serial(q, k, v, gate, beta, st0, n_snap=T)
    t0 = 16
    stages = oracle.chunk_stages(q, k, v, gate, beta, snaps[t0 - 1, 0, 0], 0, 0, t0, T - t0)
    for r in range(T - t0):
        t = t0 + r
        a = np.exp(gate[0, t, 0].astype(np.float64))
        kt = k[0, t, 0].astype(np.float64)
        delta = (snaps[t, 0, 0] - a[:, None] * snaps[t - 1, 0, 0]).T @ kt / (kt @ kt)
        np.testing.assert_allclose(stages["Delta"][r], delta, rtol=0, atol=1e-11)
    n = T - t0
    np.testing.assert_allclose(stages["Tinv"] @ (np.eye(n) + stages["A"]), np.eye(n), rtol=0, atol=1e-12)
    np.testing.assert_allclose(stages["S"], snaps[T - 1, 0, 0], rtol=0, atol=1e-12)


def test_generator_is_deterministic_and_continues():
    a = ki.make_batch(1001, 1, 2, 300, -5.0, 0.02)
    b = ki.make_batch(1001, 1, 2, 300, -5.0, 0.02)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    tail = ki.make_batch(1001, 1, 2, 44, -5.0, 0.02, row0=256)
    for key in ("q", "k", "v", "gate", "beta"):
        np.testing.assert_array_equal(tail[key][:, :44], a[key][:, 256:300])
    assert np.all(a["gate"] <= 0) and np.all(a["gate"] >= -5.0)
    assert np.all((a["beta"] > 0) & (a["beta"] < 1))
    np.testing.assert_allclose(np.linalg.norm(a["k"].astype(np.float64), axis=-1), 1.0, atol=1e-6)
