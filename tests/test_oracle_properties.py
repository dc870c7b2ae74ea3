"""Randomised properties of the oracle (CPU, hypothesis): the chunked WY/UT form equals the serial
recurrence over random sizes, head dimensions, chunk widths, gates and betas; a walk split in two equals
the whole walk bit for bit, and so does every snapshot; the front end split at any row equals the whole.
These hold for any correct implementation of the recurrence, so they pin the oracle against slips that
only show up at sizes the fixed-shape pins do not reach."""
import numpy as np
from hypothesis import given, settings, strategies as st

import kda_inputs as ki
import oracle

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True)


def _draw_inputs(seed, B, T, H, D, gate_lo, beta_lo, beta_hi, key_scale):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, H, D))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k *= key_scale / np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, D))
    gate = rng.uniform(gate_lo, 0.0, (B, T, H, D))
    beta = rng.uniform(beta_lo, beta_hi, (B, T, H))
    state = 0.1 * rng.standard_normal((B, H, D, D))
    f = lambda a: a.astype(np.float32)
    return f(q), f(k), f(v), f(gate), f(beta), state


shapes = st.tuples(st.integers(0, 10 ** 6), st.integers(1, 2), st.integers(1, 90), st.integers(1, 3),
                   st.sampled_from([1, 2, 3, 8, 16]))


@SETTINGS
@given(shape=shapes, chunk=st.integers(1, 40), gate_lo=st.floats(-6.0, 0.0),
       beta=st.tuples(st.floats(-0.5, 0.5), st.floats(0.5, 1.5)), key_scale=st.floats(0.1, 1.0))
def test_chunked_equals_serial_random(shape, chunk, gate_lo, beta, key_scale):
    seed, B, T, H, D = shape
    q, k, v, gate, b, s0 = _draw_inputs(seed, B, T, H, D, gate_lo, beta[0], beta[1], key_scale)
    out_s, st_s, _, _ = oracle.serial(q, k, v, gate, b, s0)
    out_c, st_c, _ = oracle.chunked(q, k, v, gate, b, s0, chunk)
    scale = max(1.0, float(np.abs(out_s).max()), float(np.abs(st_s).max()))
    assert np.abs(out_c - out_s).max() <= 1e-10 * scale
    assert np.abs(st_c - st_s).max() <= 1e-10 * scale


@SETTINGS
@given(shape=shapes, cut=st.floats(0.0, 1.0), n_snap=st.integers(0, 90))
def test_split_walk_and_snapshots_equal_the_whole_walk(shape, cut, n_snap):
    seed, B, T, H, D = shape
    q, k, v, gate, b, s0 = _draw_inputs(seed, B, T, H, D, -5.0, 0.0, 1.0, 1.0)
    n_snap = min(n_snap, T)
    out, st_all, snaps, _ = oracle.serial(q, k, v, gate, b, s0, n_snap=n_snap)
    t1 = int(round(cut * T))
    if 0 < t1 < T:
        o1, s1, _, _ = oracle.serial(q[:, :t1], k[:, :t1], v[:, :t1], gate[:, :t1], b[:, :t1], s0)
        o2, s2, _, _ = oracle.serial(q[:, t1:], k[:, t1:], v[:, t1:], gate[:, t1:], b[:, t1:], s1)
        np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), out)
        np.testing.assert_array_equal(s2, st_all)
    for t in range(n_snap):
        _, st_t, _, _ = oracle.serial(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], gate[:, :t + 1], b[:, :t + 1], s0)
        np.testing.assert_array_equal(snaps[t], st_t)


@SETTINGS
@given(seed=st.integers(0, 10 ** 6), B=st.integers(1, 3), T=st.integers(2, 12), H=st.integers(1, 2),
       K=st.integers(1, 4), cut=st.integers(1, 11))
def test_front_end_split_equals_the_whole(seed, B, T, H, K, cut):
    cut = min(cut, T - 1)
    x = ki.front_end_inputs(seed, B, T, H, K)
    q, k, v, s, _ = oracle.decode_front_end(x["qkv"], x["conv_w"], x["conv_state"], H, 1e-6)
    q1, k1, v1, s1, _ = oracle.decode_front_end(x["qkv"][:, :cut], x["conv_w"], x["conv_state"], H, 1e-6)
    q2, k2, v2, s2, _ = oracle.decode_front_end(x["qkv"][:, cut:], x["conv_w"], s1, H, 1e-6)
    for whole, a, b2 in ((q, q1, q2), (k, k1, k2), (v, v1, v2)):
        np.testing.assert_array_equal(np.concatenate([a, b2], axis=1), whole)
    np.testing.assert_array_equal(s2, s)
