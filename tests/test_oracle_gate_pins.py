"""Pins of the oracle's sigmoid (the beta step) and kda_gate reading (CPU only).

sigmoid is pinned against torch.sigmoid in fp64 and closed forms.  kda_gate follows a reading (the
pages name its inputs, not its formula): lower_bound * sigmoid(exp(a_log[h]) * (g_raw + dt_bias[h, i])).
Its pins are closed forms of that reading, chosen so that a dropped bias, a rate without the
exponential, a bias or rate indexed by the wrong axis, or a sign slip each fail one; the planted
slips at the end check exactly that."""
import math

import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle

H, D = 3, 128


def bits(x):
    return ki.to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_sigmoid_matches_torch_fp64():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(0, 3, 4000), rng.normal(0, 300, 1000), [0.0, -0.0, 1e-300, -1e-300, 745.0, -745.0]])
    ref = torch.sigmoid(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(oracle.sigmoid(x), ref, rtol=1e-15, atol=1e-300)


def test_sigmoid_closed_forms():
    s = oracle.sigmoid
    assert s(0.0) == 0.5
    assert s(np.inf) == 1.0 and s(-np.inf) == 0.0
    assert np.isnan(s(np.nan))
    assert abs(s(math.log(3.0)) - 0.75) < 1e-15            # 1 / (1 + 1/3)
    assert abs(s(-math.log(3.0)) - 0.25) < 1e-15
    x = np.linspace(-40, 40, 801)
    np.testing.assert_allclose(s(x) + s(-x), 1.0, rtol=0, atol=1e-15)   # symmetry
    assert np.all(np.diff(s(x)) >= 0)                       # monotone


def _inputs(seed=3, T=5):
    rng = np.random.default_rng(seed)
    g = rng.normal(0, 2, (2, T, H, D)).astype(np.float32)
    dt = rng.normal(0, 1, (H, D)).astype(np.float32)
    a = rng.normal(0, 1, (H,)).astype(np.float32)
    return bits(g), dt, a


def test_gate_at_the_bias_point_is_half_the_bound():
    """g_raw = -dt_bias makes the sigmoid's argument 0 whatever the rate: gate = lower / 2 exactly."""
    _, dt, a = _inputs()
    dt = oracle.bf16_to_f64(bits(dt)).astype(np.float32)     # dt exactly representable in BF16
    g = bits(np.broadcast_to(-dt, (2, 4, H, D)))
    out = oracle.kda_gate(g, dt, a, -5.0)
    assert np.all(out == -2.5)


def test_gate_rate_is_exp_of_a_log():
    """a_log = ln 2 doubles the argument: with g_raw + dt_bias = ln 3 / 2 the sigmoid is 3/4."""
    x = np.float32(math.log(3.0) / 2)
    g = bits(np.full((1, 1, H, D), x))
    dt = np.zeros((H, D), np.float32)
    xv = float(oracle.bf16_to_f64(g).ravel()[0])
    a = np.full((H,), math.log(2.0), np.float32)
    out = oracle.kda_gate(g, dt, a, -4.0)
    rate = math.exp(float(np.float32(math.log(2.0))))      # exp of a_log as stored (float32), about 2
    expect = -4.0 / (1.0 + math.exp(-rate * xv))
    np.testing.assert_allclose(out, expect, rtol=1e-14)
    assert abs(out.ravel()[0] - (-3.0)) < 0.02               # close to 3/4 of the bound (BF16 input)


def test_gate_limits_and_bounds():
    g, dt, a = _inputs()
    out = oracle.kda_gate(g, dt, a, -5.0)
    assert np.all(out < 0) and np.all(out > -5.0)
    big = bits(np.full((1, 1, H, D), 3e38))
    assert np.allclose(oracle.kda_gate(big, dt, a, -5.0), -5.0)
    small = bits(np.full((1, 1, H, D), -3e38))
    assert np.all(oracle.kda_gate(small, dt, a, -5.0) == -0.0)
    # a vanishing rate (a_log -> -inf) leaves the argument at 0: half the bound
    assert np.all(oracle.kda_gate(g, dt, np.full((H,), -np.inf, np.float32), -5.0) == -2.5)
    # the gate falls monotonically from 0 towards the bound as g_raw grows
    ramp = bits(np.linspace(-20, 20, 4001, dtype=np.float32).reshape(1, -1, 1, 1).repeat(H, 2).repeat(D, 3))
    o = oracle.kda_gate(ramp, dt, a, -5.0)
    assert np.all(np.diff(o, axis=1) <= 0)


def test_gate_parameter_broadcast():
    """dt_bias is per (head, channel) and a_log per head: changing one entry changes only its own
    channel or head."""
    g, dt, a = _inputs(7)
    base = oracle.kda_gate(g, dt, a, -5.0)
    dt2 = dt.copy()
    dt2[1, 17] += 1.0
    d = oracle.kda_gate(g, dt2, a, -5.0) != base
    assert d[:, :, 1, 17].all() and d.sum() == d[:, :, 1, 17].size
    a2 = a.copy()
    a2[2] += 0.5
    d = oracle.kda_gate(g, dt, a2, -5.0) != base
    assert d[:, :, 2].all() and d.sum() == d[:, :, 2].size
    # the flat [H * D] bias layout is the same as [H][D]
    assert np.array_equal(oracle.kda_gate(g, dt.reshape(-1), a, -5.0), base)


@pytest.mark.parametrize("slip", ["no_bias", "rate_without_exp", "bias_by_channel_only", "rate_by_channel",
                                  "sign", "softplus"])
def test_planted_slips_fail_the_pins(monkeypatch, slip):
    """Plausible mistakes in kda_gate, planted in the oracle here on the CPU: each breaks a pin."""
    true_gate = oracle.kda_gate

    def wrong(g_raw_bits, dt_bias, a_log, lower_bound):
        g = oracle.bf16_to_f64(g_raw_bits)
        B, T, Hh, Dd = g.shape
        dt = np.asarray(dt_bias, np.float64).reshape(Hh, Dd)
        al = np.asarray(a_log, np.float64).reshape(Hh)
        lo = float(np.float32(lower_bound))
        rate = np.exp(al)[None, None, :, None]
        arg = rate * (g + dt[None, None])
        if slip == "no_bias":
            arg = rate * g
        elif slip == "rate_without_exp":
            arg = al[None, None, :, None] * (g + dt[None, None])
        elif slip == "bias_by_channel_only":
            arg = rate * (g + dt[0][None, None, None, :])
        elif slip == "rate_by_channel":
            arg = np.exp(np.resize(al, Dd))[None, None, None, :] * (g + dt[None, None])
        elif slip == "sign":
            return -lo * oracle.sigmoid(arg)
        elif slip == "softplus":
            return np.maximum(lo, -rate * np.log1p(np.exp(g + dt[None, None])))
        return lo * oracle.sigmoid(arg)

    monkeypatch.setattr(oracle, "kda_gate", wrong)
    failed = 0
    for pin in (test_gate_at_the_bias_point_is_half_the_bound, test_gate_rate_is_exp_of_a_log,
                test_gate_limits_and_bounds, test_gate_parameter_broadcast):
        try:
            pin()
        except AssertionError:
            failed += 1
    monkeypatch.setattr(oracle, "kda_gate", true_gate)
    assert failed >= 1, f"no pin caught the slip {slip}"
