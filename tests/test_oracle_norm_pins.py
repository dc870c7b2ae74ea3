"""Pins of the oracle's gated RMSNorm (CPU only): library routines computing the same definition,
closed forms and invariants, so a dropped term, a wrong axis or a misplaced eps fails one of them."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle

D = 128


def _bits(x):
    return ki.to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_bf16_decoding_known_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x7F80, 0xFF80, 0x0001, 0x0000, 0x8000], dtype=np.uint16)
    want = [1.0, -1.0, 3.140625, np.inf, -np.inf, 2.0 ** -133, 0.0, -0.0]
    got = oracle.bf16_to_f64(bits)
    assert got.tolist() == want
    assert np.signbit(got[-1])
    # and torch's own bfloat16 decoding of the same patterns
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(t, got)


def test_bf16_encoding_rounds_to_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20, -2.5, 3.0e38],
                 dtype=np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ki.to_bf16_bits(x), t)
    assert ki.to_bf16_bits(np.float32(1.0 + 2.0 ** -8)) == 0x3F80        # tie -> even
    assert ki.to_bf16_bits(np.float32(1.0 + 3 * 2.0 ** -8)) == 0x3F82    # tie -> even (up)


@pytest.mark.parametrize("eps", [1e-6, 1e-2])
def test_matches_torch_rms_norm_times_sigmoid(eps):
    x = ki.norm_inputs(5, 9, 3)
    got = oracle.gated_rmsnorm(x["core"], x["out_gate"], x["o_norm"], eps)
    c = torch.from_numpy(x["core"]).double()
    w = torch.from_numpy(oracle.bf16_to_f64(x["o_norm"]))
    g = torch.from_numpy(oracle.bf16_to_f64(x["out_gate"]))
    want = torch.nn.functional.rms_norm(c, (D,), weight=w, eps=float(np.float32(eps))) * torch.sigmoid(g)
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-13, atol=0)


def test_one_hot_closed_form():
    eps = 1e-6
    a, j = -3.0, 17
    core = np.zeros((1, 1, D), dtype=np.float32)
    core[0, 0, j] = a
    w = np.full(D, 0.75, dtype=np.float32)
    g = np.full((1, 1, D), 2.0, dtype=np.float32)
    y = oracle.gated_rmsnorm(core, _bits(g), _bits(w), eps)
    e = float(np.float32(eps))
    want = a / np.sqrt(a * a / D + e) * 0.75 / (1.0 + np.exp(-2.0))
    assert y[0, 0, j] == pytest.approx(want, rel=1e-15)
    assert np.count_nonzero(y) == 1


def test_gate_zero_and_infinite():
    x = ki.norm_inputs(6, 4, 2)
    base = oracle.gated_rmsnorm(x["core"], np.full_like(x["out_gate"], 0x7F80), x["o_norm"], 1e-6)  # sigmoid(+inf)=1
    half = oracle.gated_rmsnorm(x["core"], np.zeros_like(x["out_gate"]), x["o_norm"], 1e-6)          # sigmoid(0)=1/2
    off = oracle.gated_rmsnorm(x["core"], np.full_like(x["out_gate"], 0xFF80), x["o_norm"], 1e-6)    # sigmoid(-inf)=0
    assert np.array_equal(half, base / 2)
    assert not np.any(off)


def test_scale_invariance_and_unit_mean_square():
    x = ki.norm_inputs(7, 6, 2)
    ones = np.full(D, 0x3F80, dtype=np.uint16)
    gate_on = np.full_like(x["out_gate"], 0x7F80)
    y = oracle.gated_rmsnorm(x["core"], gate_on, ones, 1e-30)
    y_scaled = oracle.gated_rmsnorm(x["core"] * np.float32(2.0 ** 40), gate_on, ones, 1e-30)
    np.testing.assert_allclose(y_scaled, y, rtol=1e-14, atol=0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-12)
    # eps acts inside the square root: a row of all-equal entries a gives a / sqrt(a^2 + eps)
    a = np.float32(1e-3)
    y_eps = oracle.gated_rmsnorm(np.full((1, 1, D), a, dtype=np.float32), gate_on, ones, 1e-6)
    want = float(a) / np.sqrt(float(a) ** 2 + float(np.float32(1e-6)))
    np.testing.assert_allclose(y_eps, want, rtol=1e-15)


def test_rows_and_heads_are_independent():
    x = ki.norm_inputs(8, 5, 3)
    y = oracle.gated_rmsnorm(x["core"], x["out_gate"], x["o_norm"], 1e-6)
    y1 = oracle.gated_rmsnorm(x["core"][2:3, 1:2], x["out_gate"][2:3, 1:2], x["o_norm"], 1e-6)
    assert np.array_equal(y[2:3, 1:2], y1)
