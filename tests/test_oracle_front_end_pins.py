"""Pins of the oracle's decode front end (CPU only): torch's own depthwise conv1d and SiLU on the
token history, closed forms of the L2 step, the conv state as a plain window of past inputs, and
continuation."""
import numpy as np
import torch

import kda_inputs as ki
import oracle

D = 128


def _case(seed, B, T, H, K):
    x = ki.front_end_inputs(seed, B, T, H, K)
    return x["qkv"], x["conv_w"], x["conv_state"]


def test_conv_and_silu_match_torch_on_the_history():
    B, T, H, K = 2, 5, 1, 4
    qkv, w, s0 = _case(11, B, T, H, K)
    eps = 1e-6
    q, k, v, s, _ = oracle.decode_front_end(qkv, w, s0, H, eps)
    # history per sequence: the K-1 newest slots of the initial state, then the T new inputs
    xs = torch.from_numpy(oracle.bf16_to_f64(qkv)).permute(0, 2, 1)              # [B][C][T]
    hist = torch.cat([torch.from_numpy(s0[:, :, 1:].astype(np.float64)), xs], dim=2)
    wt = torch.from_numpy(oracle.bf16_to_f64(w))[:, None, :]                      # [C][1][K]
    y = torch.nn.functional.silu(torch.nn.functional.conv1d(hist, wt, groups=3 * H * D))  # [B][C][T]
    y = y.permute(0, 2, 1).reshape(B, T, 3, H, D).numpy()
    np.testing.assert_allclose(v, y[:, :, 2], rtol=1e-13, atol=1e-15)
    for part, got in ((0, q), (1, k)):
        ref = y[:, :, part] / np.sqrt(np.sum(y[:, :, part] ** 2, axis=-1, keepdims=True) + float(np.float32(eps)))
        np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_state_is_the_window_of_past_inputs():
    B, T, H, K = 3, 6, 2, 3
    qkv, w, s0 = _case(12, B, T, H, K)
    _, _, _, s, snaps = oracle.decode_front_end(qkv, w, s0, H, 1e-6, n_snap=4)
    x = oracle.bf16_to_f64(qkv)
    assert np.array_equal(s, np.transpose(x[:, T - K:], (0, 2, 1)))
    # after row 0 the window is the K-1 newest old slots, then x_0
    assert np.array_equal(snaps[0][..., :K - 1], s0[..., 1:].astype(np.float64))
    assert np.array_equal(snaps[0][..., K - 1], x[:, 0])
    assert np.array_equal(snaps[3][..., K - 1], x[:, 3])


def test_single_tap_is_pointwise_and_l2_closed_form():
    B, T, H, K = 1, 1, 1, 1
    qkv, w, s0 = _case(13, B, T, H, K)
    qkv = qkv.copy()
    qkv[..., :D] = 0
    qkv[0, 0, 5] = ki.to_bf16_bits(np.float32(2.0))      # q: one-hot 2 at channel 5
    w = np.full_like(w, ki.to_bf16_bits(np.float32(1.5)))
    q, k, v, _, _ = oracle.decode_front_end(qkv, w, s0, H, 1e-6)
    y = 3.0 / (1.0 + np.exp(-3.0))                        # silu(1.5 * 2)
    assert q[0, 0, 0, 5] == np.float64(y / np.sqrt(y * y + float(np.float32(1e-6))))
    assert np.count_nonzero(q) == 1
    xv = oracle.bf16_to_f64(qkv[0, 0, 2 * D:]) * 1.5
    np.testing.assert_allclose(v[0, 0, 0], xv / (1.0 + np.exp(-xv)), rtol=1e-15)
    # q and k rows are unit vectors up to eps
    np.testing.assert_allclose(np.sum(k * k, axis=-1), 1.0, rtol=1e-5)


def test_continuation_is_exact():
    B, T, H, K = 2, 7, 1, 4
    qkv, w, s0 = _case(14, B, T, H, K)
    a = oracle.decode_front_end(qkv, w, s0, H, 1e-6)
    b1 = oracle.decode_front_end(qkv[:, :3], w, s0, H, 1e-6)
    b2 = oracle.decode_front_end(qkv[:, 3:], w, b1[3].astype(np.float32), H, 1e-6)
    for i in range(3):
        assert np.array_equal(a[i], np.concatenate([b1[i], b2[i]], axis=1))
    assert np.array_equal(a[3], b2[3])
