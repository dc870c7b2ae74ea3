"""GPU parity of the gated entry points (kda_gate and the beta sigmoid inside the core kernels) against
the fp64 oracle: the oracle's kda_gate and sigmoid give the gate and beta, its recurrence the result."""
import numpy as np
import pytest

import kda_inputs as ki
import oracle
from kda_testlib import SENTINEL, announce, assert_close, dev, host

pytestmark = pytest.mark.gpu
LB = ki.GATE_LOWER_BOUND


def _bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _oracle_gate_beta(gx, rows=None):
    g = oracle.kda_gate(gx["g_raw"], gx["dt_bias"], gx["a_log"], LB)
    b = oracle.sigmoid(gx["beta_logit"])
    if rows is not None:
        g, b = g[:, :rows], b[:, :rows]
    return g.astype(np.float32), b.astype(np.float32)


def _gate_dev(gx):
    return _bf16(gx["g_raw"]), dev(gx["beta_logit"]), dev(gx["dt_bias"]), dev(gx["a_log"])


@pytest.mark.parametrize("B,H,T,n_snap", [(64, 32, 1, 0), (3, 5, 4, 4), (2, 3, 9, 2)])
def test_gated_decode_matches_oracle(device, B, H, T, n_snap):
    import torch
    import kda_gated_delta_core_amd as kda
    announce(f"kda_recurrent_k_gated B={B} H={H} T={T} n_snap={n_snap}")
    x = ki.make_batch(9501 + T, B, H, T, -5.0, 0.02)
    gx = ki.gate_inputs(9601 + T, B, T, H)
    g, bl, dt, al = _gate_dev(gx)
    st = dev(x["state"])
    out = torch.full((B, T, H, 128), SENTINEL, device="cuda")
    snaps = torch.full((max(n_snap, 1), B, H, 128, 128), SENTINEL, device="cuda")
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    if T == 1:
        kda.kda_recurrent_step_gated(q, k, v, g, bl, dt, al, LB, st, out=out)
    else:
        kda.kda_recurrent_k_gated(q, k, v, g, bl, dt, al, LB, st, out=out, snapshots=snaps if n_snap else None,
                                  n_snapshots=n_snap)
    torch.cuda.synchronize()
    gate, beta = _oracle_gate_beta(gx)
    o_ref, s_ref, sn_ref, _ = oracle.serial(x["q"], x["k"], x["v"], gate, beta, x["state"], n_snap=n_snap)
    assert_close("out", host(out), o_ref)
    assert_close("state", host(st), s_ref)
    for t in range(n_snap):
        assert_close(f"snapshot[{t}]", host(snaps)[t], sn_ref[t])


def test_gated_decode_k_equals_steps_bitwise(device):
    import torch
    import kda_gated_delta_core_amd as kda
    B, H, T = 16, 8, 4
    announce(f"kda_recurrent_k_gated vs {T} steps B={B} H={H}")
    x = ki.make_batch(9510, B, H, T, -5.0, 0.02)
    gx = ki.gate_inputs(9610, B, T, H)
    g, bl, dt, al = _gate_dev(gx)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    st = dev(x["state"])
    snaps = torch.empty((T, B, H, 128, 128), device="cuda")
    out = kda.kda_recurrent_k_gated(q, k, v, g, bl, dt, al, LB, st, snapshots=snaps, n_snapshots=T)
    st2 = dev(x["state"])
    for t in range(T):
        o = kda.kda_recurrent_step_gated(q[:, t:t + 1].contiguous(), k[:, t:t + 1].contiguous(),
                                         v[:, t:t + 1].contiguous(), g[:, t:t + 1].contiguous(),
                                         bl[:, t:t + 1].contiguous(), dt, al, LB, st2)
        torch.cuda.synchronize()
        assert torch.equal(o, out[:, t:t + 1]), f"row {t}"
        assert torch.equal(st2, snaps[t]), f"snapshot {t}"
    assert torch.equal(st2, st)


@pytest.mark.parametrize("B,H,T,C", [(1, 4, 300, 64), (2, 3, 77, 16), (3, 2, 100, 32), (1, 2, 64, 64)])
def test_gated_prefill_matches_oracle(device, B, H, T, C):
    """Ragged and whole-chunk T at every chunk width, NaN in every pad row of every input (g_raw and the
    beta logits included)."""
    import torch
    import kda_gated_delta_core_amd as kda
    announce(f"kda_chunk_prefill_gated B={B} H={H} T={T} C={C}")
    t_pad = -(-T // C) * C
    x = ki.make_batch(9520 + T + C, B, H, T, -5.0, 0.02, alloc_rows=t_pad, pad_value=float("nan"))
    gx = ki.gate_inputs(9620 + T + C, B, t_pad, H)
    gx["g_raw"][:, T:] = 0x7fc0  # BF16 NaN
    gx["beta_logit"][:, T:] = np.nan
    g, bl, dt, al = _gate_dev(gx)
    st = dev(x["state"])
    out = torch.full((B, t_pad, H, 128), SENTINEL, device="cuda")
    kda.kda_chunk_prefill_gated(dev(x["q"]), dev(x["k"]), dev(x["v"]), g, bl, dt, al, LB, st, T, C, out=out)
    torch.cuda.synchronize()
    gate, beta = _oracle_gate_beta(gx, rows=T)
    sl = lambda a: np.ascontiguousarray(a[:, :T])
    o_ref, s_ref, _, _ = oracle.serial(sl(x["q"]), sl(x["k"]), sl(x["v"]), gate, beta, x["state"])
    o = host(out)
    assert_close("core", o[:, :T], o_ref)
    assert_close("state", host(st), s_ref)
    assert np.all(o[:, T:] == SENTINEL)


def test_gated_prefill_agrees_with_gated_decode_and_steep_bound(device):
    """A lower bound of -40 sends chunks down the steep-gate path; the gated prefill's final state and
    outputs agree with the gated decode over the same rows and with the oracle."""
    import torch
    import kda_gated_delta_core_amd as kda
    B, H, T, C, lb = 2, 3, 150, 64, -40.0
    announce(f"kda_chunk_prefill_gated vs kda_recurrent_k_gated, lower bound {lb}")
    t_pad = -(-T // C) * C
    x = ki.make_batch(9530, B, H, T, -5.0, 0.02, alloc_rows=t_pad)
    gx = ki.gate_inputs(9630, B, t_pad, H)
    g, bl, dt, al = _gate_dev(gx)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    st = dev(x["state"])
    out = kda.kda_chunk_prefill_gated(q, k, v, g, bl, dt, al, lb, st, T, C)
    st2 = dev(x["state"])
    sl = lambda t: t[:, :T].contiguous()
    o2 = kda.kda_recurrent_k_gated(sl(q), sl(k), sl(v), sl(g), sl(bl), dt, al, lb, st2)
    torch.cuda.synchronize()
    assert_close("prefill vs decode state", host(st), host(st2))
    assert_close("prefill vs decode out", host(out)[:, :T], host(o2))
    gate = oracle.kda_gate(gx["g_raw"], gx["dt_bias"], gx["a_log"], lb)[:, :T].astype(np.float32)
    beta = oracle.sigmoid(gx["beta_logit"])[:, :T].astype(np.float32)
    o_ref, s_ref, _, _ = oracle.serial(x["q"][:, :T].copy(), x["k"][:, :T].copy(), x["v"][:, :T].copy(), gate, beta,
                                       x["state"])
    assert gate.min() < -9.0  # the steep path is taken
    assert_close("core", host(out)[:, :T], o_ref)
    assert_close("state", host(st), s_ref)


def test_gated_prefill_full_size(device):
    """The T=8192 H=32 C=64 prefill workload's q, k, v and state with the gate inputs of its shape:
    every head against the oracle."""
    import kda_gated_delta_core_amd as kda
    w = ki.WORKLOADS["prefill_h32_t8192_c64"]
    announce(f"kda_chunk_prefill_gated {w.name} (generating inputs)")
    x = ki.workload_inputs(w)
    t_pad = w.T
    gx = ki.gate_inputs(1012, 1, t_pad, w.heads)
    g, bl, dt, al = _gate_dev(gx)
    st = dev(x["state"])
    sl = lambda a: dev(np.ascontiguousarray(a[:, :t_pad]))
    out = kda.kda_chunk_prefill_gated(sl(x["q"]), sl(x["k"]), sl(x["v"]), g, bl, dt, al, LB, st, w.T, w.chunk)
    gate, beta = _oracle_gate_beta(gx)
    announce("oracle, all heads")
    c = lambda a: np.ascontiguousarray(a[:, :w.T])
    o_ref, s_ref, _, _ = oracle.serial(c(x["q"]), c(x["k"]), c(x["v"]), gate, beta, x["state"])
    assert_close("core", host(out), o_ref)
    assert_close("state", host(st), s_ref)
