"""GPU parity of the recurrent (decode) forms against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import kda_inputs as ki
import oracle
from kda_testlib import SENTINEL, announce, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _run_step(kda, x, B, H):
    import torch
    st = dev(x["state"])
    out = torch.full((B, 1, H, 128), SENTINEL, device="cuda")
    kda.kda_recurrent_step(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["gate"]), dev(x["beta"]), st, out=out)
    torch.cuda.synchronize()
    return host(out), host(st)


@pytest.mark.parametrize("B,H", [(1, 1), (3, 5), (64, 32)])
def test_decode_step_matches_oracle(device, B, H):
    import kda_gated_delta_core_amd as kda
    w = ki.WORKLOADS["decode_b64_h32"]
    announce(f"kda_recurrent_step seed={w.seed} B={B} H={H}")
    x = ki.make_batch(w.seed, B, H, 1, w.gate_lo, w.state_std)
    out, st = _run_step(kda, x, B, H)
    o_ref, s_ref, _, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"])
    assert_close("out", out, o_ref)
    assert_close("state", st, s_ref)


def test_decode_step_extreme_gates(device):
    """Very negative and zero gates, beta at 0 and 1: the decode form has no range limit."""
    import kda_gated_delta_core_amd as kda
    B, H = 2, 4
    announce("kda_recurrent_step extreme gates")
    x = ki.make_batch(7, B, H, 1, -5.0, 0.02)
    x["gate"][0] = -60.0
    x["gate"][1, :, :2] = 0.0
    x["beta"][1, :, 0] = 0.0
    x["beta"][1, :, 1] = 1.0
    out, st = _run_step(kda, x, B, H)
    o_ref, s_ref, _, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"])
    assert_close("out", out, o_ref)
    assert_close("state", st, s_ref)


def _decode_k(kda, x, B, H, T, n_snap, n_slots=None):
    import torch
    st = dev(x["state"])
    out = torch.full((B, T, H, 128), SENTINEL, device="cuda")
    n_slots = n_snap if n_slots is None else n_slots
    snaps = torch.full((max(n_slots, 1), B, H, 128, 128), SENTINEL, device="cuda")
    kda.kda_recurrent_k(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["gate"]), dev(x["beta"]), st, out=out,
                        snapshots=snaps if n_snap else None, n_snapshots=n_snap)
    torch.cuda.synchronize()
    return out, st, snaps


@pytest.mark.parametrize("B,H,T,n_snap", [(2, 3, 4, 4), (1, 2, 7, 3), (5, 1, 1, 1), (3, 2, 9, 0)])
def test_decode_k_matches_oracle(device, B, H, T, n_snap):
    import kda_gated_delta_core_amd as kda
    w = ki.WORKLOADS["decode_k4_b128_h32"]
    announce(f"kda_recurrent_k seed={w.seed} B={B} H={H} T={T} n_snap={n_snap}")
    x = ki.make_batch(w.seed, B, H, T, w.gate_lo, w.state_std)
    out, st, snaps = _decode_k(kda, x, B, H, T, n_snap, n_slots=n_snap + 1)
    o_ref, s_ref, sn_ref, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"],
                                            n_snap=n_snap)
    assert_close("out", host(out), o_ref)
    assert_close("state", host(st), s_ref)
    sn = host(snaps)
    for t in range(n_snap):
        assert_close(f"snapshot[{t}]", sn[t], sn_ref[t])
    # the slot after the last snapshot is never written
    assert np.all(sn[n_snap] == SENTINEL)


def test_decode_k_full_size_bitwise_and_parity(device):
    """decode_k at B=128, H=32, k=4 with 4 snapshots: bit-identical to 4 serial steps, and equal to
    the oracle on every sequence and head."""
    import torch
    import kda_gated_delta_core_amd as kda
    w = ki.WORKLOADS["decode_k4_b128_h32"]
    B, H, T = w.batch, w.heads, w.T
    announce(f"kda_recurrent_k full size seed={w.seed} B={B} H={H} T={T}")
    x = ki.workload_inputs(w)
    out, st, snaps = _decode_k(kda, x, B, H, T, w.n_snap)
    # the same rows through T single steps
    st2 = dev(x["state"])
    outs = []
    for t in range(T):
        sl = lambda a: dev(a[:, t:t + 1])
        o = torch.empty((B, 1, H, 128), device="cuda")
        kda.kda_recurrent_step(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["gate"]), sl(x["beta"]), st2, out=o)
        torch.cuda.synchronize()
        assert torch.equal(st2, snaps[t]), f"snapshot {t} differs from step {t}"
        outs.append(o)
    assert torch.equal(torch.cat(outs, 1), out)
    assert torch.equal(st2, st)
    # oracle on every sequence
    o_ref, s_ref, sn_ref, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"],
                                            n_snap=w.n_snap)
    o, s, sn = host(out), host(st), host(snaps)
    assert_close("out", o, o_ref)
    assert_close("state", s, s_ref)
    for t in range(w.n_snap):
        assert_close(f"snapshot[{t}]", sn[t], sn_ref[t])
    for b in range(B):  # no sequence passes on the strength of the others
        assert_close(f"b{b} out", o[b], o_ref[b], quiet=True)
        assert_close(f"b{b} state", s[b], s_ref[b], quiet=True)
        for t in range(w.n_snap):
            assert_close(f"b{b} snapshot[{t}]", sn[t][b], sn_ref[t][b], quiet=True)


def test_decode_k_rollback_to_a_snapshot(device):
    """Speculative verify: walk 5 rows with snapshots, accept 2, restore snapshot 1 and walk the
    remaining rows again: outputs and final state equal the first walk's, bit for bit (the state
    buffer and its snapshots are the resume points)."""
    import torch
    import kda_gated_delta_core_amd as kda
    B, H, T = 3, 2, 5
    announce(f"kda_recurrent_k rollback B={B} H={H} T={T}")
    x = ki.make_batch(1404, B, H, T, -5.0, 0.02)
    out, st, snaps = _decode_k(kda, x, B, H, T, T)
    st2 = snaps[1].clone()  # the state after row 1
    rest = lambda a: dev(np.ascontiguousarray(a[:, 2:]))
    out2 = kda.kda_recurrent_k(rest(x["q"]), rest(x["k"]), rest(x["v"]), rest(x["gate"]), rest(x["beta"]), st2)
    torch.cuda.synchronize()
    assert torch.equal(out2, out[:, 2:])
    assert torch.equal(st2, st)


@pytest.mark.timeout(600)
def test_decode_step_state_past_4gib(device):
    """66,000 heads in one call: the state spans 4.03 GiB, so the byte offsets of the last heads pass
    2^32; every head against the oracle, and the heads past 2^32 on their own."""
    import kda_gated_delta_core_amd as kda
    B, H = 500, 132
    announce(f"kda_recurrent_step B={B} H={H} (state {B * H * 65536 / 2 ** 30:.2f} GiB)")
    x = ki.make_batch(9300, B, H, 1, -5.0, 0.02)
    out, st = _run_step(kda, x, B, H)
    o_ref, s_ref, _, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"])
    assert_close("out", out, o_ref)
    assert_close("state", st, s_ref)
    first = 2 ** 32 // 65536  # the first head whose state starts at or past 2^32 bytes
    assert B * H > first
    assert_close("heads past 2^32: out", out.reshape(B * H, 128)[first:], o_ref.reshape(B * H, 128)[first:])
    assert_close("heads past 2^32: state", st.reshape(B * H, 128, 128)[first:],
                 s_ref.reshape(B * H, 128, 128)[first:])


@pytest.mark.timeout(600)
def test_decode_k_snapshots_past_4gib(device):
    """8 rows and 8 snapshots of 8,448 heads: the snapshot array spans 4.1 GiB, so the last snapshots'
    byte offsets pass 2^32; every snapshot, the rows and the final state against the oracle."""
    import torch
    import kda_gated_delta_core_amd as kda
    B, H, T = 66, 128, 8
    announce(f"kda_recurrent_k B={B} H={H} k={T} (snapshots {T * B * H * 65536 / 2 ** 30:.2f} GiB)")
    x = ki.make_batch(9301, B, H, T, -5.0, 0.02)
    st = dev(x["state"])
    snaps = torch.full((T, B, H, 128, 128), SENTINEL, device="cuda")
    out = kda.kda_recurrent_k(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["gate"]), dev(x["beta"]), st,
                              snapshots=snaps, n_snapshots=T)
    torch.cuda.synchronize()
    o_ref, s_ref, sn_ref, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"], n_snap=T)
    assert_close("out", host(out), o_ref)
    assert_close("state", host(st), s_ref)
    assert T * B * H * 65536 > 2 ** 32
    for t in range(T):
        assert_close(f"snapshot[{t}]", host(snaps[t]), sn_ref[t])
