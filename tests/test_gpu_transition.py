"""GPU parity of the segment transition (P, Q) of a prefill and of the fold S <- P S + Q, through the
C ABI, against the fp64 oracle; and the split of one sequence into token segments (each segment's
transition, the fold in segment order, then each segment's prefill from its folded initial state)
against the prefill of the whole sequence."""
import numpy as np
import pytest

import kda_inputs as ki
import oracle
from kda_testlib import SENTINEL, announce, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _padded(x, t0, t1, C):
    """Rows [t0, t1) of every input, NaN rows appended up to the next multiple of the chunk width."""
    n = t1 - t0
    t_pad = -(-n // C) * C
    res = {}
    for name in ("q", "k", "v", "gate", "beta"):
        a = x[name][:, t0:t1]
        pad = np.full((a.shape[0], t_pad - n) + a.shape[2:], np.nan, np.float32)
        res[name] = dev(np.concatenate([a, pad], axis=1))
    return res


def _transition(kda, seg, T, C):
    import torch
    B, _, H, _ = seg["q"].shape
    P = torch.full((B, H, 128, 128), SENTINEL, device="cuda")
    Q = torch.full((B, H, 128, 128), SENTINEL, device="cuda")
    kda.kda_chunk_prefill_transition(seg["q"], seg["k"], seg["v"], seg["gate"], seg["beta"], T, C,
                                     trans_p=P, trans_q=Q)
    torch.cuda.synchronize()
    return P, Q


def _check_contract(x, T, P, Q, seed):
    """P S + Q against the state the oracle's recurrence reaches from a random initial state S: the
    contract itself, meaningful also where P has decayed below the FP32 range (every row shrinks
    each key direction it updates, so over long segments P tends to zero whatever the gates)."""
    S = np.random.default_rng(seed).standard_normal(x["state"].shape).astype(np.float32)
    sl = lambda n: x[n][:, :T]
    _, s_ref, _, _ = oracle.serial(sl("q"), sl("k"), sl("v"), sl("gate"), sl("beta"), S)
    got = np.matmul(host(P).astype(np.float64), S.astype(np.float64)) + host(Q)
    assert_close("P S + Q", got, s_ref)


# Gates near 0 and short segments keep P inside the FP32 range, so P itself is compared; with gates
# down to -5 (the prefill workloads' range) P underflows within a few dozen tokens and only the
# contract P S + Q and Q are meaningful.
@pytest.mark.parametrize("B,H,T,C", [(1, 2, 64, 16), (2, 3, 100, 32), (1, 2, 130, 64), (2, 1, 1, 64),
                                     (1, 3, 17, 16), (1, 2, 200, 64)])
def test_transition_matches_oracle(device, B, H, T, C):
    import kda_gated_delta_core_amd as kda
    announce(f"kda_chunk_prefill_transition B={B} H={H} T={T} C={C} mild gates")
    x = ki.make_batch(7000 + T + C, B, H, T, -0.02, 0.02)
    P, Q = _transition(kda, _padded(x, 0, T, C), T, C)
    P_ref, Q_ref = oracle.transition(x["q"], x["k"], x["v"], x["gate"], x["beta"])
    assert float(np.linalg.norm(P_ref)) > 0.1
    assert_close("P", host(P), P_ref)
    assert_close("Q", host(Q), Q_ref)
    _check_contract(x, T, P, Q, 7001)


@pytest.mark.parametrize("T,C,lo", [(100, 16, -5.0), (130, 64, -5.0), (333, 32, -5.0), (130, 64, -15.0),
                                    (100, 16, -40.0)])
def test_transition_steep_gates(device, T, C, lo):
    """gates drawn down to -5, and down to -15 and -40 (the prefill's steep-gate path)"""
    import kda_gated_delta_core_amd as kda
    B, H = 2, 3
    announce(f"kda_chunk_prefill_transition B={B} H={H} T={T} C={C} gates to {lo}")
    x = ki.make_batch(7050 + T + int(-lo), B, H, T, lo, 0.02)
    P, Q = _transition(kda, _padded(x, 0, T, C), T, C)
    P_ref, Q_ref = oracle.transition(x["q"], x["k"], x["v"], x["gate"], x["beta"])
    assert_close("Q", host(Q), Q_ref)
    assert float(np.abs(host(P) - P_ref).max()) <= 1e-6
    _check_contract(x, T, P, Q, 7051)


def test_transition_mild_gates_long(device):
    """gates near 0 over many chunks keep P well inside the FP32 range (the homogeneous part is
    exercised, not decayed away)"""
    import kda_gated_delta_core_amd as kda
    B, H, T, C = 1, 2, 1000, 64
    announce(f"kda_chunk_prefill_transition mild gates B={B} H={H} T={T} C={C}")
    x = ki.make_batch(7101, B, H, T, -0.005, 0.02)
    P, Q = _transition(kda, _padded(x, 0, T, C), T, C)
    P_ref, Q_ref = oracle.transition(x["q"], x["k"], x["v"], x["gate"], x["beta"])
    assert float(np.abs(P_ref).max()) > 1e-3
    assert_close("P", host(P), P_ref)
    assert_close("Q", host(Q), Q_ref)
    _check_contract(x, T, P, Q, 7102)


def test_transition_full_size(device):
    """the T=8192, H=32, C=64 prefill workload: Q of every head, and P through the contract from the
    workload's own initial state"""
    import kda_gated_delta_core_amd as kda
    w = ki.WORKLOADS["prefill_h32_t8192_c64"]
    announce(f"kda_chunk_prefill_transition {w.name} seed={w.seed}")
    x = ki.workload_inputs(w)
    P, Q = _transition(kda, _padded(x, 0, w.T, w.chunk), w.T, w.chunk)
    sl = lambda n: x[n][:, :w.T]
    P_ref, Q_ref = oracle.transition(sl("q"), sl("k"), sl("v"), sl("gate"), sl("beta"))
    assert_close("Q", host(Q), Q_ref)
    assert float(np.abs(host(P) - P_ref).max()) <= 1e-6
    _, s_ref, _, _ = oracle.serial(sl("q"), sl("k"), sl("v"), sl("gate"), sl("beta"), x["state"])
    got = np.matmul(host(P).astype(np.float64), x["state"].astype(np.float64)) + host(Q)
    assert_close("P S0 + Q", got, s_ref)


@pytest.mark.parametrize("B,H", [(2, 5), (2, 8), (1, 1), (3, 11)])
def test_apply_matches_oracle(device, B, H):
    """Whole and partial groups of eight states (each state split over column groups)."""
    import torch
    import kda_gated_delta_core_amd as kda
    announce(f"kda_state_transition_apply B={B} H={H}")
    rng = np.random.default_rng(7200 + B * H)
    P = (rng.standard_normal((B, H, 128, 128)) / 8).astype(np.float32)
    Q = rng.standard_normal((B, H, 128, 128)).astype(np.float32)
    S = rng.standard_normal((B, H, 128, 128)).astype(np.float32)
    Pd, Qd = dev(P), dev(Q)
    Sd = dev(S)
    kda.kda_state_transition_apply(Pd, Qd, Sd)
    torch.cuda.synchronize()
    assert_close("P S + Q", host(Sd), oracle.apply_transition(P, Q, S))
    Sd = dev(S)
    kda.kda_state_transition_apply(Pd, None, Sd)
    torch.cuda.synchronize()
    assert_close("P S", host(Sd), oracle.apply_transition(P, None, S))
    assert np.array_equal(host(Pd), P) and np.array_equal(host(Qd), Q), "inputs were written"


def test_segments_fold_to_the_whole_prefill(device):
    """One sequence split at token boundaries that cut chunks: transitions per segment, folded in
    order from the initial state, then every segment's prefill from its folded initial state gives
    the whole sequence's outputs and final state."""
    import torch
    import kda_gated_delta_core_amd as kda
    B, H, T, C = 2, 3, 300, 64
    cuts = [0, 70, 200, 300]
    announce(f"segment fold B={B} H={H} T={T} C={C} cuts={cuts}")
    x = ki.make_batch(7300, B, H, T, -3.0, 0.05)
    S = dev(x["state"])
    outs, s_in = [], []
    for t0, t1 in zip(cuts[:-1], cuts[1:]):
        seg = _padded(x, t0, t1, C)
        P, Q = _transition(kda, seg, t1 - t0, C)
        s_in.append(S.clone())
        kda.kda_state_transition_apply(P, Q, S)
    folded_final = S
    for (t0, t1), s0 in zip(zip(cuts[:-1], cuts[1:]), s_in):
        seg = _padded(x, t0, t1, C)
        st = s0.clone()
        out = kda.kda_chunk_prefill(seg["q"], seg["k"], seg["v"], seg["gate"], seg["beta"], st, t1 - t0, C)
        outs.append(host(out)[:, :t1 - t0])
        last_state = st
    torch.cuda.synchronize()
    o_ref, s_ref, _, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"])
    assert_close("outputs", np.concatenate(outs, axis=1), o_ref)
    assert_close("final state (last segment's prefill)", host(last_state), s_ref)
    assert_close("final state (fold)", host(folded_final), s_ref)


def test_transitions_compose(device):
    """(P2 P1, P2 Q1 + Q2) from two segments equals the transition of their concatenation"""
    import torch
    import kda_gated_delta_core_amd as kda
    B, H, C = 1, 2, 32
    announce(f"transition composition B={B} H={H} C={C}")
    x = ki.make_batch(7400, B, H, 150, -0.02, 0.02)
    P1, Q1 = _transition(kda, _padded(x, 0, 61, C), 61, C)
    P2, Q2 = _transition(kda, _padded(x, 61, 150, C), 89, C)
    kda.kda_state_transition_apply(P2, None, P1)  # P1 <- P2 P1
    kda.kda_state_transition_apply(P2, Q2, Q1)    # Q1 <- P2 Q1 + Q2
    torch.cuda.synchronize()
    P_ref, Q_ref = oracle.transition(x["q"], x["k"], x["v"], x["gate"], x["beta"])
    assert_close("P2 P1", host(P1), P_ref)
    assert_close("P2 Q1 + Q2", host(Q1), Q_ref)


def test_chunk_scan_reruns_the_prefill_bitwise(device):
    """kda_chunk_scan from the records a kda_chunk_prefill left equals a second kda_chunk_prefill from
    the same initial state bit for bit, and so do the records a transition leaves"""
    import torch
    import kda_gated_delta_core_amd as kda
    B, H, T, C = 2, 3, 250, 64
    announce(f"kda_chunk_scan B={B} H={H} T={T} C={C}")
    x = ki.make_batch(7500, B, H, T, -4.0, 0.05)
    seg = _padded(x, 0, T, C)
    args = [seg[n] for n in ("q", "k", "v", "gate", "beta")]
    ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T, C), dtype=torch.uint8, device="cuda")
    s_a = dev(x["state"])
    out_a = kda.kda_chunk_prefill(*args, s_a, T, C, workspace=ws)
    s_b = dev(x["state"])
    out_b = torch.full_like(out_a, SENTINEL)
    kda.kda_chunk_scan(s_b, T, C, ws, out=out_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a[:, :T], out_b[:, :T]) and torch.equal(s_a, s_b)
    assert bool((out_b[:, T:] == SENTINEL).all()), "rows >= T were written"
    kda.kda_chunk_prefill_transition(*args, T, C, workspace=ws)
    s_c = dev(x["state"])
    out_c = kda.kda_chunk_scan(s_c, T, C, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_a[:, :T], out_c[:, :T]) and torch.equal(s_a, s_c)
    o_ref, st_ref, _, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"])
    assert_close("out", host(out_c)[:, :T], o_ref)
    assert_close("state", host(s_c), st_ref)


def test_segments_from_kept_records(device):
    """the split as a device runs it: transition (records kept), fold, then kda_chunk_scan from the
    kept records and the folded state, per segment; equals the whole sequence's prefill"""
    import torch
    import kda_gated_delta_core_amd as kda
    B, H, C = 2, 2, 32
    cuts = [0, 45, 128, 200, 260]
    announce(f"segments from kept records B={B} H={H} C={C} cuts={cuts}")
    x = ki.make_batch(7600, B, H, cuts[-1], -2.0, 0.05)
    segs, wss, trans = [], [], []
    for t0, t1 in zip(cuts[:-1], cuts[1:]):
        seg = _padded(x, t0, t1, C)
        ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, t1 - t0, C), dtype=torch.uint8, device="cuda")
        trans.append(kda.kda_chunk_prefill_transition(*(seg[n] for n in ("q", "k", "v", "gate", "beta")), t1 - t0, C,
                                                      workspace=ws))
        segs.append(seg)
        wss.append(ws)
    S = dev(x["state"])
    outs = []
    for (t0, t1), ws, (P, Q) in zip(zip(cuts[:-1], cuts[1:]), wss, trans):
        s_in = S.clone()
        outs.append(host(kda.kda_chunk_scan(s_in, t1 - t0, C, ws))[:, :t1 - t0])
        kda.kda_state_transition_apply(P, Q, S)
    torch.cuda.synchronize()
    o_ref, s_ref, _, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"])
    assert_close("outputs", np.concatenate(outs, axis=1), o_ref)
    assert_close("final state (fold)", host(S), s_ref)
