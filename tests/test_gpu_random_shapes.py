"""Seeded random shapes against the fp64 oracle (through the C ABI): prefill at any chunk width with
ragged lengths, decode_k with any snapshot count, varlen batches with empty and one-token sequences.
The fixed-shape tests cover the workloads and edges by name; these sweep the space between them."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testlib import SENTINEL, announce, assert_close, dev, host

pytestmark = pytest.mark.gpu
RNG_SEED = 20261202


def _cases(n, draw):
    rng = np.random.default_rng(RNG_SEED + n)
    return [draw(rng) for _ in range(n)]


PREFILL = _cases(10, lambda r: (int(r.integers(1, 4)), int(r.integers(1, 10)), int(r.integers(1, 400)),
                                int(r.choice([16, 32, 64])), float(r.uniform(-9.0, 0.0)), int(r.integers(0, 10 ** 6))))


@pytest.mark.parametrize("B,H,T,C,gate_lo,seed", PREFILL)
def test_random_prefill(device, B, H, T, C, gate_lo, seed):
    import kda_gated_delta_core_amd as kda
    announce(f"kda_chunk_prefill B={B} H={H} T={T} C={C} gate_lo={gate_lo:.2f} seed={seed}")
    t_pad = -(-T // C) * C
    x = ki.make_batch(seed, B, H, T, gate_lo, 0.02, alloc_rows=t_pad, pad_value=float("nan"))
    st = dev(x["state"])
    out = torch.full((B, t_pad, H, 128), SENTINEL, device="cuda")
    kda.kda_chunk_prefill(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["gate"]), dev(x["beta"]), st, T, C, out=out)
    torch.cuda.synchronize()
    sl = lambda a: np.ascontiguousarray(a[:, :T])
    o_ref, s_ref, _, _ = oracle.serial(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["gate"]), sl(x["beta"]), x["state"])
    assert_close("out", host(out)[:, :T], o_ref)
    assert_close("state", host(st), s_ref)
    assert np.all(host(out)[:, T:] == SENTINEL)


DECODE_K = _cases(10, lambda r: (int(r.integers(1, 20)), int(r.integers(1, 12)), int(r.integers(1, 9)),
                                 float(r.uniform(-20.0, 0.0)), int(r.integers(0, 10 ** 6))))


@pytest.mark.parametrize("B,H,T,gate_lo,seed", DECODE_K)
def test_random_decode_k(device, B, H, T, gate_lo, seed):
    import kda_gated_delta_core_amd as kda
    n_snap = seed % (T + 1)
    announce(f"kda_recurrent_k B={B} H={H} T={T} n_snap={n_snap} gate_lo={gate_lo:.2f} seed={seed}")
    x = ki.make_batch(seed, B, H, T, gate_lo, 0.02)
    st = dev(x["state"])
    snaps = torch.full((n_snap + 1, B, H, 128, 128), SENTINEL, device="cuda")
    out = kda.kda_recurrent_k(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["gate"]), dev(x["beta"]), st,
                              snapshots=snaps if n_snap else None, n_snapshots=n_snap)
    torch.cuda.synchronize()
    o_ref, s_ref, sn_ref, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"], n_snap=n_snap)
    assert_close("out", host(out), o_ref)
    assert_close("state", host(st), s_ref)
    sn = host(snaps)
    for t in range(n_snap):
        assert_close(f"snapshot[{t}]", sn[t], sn_ref[t])
    assert np.all(sn[n_snap] == SENTINEL)


VARLEN = _cases(6, lambda r: ([int(x) for x in r.choice([0, 1, 2, 15, 64, 65, 200], size=int(r.integers(1, 7)))],
                              int(r.integers(1, 6)), int(r.choice([16, 32, 64])), int(r.integers(0, 10 ** 6))))


@pytest.mark.parametrize("lens,H,C,seed", VARLEN)
def test_random_varlen(device, lens, H, C, seed):
    import kda_gated_delta_core_amd as kda
    if sum(lens) == 0:
        lens = lens + [3]
    announce(f"kda_chunk_prefill_varlen lens={lens} H={H} C={C} seed={seed}")
    x = ki.varlen_inputs(seed, lens, H, -5.0, 0.02)
    d = {n: torch.from_numpy(x[n]).cuda() for n in ("q", "k", "v", "gate", "beta", "state", "cu_seqlens")}
    out = torch.full_like(d["q"], SENTINEL)
    kda.kda_chunk_prefill_varlen(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["state"], d["cu_seqlens"], C,
                                 out=out)
    torch.cuda.synchronize()
    got_o, got_s = host(out), host(d["state"])
    cu = x["cu_seqlens"]
    for s, n in enumerate(lens):
        a, b = int(cu[s]), int(cu[s + 1])
        if n == 0:
            np.testing.assert_array_equal(got_s[s], x["state"][s])  # an empty sequence keeps its state
            continue
        sl = lambda arr: np.ascontiguousarray(arr[None, a:b])
        o_ref, s_ref, _, _ = oracle.serial(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["gate"]), sl(x["beta"]),
                                           x["state"][s:s + 1])
        assert_close(f"seq {s} out", got_o[None, a:b], o_ref)
        assert_close(f"seq {s} state", got_s[s:s + 1], s_ref)


TRANSITION = _cases(8, lambda r: (int(r.integers(1, 3)), int(r.integers(1, 6)), int(r.integers(1, 300)),
                                  int(r.choice([16, 32, 64])), float(r.uniform(-6.0, 0.0)),
                                  int(r.integers(0, 10 ** 6))))


@pytest.mark.parametrize("B,H,T,C,gate_lo,seed", TRANSITION)
def test_random_transition(device, B, H, T, C, gate_lo, seed):
    """the contract P S + Q against the recurrence from a random state, and Q; P itself only where it
    stays inside the FP32 range (elsewhere within an absolute 1e-6)"""
    import kda_gated_delta_core_amd as kda
    announce(f"kda_chunk_prefill_transition B={B} H={H} T={T} C={C} gate_lo={gate_lo:.2f} seed={seed}")
    t_pad = -(-T // C) * C
    x = ki.make_batch(seed, B, H, T, gate_lo, 0.02, alloc_rows=t_pad, pad_value=float("nan"))
    P = torch.full((B, H, 128, 128), SENTINEL, device="cuda")
    Q = torch.full((B, H, 128, 128), SENTINEL, device="cuda")
    kda.kda_chunk_prefill_transition(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["gate"]), dev(x["beta"]), T, C,
                                     trans_p=P, trans_q=Q)
    torch.cuda.synchronize()
    sl = lambda a: np.ascontiguousarray(a[:, :T])
    P_ref, Q_ref = oracle.transition(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["gate"]), sl(x["beta"]))
    assert_close("Q", host(Q), Q_ref)
    if float(np.abs(P_ref).max()) > 1e-3:
        assert_close("P", host(P), P_ref)
    else:
        assert float(np.abs(host(P) - P_ref).max()) <= 1e-6
    S = np.random.default_rng(seed + 1).standard_normal((B, H, 128, 128)).astype(np.float32)
    _, s_ref, _, _ = oracle.serial(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["gate"]), sl(x["beta"]), S)
    assert_close("P S + Q", np.matmul(host(P).astype(np.float64), S.astype(np.float64)) + host(Q), s_ref)


FUSED = _cases(6, lambda r: (int(r.integers(1, 3)), int(r.integers(1, 5)), int(r.integers(1, 300)),
                             int(r.choice([16, 32, 64])), float(r.uniform(-9.0, 0.0)), int(r.integers(0, 10 ** 6))))


@pytest.mark.parametrize("B,H,T,C,gate_lo,seed", FUSED)
def test_random_fused_prefill(device, B, H, T, C, gate_lo, seed):
    """kda_chunk_prefill_fused against the oracle's front end followed by its recurrence"""
    import kda_gated_delta_core_amd as kda
    announce(f"kda_chunk_prefill_fused B={B} H={H} T={T} C={C} gate_lo={gate_lo:.2f} seed={seed}")
    t_pad = -(-T // C) * C
    fx = ki.front_end_inputs(seed, B, T, H, 4)
    x = ki.make_batch(seed + 1, B, H, T, gate_lo, 0.02, alloc_rows=t_pad, pad_value=float("nan"))
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    cst, st = dev(fx["conv_state"]), dev(x["state"])
    out = torch.full((B, t_pad, H, 128), SENTINEL, device="cuda")
    kda.kda_chunk_prefill_fused(bits(fx["qkv"]), bits(fx["conv_w"]), cst, dev(x["gate"]), dev(x["beta"]), st, C,
                                ki.L2_EPS, out=out)
    torch.cuda.synchronize()
    q, k, v, c_ref, _ = oracle.decode_front_end(fx["qkv"], fx["conv_w"], fx["conv_state"], H, ki.L2_EPS)
    sl = lambda a: np.ascontiguousarray(a[:, :T])
    o_ref, s_ref, _, _ = oracle.serial(q, k, v, sl(x["gate"]), sl(x["beta"]), x["state"])
    assert_close("out", host(out)[:, :T], o_ref)
    assert_close("state", host(st), s_ref)
    assert np.array_equal(host(cst), c_ref)
    assert np.all(host(out)[:, T:] == SENTINEL)
