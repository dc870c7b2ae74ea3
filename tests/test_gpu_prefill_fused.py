"""GPU parity of kda_chunk_prefill_fused (the front end fused into the prefill's prepare kernel), through
the C ABI: against the fp64 oracle's front end followed by its recurrence, against the two separate
calls (kda_prefill_front_end + kda_chunk_prefill), at ragged lengths, every chunk width and the
T=8192, H=32 workload."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testlib import SENTINEL, announce, assert_close, host

pytestmark = pytest.mark.gpu
D = 128
K = 4


def _bits_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _inputs(seed, B, T, H, C, gate_lo=-5.0):
    fx = ki.front_end_inputs(seed, B, T, H, K)
    t_pad = -(-T // C) * C
    core = ki.make_batch(seed + 1, B, H, T, gate_lo, 0.02, alloc_rows=t_pad, pad_value=float("nan"))
    return fx, core, t_pad


def _fused(kda, fx, core, H, T, C):
    B = fx["qkv"].shape[0]
    t_pad = -(-T // C) * C
    cst = torch.from_numpy(fx["conv_state"]).cuda()
    st = torch.from_numpy(core["state"]).cuda()
    out = torch.full((B, t_pad, H, D), SENTINEL, device="cuda")
    kda.kda_chunk_prefill_fused(_bits_dev(fx["qkv"]), _bits_dev(fx["conv_w"]), cst,
                                torch.from_numpy(core["gate"]).cuda(), torch.from_numpy(core["beta"]).cuda(), st, C,
                                ki.L2_EPS, out=out)
    torch.cuda.synchronize()
    return out, st, cst


def _oracle(fx, core, H, T):
    q, k, v, cst, _ = oracle.decode_front_end(fx["qkv"], fx["conv_w"], fx["conv_state"], H, ki.L2_EPS)
    o, s, _, _ = oracle.serial(q, k, v, core["gate"][:, :T], core["beta"][:, :T], core["state"])
    return o, s, cst


@pytest.mark.parametrize("B,T,H,C", [(1, 64, 2, 16), (2, 17, 3, 16), (2, 100, 3, 32), (1, 130, 2, 64),
                                     (2, 1, 1, 64), (1, 200, 4, 64), (1, 3, 2, 32)])
def test_fused_prefill_matches_oracle(device, B, T, H, C):
    import kda_gated_delta_core_amd as kda
    announce(f"kda_chunk_prefill_fused B={B} T={T} H={H} C={C}")
    fx, core, t_pad = _inputs(9000 + T + C, B, T, H, C)
    out, st, cst = _fused(kda, fx, core, H, T, C)
    o_ref, s_ref, c_ref = _oracle(fx, core, H, T)
    assert_close("out", host(out)[:, :T], o_ref)
    assert_close("state", host(st), s_ref)
    assert np.array_equal(host(cst), c_ref), "conv state"
    assert np.all(host(out)[:, T:] == SENTINEL), "rows >= T of out were written"


def test_fused_prefill_against_the_separate_calls(device):
    """the same inputs through kda_prefill_front_end + kda_chunk_prefill: outputs and state within the
    tolerance of each other, the conv state bit for bit"""
    import kda_gated_delta_core_amd as kda
    B, T, H, C = 2, 300, 4, 64
    announce(f"kda_chunk_prefill_fused vs separate calls B={B} T={T} H={H} C={C}")
    fx, core, t_pad = _inputs(9100, B, T, H, C)
    out, st, cst = _fused(kda, fx, core, H, T, C)
    cst2 = torch.from_numpy(fx["conv_state"]).cuda()
    q, k, v = kda.kda_prefill_front_end(_bits_dev(fx["qkv"]), _bits_dev(fx["conv_w"]), cst2, H, C, ki.L2_EPS)
    st2 = torch.from_numpy(core["state"]).cuda()
    out2 = kda.kda_chunk_prefill(q, k, v, torch.from_numpy(core["gate"]).cuda(), torch.from_numpy(core["beta"]).cuda(),
                                 st2, T, C)
    torch.cuda.synchronize()
    assert_close("out vs separate", host(out)[:, :T], host(out2)[:, :T])
    assert_close("state vs separate", host(st), host(st2))
    assert torch.equal(cst, cst2)


def test_fused_prefill_continues_across_calls(device):
    """two fused calls (the second from the first's state and conv state) equal one call over both parts"""
    import kda_gated_delta_core_amd as kda
    B, T1, T2, H, C = 1, 70, 90, 2, 32
    announce(f"kda_chunk_prefill_fused split B={B} T={T1}+{T2} H={H} C={C}")
    fx, core, _ = _inputs(9200, B, T1 + T2, H, C)
    o_ref, s_ref, c_ref = _oracle(fx, core, H, T1 + T2)
    cst = torch.from_numpy(fx["conv_state"]).cuda()
    st = torch.from_numpy(core["state"]).cuda()
    outs = []
    for t0, t1 in ((0, T1), (T1, T1 + T2)):
        n = t1 - t0
        t_pad = -(-n // C) * C
        pad = lambda a: np.concatenate([a[:, t0:t1], np.zeros((B, t_pad - n) + a.shape[2:], np.float32)], 1)
        out = kda.kda_chunk_prefill_fused(_bits_dev(fx["qkv"][:, t0:t1]), _bits_dev(fx["conv_w"]), cst,
                                          torch.from_numpy(pad(core["gate"])).cuda(),
                                          torch.from_numpy(pad(core["beta"])).cuda(), st, C, ki.L2_EPS)
        outs.append(host(out)[:, :n])
    torch.cuda.synchronize()
    assert_close("out", np.concatenate(outs, axis=1), o_ref)
    assert_close("state", host(st), s_ref)
    assert np.array_equal(host(cst), c_ref)


def test_fused_prefill_full_size(device):
    """the T=8192, H=32, C=64 prefill with its front end"""
    import kda_gated_delta_core_amd as kda
    B, T, H, K_, C, seed = ki.PREFILL_FRONT_END_WORKLOADS["prefill_front_end_t8192_h32_k4"]
    announce(f"kda_chunk_prefill_fused B={B} T={T} H={H} C={C} seed={seed}")
    fx = ki.front_end_inputs(seed, B, T, H, K_)
    w = ki.WORKLOADS["prefill_h32_t8192_c64"]
    core = ki.workload_inputs(w)
    core = {n: (np.ascontiguousarray(a[:, :T + (-T) % C]) if n != "state" else a) for n, a in core.items()}
    out, st, cst = _fused(kda, fx, core, H, T, C)
    o_ref, s_ref, c_ref = _oracle(fx, core, H, T)
    assert_close("out", host(out)[:, :T], o_ref)
    assert_close("state", host(st), s_ref)
    assert np.array_equal(host(cst), c_ref)
