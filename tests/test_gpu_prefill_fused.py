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


def _varlen(seed, lens, H, gate_lo=-5.0):
    total = sum(lens)
    fx = ki.front_end_inputs(seed, 1, total, H, K)
    cst = ki.front_end_inputs(seed + 1, len(lens), 1, H, K)["conv_state"]  # one conv state per sequence
    core = ki.varlen_inputs(seed + 2, lens, H, gate_lo, 0.02)
    return fx["qkv"][0], fx["conv_w"], cst, core


def _varlen_fused(kda, qkv, w, cst, core, C):
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    cst_d, st = d(cst), d(core["state"])
    out = torch.full(core["q"].shape, SENTINEL, device="cuda")
    kda.kda_chunk_prefill_varlen_fused(_bits_dev(qkv), _bits_dev(w), cst_d, d(core["gate"]), d(core["beta"]), st,
                                       d(core["cu_seqlens"]), C, ki.L2_EPS, out=out)
    torch.cuda.synchronize()
    return out, st, cst_d


@pytest.mark.parametrize("C", [16, 64])
def test_varlen_fused_prefill_matches_oracle(device, C):
    """per sequence: the oracle's front end from that sequence's conv state, then its recurrence from that
    sequence's state; empty and one-token sequences included"""
    import kda_gated_delta_core_amd as kda
    lens, H = [100, 1, 0, 257, 64, 3], 2
    announce(f"kda_chunk_prefill_varlen_fused lens={lens} H={H} C={C}")
    qkv, w, cst, core = _varlen(9300 + C, lens, H)
    out, st, cst_d = _varlen_fused(kda, qkv, w, cst, core, C)
    cu = core["cu_seqlens"]
    got_out, got_st, got_cst = host(out), host(st), host(cst_d)
    for s, n in enumerate(lens):
        a, e = int(cu[s]), int(cu[s + 1])
        if n == 0:
            assert np.array_equal(got_st[s], core["state"][s]) and np.array_equal(got_cst[s], cst[s])
            continue
        q, k, v, c_ref, _ = oracle.decode_front_end(qkv[None, a:e], w, cst[s:s + 1], H, ki.L2_EPS)
        o_ref, s_ref, _, _ = oracle.serial(q, k, v, core["gate"][None, a:e], core["beta"][None, a:e],
                                           core["state"][s:s + 1])
        assert_close(f"seq {s} out", got_out[a:e], o_ref[0])
        assert_close(f"seq {s} state", got_st[s], s_ref[0])
        assert np.array_equal(got_cst[s], c_ref[0]), f"seq {s} conv state"


def test_varlen_fused_prefill_against_the_separate_calls(device):
    import kda_gated_delta_core_amd as kda
    lens, H, C = [300, 77, 1, 640], 3, 64
    announce(f"kda_chunk_prefill_varlen_fused vs separate calls lens={lens} H={H} C={C}")
    qkv, w, cst, core = _varlen(9400, lens, H)
    out, st, cst_d = _varlen_fused(kda, qkv, w, cst, core, C)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    cst2, st2, cu = d(cst), d(core["state"]), d(core["cu_seqlens"])
    q, k, v = kda.kda_prefill_front_end_varlen(_bits_dev(qkv), _bits_dev(w), cst2, cu, H, ki.L2_EPS)
    out2 = kda.kda_chunk_prefill_varlen(q, k, v, d(core["gate"]), d(core["beta"]), st2, cu, C)
    torch.cuda.synchronize()
    assert_close("out vs separate", host(out), host(out2))
    assert_close("state vs separate", host(st), host(st2))
    assert torch.equal(cst_d, cst2)


def _gate_inputs_padded(seed, B, T, H, t_pad):
    """kda_gate inputs with NaN in the pad rows (rows >= T), which the prefill must ignore."""
    gx = ki.gate_inputs(seed, B, t_pad, H)
    gx["g_raw"][:, T:] = 0x7FC0            # BF16 NaN
    gx["beta_logit"][:, T:] = np.nan
    return gx


def _gate_dev(gx):
    return (_bits_dev(gx["g_raw"]), torch.from_numpy(gx["beta_logit"]).cuda(), torch.from_numpy(gx["dt_bias"]).cuda(),
            torch.from_numpy(gx["a_log"]).cuda())


@pytest.mark.parametrize("B,T,H,C", [(1, 64, 2, 16), (2, 100, 3, 32), (1, 130, 2, 64), (2, 1, 1, 64)])
def test_fused_gated_prefill_matches_oracle(device, B, T, H, C):
    """kda_chunk_prefill_fused_gated against the oracle's front end, kda_gate and sigmoid, then its
    recurrence; pad rows of every input hold NaN and must not reach a result"""
    import kda_gated_delta_core_amd as kda
    announce(f"kda_chunk_prefill_fused_gated B={B} T={T} H={H} C={C}")
    fx, core, t_pad = _inputs(9300 + T + C, B, T, H, C)
    gx = _gate_inputs_padded(9350 + T, B, T, H, t_pad)
    cst = torch.from_numpy(fx["conv_state"]).cuda()
    st = torch.from_numpy(core["state"]).cuda()
    out = torch.full((B, t_pad, H, D), SENTINEL, device="cuda")
    kda.kda_chunk_prefill_fused_gated(_bits_dev(fx["qkv"]), _bits_dev(fx["conv_w"]), cst, *_gate_dev(gx),
                                      ki.GATE_LOWER_BOUND, st, C, ki.L2_EPS, out=out)
    torch.cuda.synchronize()
    q, k, v, c_ref, _ = oracle.decode_front_end(fx["qkv"], fx["conv_w"], fx["conv_state"], H, ki.L2_EPS)
    gate = oracle.kda_gate(gx["g_raw"][:, :T], gx["dt_bias"], gx["a_log"], ki.GATE_LOWER_BOUND).astype(np.float32)
    beta = oracle.sigmoid(gx["beta_logit"][:, :T]).astype(np.float32)
    o_ref, s_ref, _, _ = oracle.serial(q, k, v, gate, beta, core["state"])
    assert_close("out", host(out)[:, :T], o_ref)
    assert_close("state", host(st), s_ref)
    assert np.array_equal(host(cst), c_ref), "conv state"
    assert np.all(host(out)[:, T:] == SENTINEL), "rows >= T of out were written"


def test_fused_gated_prefill_against_the_separate_calls(device):
    """kda_prefill_front_end + kda_chunk_prefill_gated on the same inputs: within tolerance, conv state
    bit for bit"""
    import kda_gated_delta_core_amd as kda
    B, T, H, C = 2, 1000, 8, 64
    announce(f"kda_chunk_prefill_fused_gated vs separate calls B={B} T={T} H={H} C={C}")
    fx, core, t_pad = _inputs(9400, B, T, H, C)
    gx = _gate_inputs_padded(9450, B, T, H, t_pad)
    g = _gate_dev(gx)
    cst = torch.from_numpy(fx["conv_state"]).cuda()
    st = torch.from_numpy(core["state"]).cuda()
    out = kda.kda_chunk_prefill_fused_gated(_bits_dev(fx["qkv"]), _bits_dev(fx["conv_w"]), cst, *g,
                                            ki.GATE_LOWER_BOUND, st, C, ki.L2_EPS)
    cst2 = torch.from_numpy(fx["conv_state"]).cuda()
    q, k, v = kda.kda_prefill_front_end(_bits_dev(fx["qkv"]), _bits_dev(fx["conv_w"]), cst2, H, C, ki.L2_EPS)
    st2 = torch.from_numpy(core["state"]).cuda()
    out2 = kda.kda_chunk_prefill_gated(q, k, v, *g, ki.GATE_LOWER_BOUND, st2, T, C)
    torch.cuda.synchronize()
    assert_close("out vs separate", host(out)[:, :T], host(out2)[:, :T])
    assert_close("state vs separate", host(st), host(st2))
    assert torch.equal(cst, cst2)
