"""HIP graph capture of the C ABI calls (torch.cuda.graph around the bindings): every replay equals
the eager calls bit for bit, with eager work, state resets and synchronisations between replays.
None of the entry points allocates, fills or copies, so their launches are all a graph records."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
from kda_testlib import announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def test_graph_replays_of_decode_steps_and_prefill(device):
    import kda_gated_delta_core_amd as kda
    B, H, steps, T, C = 4, 8, 6, 100, 64
    announce(f"graph capture: {steps} decode steps B={B} H={H}, then a prefill T={T}")
    x = ki.make_batch(1500, B, H, steps, -5.0, 0.02)
    d = {n: torch.from_numpy(a).cuda() for n, a in x.items()}
    rows = [{n: d[n][:, t:t + 1].contiguous() for n in ("q", "k", "v", "gate", "beta")} for t in range(steps)]
    t_pad = -(-T // C) * C
    p = ki.make_batch(1501, B, H, T, -5.0, 0.02, alloc_rows=t_pad)
    pd = {n: torch.from_numpy(a).cuda() for n, a in p.items()}
    ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T, C), dtype=torch.uint8, device="cuda")

    state = torch.empty_like(d["state"])
    outs = [torch.empty_like(rows[0]["q"]) for _ in range(steps)]
    pstate = torch.empty_like(pd["state"])
    pout = torch.zeros_like(pd["q"])

    def work(stream=None):
        for t in range(steps):
            r = rows[t]
            kda.kda_recurrent_step(r["q"], r["k"], r["v"], r["gate"], r["beta"], state, out=outs[t], stream=stream)
        kda.kda_chunk_prefill(pd["q"], pd["k"], pd["v"], pd["gate"], pd["beta"], pstate, T, C, out=pout,
                              workspace=ws, stream=stream)

    # eager reference
    state.copy_(d["state"]); pstate.copy_(pd["state"])
    work()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs] + [state.clone(), pout.clone(), pstate.clone()]

    g = torch.cuda.graph_pool_handle()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        state.copy_(d["state"]); pstate.copy_(pd["state"])
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, pool=g, stream=s):
            work(stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        # eager work of the program between replays, then reset the carried states
        kda.kda_recurrent_step(rows[0]["q"], rows[0]["k"], rows[0]["v"], rows[0]["gate"], rows[0]["beta"],
                               torch.zeros_like(state))
        state.copy_(d["state"]); pstate.copy_(pd["state"])
        for o in outs:
            o.fill_(np.nan)
        pout.fill_(np.nan)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outs + [state, pout, pstate]
        for i, (a, b) in enumerate(zip(got, ref)):
            if i == len(got) - 2:  # prefill output: rows < T only (rows >= T are not written)
                a, b = a[:, :T], b[:, :T]
            assert torch.equal(a, b), f"replay {rep}, tensor {i}"


def _capture_and_replay(kda, name, work, reset, results, reps=3):
    """Eager reference, capture `work` on a side stream, then replays with eager work, resets and
    synchronisations between them; every replay must equal the eager run bit for bit."""
    reset()
    work(None)
    torch.cuda.synchronize()
    ref = [t.clone() for t in results()]
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, pool=torch.cuda.graph_pool_handle(), stream=s):
            work(s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(reps):
        for t in results():  # outputs poisoned first, then the carried states (also results) restored
            if t.is_floating_point():
                t.fill_(float("nan"))
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(results(), ref)):
            assert torch.equal(a, b), f"{name}: replay {rep}, tensor {i}"


def _bits(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def test_graph_replays_of_the_bf16_decode_chain(device):
    """BF16 front end -> kda_recurrent_k_bf16 (snapshots) -> gated RMSNorm, captured as one graph."""
    import kda_gated_delta_core_amd as kda
    B, T, H, K = 8, 4, 4, 4
    announce(f"graph capture: BF16 decode chain B={B} k={T} H={H}")
    fx = ki.front_end_inputs(1510, B, T, H, K)
    core = ki.make_batch(1511, B, H, T, -5.0, 0.02)
    nx = ki.norm_inputs(1512, B * T, H)
    qkv, w, og, on = _bits(fx["qkv"]), _bits(fx["conv_w"]), _bits(nx["out_gate"]), _bits(nx["o_norm"])
    g, b = torch.from_numpy(core["gate"]).cuda(), torch.from_numpy(core["beta"]).cuda()
    cst0, st0 = torch.from_numpy(fx["conv_state"]).cuda(), torch.from_numpy(core["state"]).cuda()
    cst, st = torch.empty_like(cst0), torch.empty_like(st0)
    conv_out = torch.empty((B, T, 3 * H * 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, T, H, 128), device="cuda")
    snaps = torch.empty((T, B, H, 128, 128), device="cuda")
    y = torch.empty((B * T, H, 128), dtype=torch.bfloat16, device="cuda")

    def work(s):
        kda.kda_decode_front_end_bf16(qkv, w, cst, H, ki.L2_EPS, conv_out=conv_out, stream=s)
        kda.kda_recurrent_k_bf16(conv_out, g, b, st, out=out, snapshots=snaps, n_snapshots=T, stream=s)
        kda.kda_gated_rmsnorm(out.view(B * T, H, 128), og, on, ki.NORM_EPS, out=y, stream=s)

    def reset():
        cst.copy_(cst0)
        st.copy_(st0)

    _capture_and_replay(kda, "BF16 decode chain", work, reset, lambda: (conv_out, cst, out, st, snaps, y))


def test_graph_replays_of_the_prefill_chain(device):
    """Prefill front end -> chunked prefill -> gated RMSNorm, and a varlen prefill, captured as one graph."""
    import kda_gated_delta_core_amd as kda
    B, T, H, K, C = 2, 300, 4, 4, 64
    announce(f"graph capture: prefill chain B={B} T={T} H={H}, varlen prefill")
    t_pad = -(-T // C) * C
    fx = ki.front_end_inputs(1520, B, T, H, K)
    core = ki.make_batch(1521, B, H, T, -5.0, 0.02, alloc_rows=t_pad)
    nx = ki.norm_inputs(1522, B * t_pad, H)
    qkv, w, og, on = _bits(fx["qkv"]), _bits(fx["conv_w"]), _bits(nx["out_gate"]), _bits(nx["o_norm"])
    g, b = torch.from_numpy(core["gate"]).cuda(), torch.from_numpy(core["beta"]).cuda()
    cst0, st0 = torch.from_numpy(fx["conv_state"]).cuda(), torch.from_numpy(core["state"]).cuda()
    cst, st = torch.empty_like(cst0), torch.empty_like(st0)
    q, k, v = (torch.zeros((B, t_pad, H, 128), device="cuda") for _ in range(3))
    out = torch.zeros((B, t_pad, H, 128), device="cuda")
    ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T, C), dtype=torch.uint8, device="cuda")
    y = torch.empty((B * t_pad, H, 128), dtype=torch.bfloat16, device="cuda")
    lens = [100, 1, 257]
    vx = ki.varlen_inputs(1523, lens, H, -5.0, 0.02)
    vd = {n: torch.from_numpy(vx[n]).cuda() for n in ("q", "k", "v", "gate", "beta", "cu_seqlens")}
    vst0 = torch.from_numpy(vx["state"]).cuda()
    vst, vout = torch.empty_like(vst0), torch.zeros_like(vd["q"])
    vws = torch.empty(kda.kda_chunk_prefill_varlen_workspace_bytes(len(lens), H, sum(lens), C), dtype=torch.uint8,
                      device="cuda")

    def work(s):
        kda.kda_prefill_front_end(qkv, w, cst, H, C, ki.L2_EPS, q=q, k=k, v=v, stream=s)
        kda.kda_chunk_prefill(q, k, v, g, b, st, T, C, out=out, workspace=ws, stream=s)
        kda.kda_gated_rmsnorm(out.view(B * t_pad, H, 128), og, on, ki.NORM_EPS, out=y, stream=s)
        kda.kda_chunk_prefill_varlen(vd["q"], vd["k"], vd["v"], vd["gate"], vd["beta"], vst, vd["cu_seqlens"], C,
                                     out=vout, workspace=vws, stream=s)

    def reset():
        cst.copy_(cst0)
        st.copy_(st0)
        vst.copy_(vst0)

    # rows >= T of q, k, v and out are never written: compare rows < T; those rows stay zero, so the
    # norm's rows for them are zero too and the whole norm output is compared
    _capture_and_replay(kda, "prefill chain", work, reset,
                        lambda: (q[:, :T], k[:, :T], v[:, :T], cst, out[:, :T], st, y, vout, vst))


def test_graph_replays_of_the_segment_split(device):
    """Two segments' transitions, the fold of the first into the sequence's state, and the second
    segment's prefill from the folded state, captured as one graph."""
    import kda_gated_delta_core_amd as kda
    B, H, C = 2, 3, 64
    T1, T2 = 150, 90
    announce(f"graph capture: segment transitions + fold + prefill B={B} H={H} T1={T1} T2={T2}")
    x = ki.make_batch(1530, B, H, T1 + T2, -3.0, 0.05)

    def seg(t0, t1):
        t_pad = -(-(t1 - t0) // C) * C
        res = {}
        for n in ("q", "k", "v", "gate", "beta"):
            a = x[n][:, t0:t1]
            res[n] = torch.from_numpy(np.ascontiguousarray(
                np.concatenate([a, np.zeros((B, t_pad - (t1 - t0)) + a.shape[2:], np.float32)], 1))).cuda()
        return res

    s1, s2 = seg(0, T1), seg(T1, T1 + T2)
    st0 = torch.from_numpy(x["state"]).cuda()
    st = torch.empty_like(st0)
    P1, Q1, P2, Q2 = (torch.empty((B, H, 128, 128), device="cuda") for _ in range(4))
    out2 = torch.zeros((B, s2["q"].shape[1], H, 128), device="cuda")
    ws1 = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T1, C), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T2, C), dtype=torch.uint8, device="cuda")

    def work(s):
        kda.kda_chunk_prefill_transition(*(s1[n] for n in ("q", "k", "v", "gate", "beta")), T1, C, trans_p=P1,
                                         trans_q=Q1, workspace=ws1, stream=s)
        kda.kda_chunk_prefill_transition(*(s2[n] for n in ("q", "k", "v", "gate", "beta")), T2, C, trans_p=P2,
                                         trans_q=Q2, workspace=ws2, stream=s)
        kda.kda_state_transition_apply(P1, Q1, st, stream=s)
        kda.kda_chunk_prefill(*(s2[n] for n in ("q", "k", "v", "gate", "beta")), st, T2, C, out=out2,
                              workspace=ws2, stream=s)

    def reset():
        st.copy_(st0)

    _capture_and_replay(kda, "segment split", work, reset, lambda: (P1, Q1, P2, Q2, st, out2[:, :T2]))


def test_graph_replays_of_the_fused_prefills(device):
    """kda_chunk_prefill_fused and kda_chunk_prefill_varlen_fused captured as one graph"""
    import kda_gated_delta_core_amd as kda
    B, T, H, C = 2, 150, 3, 64
    announce(f"graph capture: fused prefill B={B} T={T} H={H}, varlen fused prefill")
    t_pad = -(-T // C) * C
    fx = ki.front_end_inputs(1540, B, T, H, 4)
    core = ki.make_batch(1541, B, H, T, -5.0, 0.02, alloc_rows=t_pad)
    qkv, w = _bits(fx["qkv"]), _bits(fx["conv_w"])
    g, b = torch.from_numpy(core["gate"]).cuda(), torch.from_numpy(core["beta"]).cuda()
    cst0, st0 = torch.from_numpy(fx["conv_state"]).cuda(), torch.from_numpy(core["state"]).cuda()
    cst, st = torch.empty_like(cst0), torch.empty_like(st0)
    out = torch.zeros((B, t_pad, H, 128), device="cuda")
    ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T, C), dtype=torch.uint8, device="cuda")
    lens = [70, 0, 1, 130]
    vfx = ki.front_end_inputs(1542, 1, sum(lens), H, 4)
    vcst0 = torch.from_numpy(ki.front_end_inputs(1543, len(lens), 1, H, 4)["conv_state"]).cuda()
    vx = ki.varlen_inputs(1544, lens, H, -5.0, 0.02)
    vd = {n: torch.from_numpy(vx[n]).cuda() for n in ("gate", "beta", "cu_seqlens")}
    vqkv = _bits(vfx["qkv"][0])
    vst0 = torch.from_numpy(vx["state"]).cuda()
    vcst, vst = torch.empty_like(vcst0), torch.empty_like(vst0)
    vout = torch.zeros((sum(lens), H, 128), device="cuda")
    vws = torch.empty(kda.kda_chunk_prefill_varlen_workspace_bytes(len(lens), H, sum(lens), C), dtype=torch.uint8,
                      device="cuda")

    def work(s):
        kda.kda_chunk_prefill_fused(qkv, w, cst, g, b, st, C, ki.L2_EPS, out=out, workspace=ws, stream=s)
        kda.kda_chunk_prefill_varlen_fused(vqkv, w, vcst, vd["gate"], vd["beta"], vst, vd["cu_seqlens"], C,
                                           ki.L2_EPS, out=vout, workspace=vws, stream=s)

    def reset():
        cst.copy_(cst0)
        st.copy_(st0)
        vcst.copy_(vcst0)
        vst.copy_(vst0)

    _capture_and_replay(kda, "fused prefills", work, reset, lambda: (out[:, :T], st, cst, vout, vst, vcst))


def test_graph_replays_of_the_fused_decode(device):
    """kda_decode_fused_step and kda_decode_fused_k_gated (3 rows, snapshots of both states) captured as one
    graph, the form the decode loop replays."""
    import kda_gated_delta_core_amd as kda
    B, H, K, T = 8, 4, 4, 3
    announce(f"graph capture: fused decode step B={B} H={H}, gated fused walk k={T}")
    fx1 = ki.front_end_inputs(1550, B, 1, H, K)
    c1 = ki.make_batch(1551, B, H, 1, -5.0, 0.02)
    n1 = ki.norm_inputs(1552, B, H)
    fx2 = ki.front_end_inputs(1553, B, T, H, K)
    c2 = ki.make_batch(1554, B, H, T, -5.0, 0.02)
    n2 = ki.norm_inputs(1555, B * T, H)
    gx = ki.gate_inputs(1556, B, T, H)
    q1, w1, og1, on1 = _bits(fx1["qkv"]), _bits(fx1["conv_w"]), _bits(n1["out_gate"]).view(B, 1, H, 128), \
        _bits(n1["o_norm"])
    q2, w2, og2, on2 = _bits(fx2["qkv"]), _bits(fx2["conv_w"]), _bits(n2["out_gate"]).view(B, T, H, 128), \
        _bits(n2["o_norm"])
    g1, b1 = torch.from_numpy(c1["gate"]).cuda(), torch.from_numpy(c1["beta"]).cuda()
    graw, blog = _bits(gx["g_raw"]), torch.from_numpy(gx["beta_logit"]).cuda()
    dtb, alog = torch.from_numpy(gx["dt_bias"]).cuda(), torch.from_numpy(gx["a_log"]).cuda()
    cs10, st10 = torch.from_numpy(fx1["conv_state"]).cuda(), torch.from_numpy(c1["state"]).cuda()
    cs20, st20 = torch.from_numpy(fx2["conv_state"]).cuda(), torch.from_numpy(c2["state"]).cuda()
    cs1, st1, cs2, st2 = (torch.empty_like(t) for t in (cs10, st10, cs20, st20))
    y1 = torch.empty((B, 1, H, 128), dtype=torch.bfloat16, device="cuda")
    o1 = torch.empty((B, 1, H, 128), device="cuda")
    y2 = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty((B, T, H, 128), device="cuda")
    snaps = torch.empty((T, B, H, 128, 128), device="cuda")
    csn = torch.empty((T,) + tuple(cs20.shape), device="cuda")

    def work(s):
        kda.kda_decode_fused_step(q1, w1, cs1, g1, b1, st1, og1, on1, H, ki.NORM_EPS, ki.L2_EPS, y=y1, out=o1,
                                  stream=s)
        kda.kda_decode_fused_k_gated(q2, w2, cs2, graw, blog, dtb, alog, ki.GATE_LOWER_BOUND, st2, og2, on2, H,
                                     ki.NORM_EPS, ki.L2_EPS, y=y2, out=o2, snapshots=snaps, conv_snapshots=csn,
                                     n_snapshots=T, stream=s)

    def reset():
        cs1.copy_(cs10)
        st1.copy_(st10)
        cs2.copy_(cs20)
        st2.copy_(st20)

    _capture_and_replay(kda, "fused decode", work, reset, lambda: (y1, o1, st1, cs1, y2, o2, st2, cs2, snaps, csn))


def test_graph_replays_of_the_bf16_prefill(device):
    """kda_chunk_prefill_bf16 (BF16 q | k | v packed per token) captured as one graph."""
    import kda_gated_delta_core_amd as kda
    B, T, H, C = 2, 150, 3, 64
    announce(f"graph capture: BF16 prefill B={B} T={T} H={H}")
    t_pad = -(-T // C) * C
    x = ki.make_batch(1560, B, H, T, -5.0, 0.02, alloc_rows=t_pad)
    bits = np.stack([ki.to_bf16_bits(x[n]) for n in ("q", "k", "v")], axis=2)
    qkv = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    g, b = torch.from_numpy(x["gate"]).cuda(), torch.from_numpy(x["beta"]).cuda()
    st0 = torch.from_numpy(x["state"]).cuda()
    st = torch.empty_like(st0)
    out = torch.zeros((B, t_pad, H, 128), device="cuda")
    ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T, C), dtype=torch.uint8, device="cuda")

    def work(s):
        kda.kda_chunk_prefill_bf16(qkv, g, b, st, T, C, out=out, workspace=ws, stream=s)

    def reset():
        st.copy_(st0)

    _capture_and_replay(kda, "BF16 prefill", work, reset, lambda: (out[:, :T], st))
