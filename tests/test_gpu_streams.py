"""Concurrent calls on separate streams: every entry point, each on a stream of its own with buffers of
its own, launched back to back with no synchronisation between them, gives the bits of the same calls
made one after another on one stream.  The prefill's persistent workgroups and the others' grids then
share the compute units; no kernel waits on another workgroup, so none depends on having the device
to itself."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
from kda_testlib import announce

pytestmark = pytest.mark.gpu
D = 128


def _bits(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _jobs(kda):
    """(name, setup) pairs: setup() makes fresh device buffers and returns (launch(stream), results())."""
    jobs = []

    def prefill():
        B, H, T, C = 2, 16, 1000, 64
        t_pad = -(-T // C) * C
        x = ki.make_batch(1600, B, H, T, -5.0, 0.02, alloc_rows=t_pad)
        d = {n: torch.from_numpy(a).cuda() for n, a in x.items()}
        out = torch.zeros_like(d["q"])
        ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T, C), dtype=torch.uint8, device="cuda")
        launch = lambda s: kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["state"], T, C,
                                                 out=out, workspace=ws, stream=s)
        return launch, lambda: (out, d["state"])
    jobs.append(("kda_chunk_prefill B=2 H=16 T=1000", prefill))

    def varlen():
        lens = [300, 1, 129, 700]
        x = ki.varlen_inputs(1601, lens, 8, -5.0, 0.02)
        d = {n: torch.from_numpy(x[n]).cuda() for n in ("q", "k", "v", "gate", "beta", "state", "cu_seqlens")}
        out = torch.zeros_like(d["q"])
        ws = torch.empty(kda.kda_chunk_prefill_varlen_workspace_bytes(len(lens), 8, sum(lens), 64),
                         dtype=torch.uint8, device="cuda")
        launch = lambda s: kda.kda_chunk_prefill_varlen(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["state"],
                                                        d["cu_seqlens"], 64, out=out, workspace=ws, stream=s)
        return launch, lambda: (out, d["state"])
    jobs.append(("kda_chunk_prefill_varlen 4 sequences H=8", varlen))

    def decode_k():
        B, H, T = 16, 8, 4
        x = ki.make_batch(1602, B, H, T, -5.0, 0.02)
        d = {n: torch.from_numpy(a).cuda() for n, a in x.items()}
        out = torch.zeros((B, T, H, D), device="cuda")
        snaps = torch.zeros((T, B, H, D, D), device="cuda")
        launch = lambda s: kda.kda_recurrent_k(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["state"], out=out,
                                               snapshots=snaps, n_snapshots=T, stream=s)
        return launch, lambda: (out, d["state"], snaps)
    jobs.append(("kda_recurrent_k B=16 H=8 k=4", decode_k))

    def step():
        B, H = 32, 8
        x = ki.make_batch(1603, B, H, 1, -5.0, 0.02)
        d = {n: torch.from_numpy(a).cuda() for n, a in x.items()}
        out = torch.zeros((B, 1, H, D), device="cuda")
        launch = lambda s: kda.kda_recurrent_step(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["state"], out=out,
                                                  stream=s)
        return launch, lambda: (out, d["state"])
    jobs.append(("kda_recurrent_step B=32 H=8", step))

    def chain_bf16():
        B, T, H, K = 8, 3, 4, 4
        fx = ki.front_end_inputs(1604, B, T, H, K)
        core = ki.make_batch(1605, B, H, T, -5.0, 0.02)
        nx = ki.norm_inputs(1606, B * T, H)
        qkv, w = _bits(fx["qkv"]), _bits(fx["conv_w"])
        cst = torch.from_numpy(fx["conv_state"]).cuda()
        g, b = torch.from_numpy(core["gate"]).cuda(), torch.from_numpy(core["beta"]).cuda()
        st = torch.from_numpy(core["state"]).cuda()
        conv_out = torch.zeros((B, T, 3 * H * D), dtype=torch.bfloat16, device="cuda")
        out = torch.zeros((B, T, H, D), device="cuda")
        y = torch.zeros((B * T, H, D), dtype=torch.bfloat16, device="cuda")
        og, on = _bits(nx["out_gate"]), _bits(nx["o_norm"])

        def launch(s):
            kda.kda_decode_front_end_bf16(qkv, w, cst, H, ki.L2_EPS, conv_out=conv_out, stream=s)
            kda.kda_recurrent_k_bf16(conv_out, g, b, st, out=out, stream=s)
            kda.kda_gated_rmsnorm(out.view(B * T, H, D), og, on, ki.NORM_EPS, out=y, stream=s)
        return launch, lambda: (conv_out, cst, out, st, y)
    jobs.append(("BF16 front end -> kda_recurrent_k_bf16 -> kda_gated_rmsnorm B=8 T=3 H=4", chain_bf16))
    return jobs


def test_concurrent_streams_match_serial_calls_bitwise(device):
    import kda_gated_delta_core_amd as kda
    jobs = _jobs(kda)
    # serial: one job after another on the current stream
    serial = []
    for name, setup in jobs:
        announce(f"serial: {name}")
        launch, results = setup()
        launch(None)
        torch.cuda.synchronize()
        serial.append([t.clone() for t in results()])
    # concurrent: every job on a stream of its own, launched back to back; two rounds on fresh buffers
    for rnd in range(2):
        announce(f"concurrent round {rnd}: {len(jobs)} jobs on {len(jobs)} streams")
        streams = [torch.cuda.Stream() for _ in jobs]
        ready = [setup() for _, setup in jobs]
        torch.cuda.synchronize()
        for (launch, _), s in zip(ready, streams):
            launch(s)
        torch.cuda.synchronize()
        for (name, _), (_, results), ref in zip(jobs, ready, serial):
            got = results()
            assert all(torch.equal(a, b) for a, b in zip(got, ref)), name


def test_binding_workspace_is_not_handed_out_while_its_call_runs(device):
    """A workspace the binding allocates for a call on another stream is dropped when the call returns;
    its memory must not go to the next allocation on the current stream while the call still runs.
    The launch stream is held busy first (a bounded device sleep), then a buffer of the same size is
    allocated and filled on the current stream: it must keep its contents, and the prefill its bits."""
    import kda_gated_delta_core_amd as kda
    B, H, T, C = 1, 8, 640, 64
    announce(f"binding workspace on a side stream: kda_chunk_prefill B={B} H={H} T={T}")
    x = ki.make_batch(1610, B, H, T, -5.0, 0.02)
    d = {n: torch.from_numpy(a).cuda() for n, a in x.items()}
    ref_state = d["state"].clone()
    ref_out = kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["gate"], d["beta"], ref_state, T, C)
    torch.cuda.synchronize()
    nbytes = kda.kda_chunk_prefill_workspace_bytes(B, H, T, C)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = torch.zeros_like(d["q"])
    with torch.cuda.stream(side):
        torch.cuda._sleep(50_000_000)  # ~25 ms of device time on the side stream only
    kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["state"], T, C, out=out, stream=side)
    other = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    other.fill_(0xA5)  # runs at once on the idle current stream
    torch.cuda.synchronize()
    assert bool((other == 0xA5).all()), "the call's workspace memory was handed out while the call ran"
    assert torch.equal(out, ref_out) and torch.equal(d["state"], ref_state)


def test_calls_with_caller_buffers_allocate_nothing(device):
    """With every output and workspace passed in, a round of calls of every entry point leaves torch's
    allocator where it was (the library itself links no HIP allocation call)."""
    import kda_gated_delta_core_amd as kda
    jobs = _jobs(kda)
    ready = [setup() for _, setup in jobs]
    for launch, _ in ready:  # first round: any lazy initialisation of the runtime happens here
        launch(None)
    torch.cuda.synchronize()
    state = lambda: (torch.cuda.memory_stats()["allocation.all.allocated"], torch.cuda.memory_allocated(),
                     torch.cuda.memory_reserved())
    before = state()
    announce(f"allocator before: {before[0]} allocations so far, {before[1]} B allocated, {before[2]} B reserved")
    for _ in range(3):
        for launch, _ in ready:
            launch(None)
    torch.cuda.synchronize()
    assert state() == before, (before, state())
