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
