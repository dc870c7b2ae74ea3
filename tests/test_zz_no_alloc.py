"""kda_chunk_prefill_noalloc: the prefill with its chunk records in the library's static device
array.  Through the C ABI, its results must equal kda_chunk_prefill's (bit for bit: the same
kernels) and the fp64 oracle's, on two calls in a row, the second smaller than the first (the
array keeps the first call's records, which the second must not depend on)."""
import numpy as np
import pytest

import kda_inputs as ki
import oracle
from kda_testlib import SENTINEL, announce, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _inputs(seed, B, H, T, C):
    t_pad = -(-T // C) * C
    return ki.make_batch(seed, B, H, T, -5.0, 0.02, alloc_rows=t_pad, pad_value=float("nan"))


def _both(kda, x, B, H, T, C):
    import torch
    t_pad = -(-T // C) * C
    args = [dev(x[n]) for n in ("q", "k", "v", "gate", "beta")]
    st_ref, st_na = dev(x["state"]), dev(x["state"])
    out_ref = torch.full((B, t_pad, H, 128), SENTINEL, device="cuda")
    out_na = torch.full((B, t_pad, H, 128), SENTINEL, device="cuda")
    kda.kda_chunk_prefill(*args, st_ref, T, C, out=out_ref)
    torch.cuda.synchronize()
    free0 = torch.cuda.memory_allocated()
    kda.kda_chunk_prefill_noalloc(*args, st_na, T, C, out=out_na)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == free0
    return out_ref, st_ref, out_na, st_na


def test_noalloc_matches_prefill_two_calls(device):
    import torch
    import kda_gated_delta_core_amd as kda
    # the first call fills most of the array (1,536 records of 164,352 B at C=64), the second is smaller
    for seed, B, H, T, C in ((9301, 3, 32, 1000, 64), (9302, 2, 5, 77, 32)):
        announce(f"kda_chunk_prefill_noalloc seed={seed} B={B} H={H} T={T} C={C}")
        assert kda.kda_chunk_prefill_workspace_bytes(B, H, T, C) <= kda.STATIC_WORKSPACE_BYTES
        x = _inputs(seed, B, H, T, C)
        out_ref, st_ref, out_na, st_na = _both(kda, x, B, H, T, C)
        assert torch.equal(out_na, out_ref), "out differs from kda_chunk_prefill"
        assert torch.equal(st_na, st_ref), "state differs from kda_chunk_prefill"
        o = host(out_na)
        assert np.all(o[:, T:] == SENTINEL)
        o_ref, s_ref, _, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"], T=T)
        assert_close("core", o[:, :T], o_ref)
        assert_close("state", host(st_na), s_ref)


def test_noalloc_refuses_beyond_the_array(device):
    import torch
    import kda_gated_delta_core_amd as kda
    B, H, T, C = 1, 32, 8192, 64
    announce("kda_chunk_prefill_noalloc refusal above the static array")
    assert kda.kda_chunk_prefill_workspace_bytes(B, H, T, C) > kda.STATIC_WORKSPACE_BYTES
    z = lambda: torch.zeros((B, T, H, 128), device="cuda")
    st = torch.zeros((B, H, 128, 128), device="cuda")
    out = torch.full((B, T, H, 128), SENTINEL, device="cuda")
    with pytest.raises(kda.KdaError) as e:
        kda.kda_chunk_prefill_noalloc(z(), z(), z(), z(), torch.zeros((B, T, H), device="cuda"), st, T, C, out=out)
    assert e.value.status == kda.KDA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(out == SENTINEL)) and bool(torch.all(st == 0))
