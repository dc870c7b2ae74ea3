"""GPU parity of kda_chunk_prefill_varlen (through the C ABI): against the fp64 oracle run on each
sequence, and bit for bit against kda_chunk_prefill on each sequence alone."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testlib import announce, assert_close

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _run_varlen(kda, x, C, cu=None, out_fill=None):
    d = {n: torch.from_numpy(x[n]).cuda() for n in ("q", "k", "v", "gate", "beta", "state")}
    cu_t = torch.from_numpy(np.asarray(x["cu_seqlens"] if cu is None else cu, dtype=np.int32)).cuda()
    out = torch.full_like(d["q"], np.nan if out_fill is None else out_fill)
    kda.kda_chunk_prefill_varlen(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["state"], cu_t, C, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), d["state"].cpu().numpy()


def _check_sequences(x, cu, out, st, heads=None):
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        n = b - a
        if n == 0:
            assert np.array_equal(st[s], x["state"][s]), f"seq {s}: empty sequence changed its state"
            continue
        hs = range(x["q"].shape[1]) if heads is None else heads
        for h in hs:
            sl = lambda name: np.ascontiguousarray(x[name][a:b, h:h + 1][None])
            o, sref, _, _ = oracle.serial(sl("q"), sl("k"), sl("v"), sl("gate"), sl("beta")[..., :],
                                          x["state"][s:s + 1, h:h + 1])
            assert_close(f"seq {s} (len {n}) h{h} out", out[None, a:b, h:h + 1], o)
            assert_close(f"seq {s} (len {n}) h{h} state", st[s:s + 1, h:h + 1], sref)


@pytest.mark.parametrize("C", [16, 32, 64])
def test_varlen_matches_oracle(device, C):
    import kda_gated_delta_core_amd as kda
    lens = [0, 1, C - 1, C, C + 1, 2 * C + 5, 3, 0, 130]
    announce(f"kda_chunk_prefill_varlen C={C} lengths={lens}")
    x = ki.varlen_inputs(400 + C, lens, 3, -5.0, 0.02)
    out, st = _run_varlen(kda, x, C)
    _check_sequences(x, x["cu_seqlens"], out, st)


@pytest.mark.parametrize("C", [16, 64])
def test_varlen_equals_dense_per_sequence_bitwise(device, C):
    import kda_gated_delta_core_amd as kda
    lens = [200, 1, 63, 64, 65, 7, 128]
    H = 4
    announce(f"kda_chunk_prefill_varlen vs kda_chunk_prefill, C={C}")
    x = ki.varlen_inputs(500 + C, lens, H, -5.0, 0.02)
    out, st = _run_varlen(kda, x, C)
    cu = x["cu_seqlens"]
    for s, n in enumerate(lens):
        t_pad = -(-n // C) * C
        dd = {}
        for name in ("q", "k", "v", "gate"):
            a = np.zeros((1, t_pad, H, D), dtype=np.float32)
            a[0, :n] = x[name][cu[s]:cu[s + 1]]
            dd[name] = torch.from_numpy(a).cuda()
        bb = np.zeros((1, t_pad, H), dtype=np.float32)
        bb[0, :n] = x["beta"][cu[s]:cu[s + 1]]
        dd["beta"] = torch.from_numpy(bb).cuda()
        st1 = torch.from_numpy(x["state"][s:s + 1].copy()).cuda()
        o1 = kda.kda_chunk_prefill(dd["q"], dd["k"], dd["v"], dd["gate"], dd["beta"], st1, n, C)
        torch.cuda.synchronize()
        assert np.array_equal(o1.cpu().numpy()[0, :n], out[cu[s]:cu[s + 1]]), f"seq {s} out"
        assert np.array_equal(st1.cpu().numpy()[0], st[s]), f"seq {s} state"


def test_varlen_rows_outside_sequences_and_offsets_out_of_range(device):
    """Tokens after the last sequence are not written; offsets that decrease or pass the token count
    are clamped to [0, total] and raised to the largest before them (documented), so the call stays
    inside the buffers and computes the clamped sequences."""
    import kda_gated_delta_core_amd as kda
    announce("kda_chunk_prefill_varlen pad tokens and clamped offsets")
    lens = [40, 70, 5]
    x = ki.varlen_inputs(600, lens, 2, -5.0, 0.02, pad_tokens=37)
    out, st = _run_varlen(kda, x, 64, out_fill=123.0)
    total_used = sum(lens)
    assert np.all(out[total_used:] == 123.0)
    _check_sequences(x, x["cu_seqlens"], out, st)
    total = x["q"].shape[0]
    bad = np.array([0, 60, 30, 500, 10**9], dtype=np.int32)   # decreasing, then past the end
    clean = np.maximum.accumulate(np.clip(bad, 0, total))     # [0, 60, 60, total, total]
    out2, st2 = _run_varlen(kda, dict(x, state=np.concatenate([x["state"], x["state"][:1]])), 64, cu=bad)
    x2 = dict(x, state=np.concatenate([x["state"], x["state"][:1]]))
    _check_sequences(x2, clean, out2, st2)


def test_varlen_many_sequences(device):
    """More sequences than the set-up kernel has threads (several offsets per thread)."""
    import kda_gated_delta_core_amd as kda
    g = np.random.default_rng(7)
    lens = [int(n) for n in g.integers(0, 9, size=2500)]
    announce(f"kda_chunk_prefill_varlen {len(lens)} sequences")
    x = ki.varlen_inputs(700, lens, 1, -5.0, 0.02)
    out, st = _run_varlen(kda, x, 16)
    cu = x["cu_seqlens"]
    # every sequence through the oracle at once: batch them by padding is not bitwise, so sample
    for s in list(range(0, len(lens), 97)) + [len(lens) - 1]:
        n = cu[s + 1] - cu[s]
        if n == 0:
            assert np.array_equal(st[s], x["state"][s])
            continue
        sl = lambda name: np.ascontiguousarray(x[name][cu[s]:cu[s + 1]][None])
        o, sref, _, _ = oracle.serial(sl("q"), sl("k"), sl("v"), sl("gate"), sl("beta"), x["state"][s:s + 1])
        assert_close(f"seq {s} out", out[None, cu[s]:cu[s + 1]], o)
        assert_close(f"seq {s} state", st[s:s + 1], sref)


@pytest.mark.timeout(600)
def test_varlen_workload_sampled(device):
    """The benchmarked mix (32768 tokens, H=32, C=64), two heads of every sequence against the oracle."""
    import kda_gated_delta_core_amd as kda
    total, H, C, mean, seed = ki.VARLEN_WORKLOADS["prefill_varlen_h32_t32768_c64"]
    lens = ki.varlen_lengths(seed, total, mean)
    announce(f"kda_chunk_prefill_varlen workload: {len(lens)} sequences, {total} tokens")
    x = ki.varlen_inputs(seed, lens, H, -5.0, 0.02)
    out, st = _run_varlen(kda, x, C)
    _check_sequences(x, x["cu_seqlens"], out, st, heads=[0, 31])
