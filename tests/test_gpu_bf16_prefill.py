"""GPU parity of kda_chunk_prefill_bf16 (BF16 q | k | v packed per token), through the C ABI: bit for bit
equal to kda_chunk_prefill on the widened values at every chunk width, ragged lengths, pads of NaN and
steep gates, and against the fp64 oracle on every head at T=8192 H=32."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testlib import SENTINEL, announce, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _bf16(x):
    """FP32 array -> (BF16 bit patterns, the same values widened to FP32)."""
    bits = ki.to_bf16_bits(x)
    return bits, (bits.astype(np.uint32) << 16).view(np.float32)


def _packed(x, rows):
    """q, k, v of a batch as BF16 [B][rows][3][H][128] bits (rows >= T hold what the batch holds there) and
    the widened FP32 q, k, v."""
    parts = [_bf16(np.ascontiguousarray(x[n][:, :rows])) for n in ("q", "k", "v")]
    packed = np.ascontiguousarray(np.stack([p[0] for p in parts], axis=2))
    return packed, [p[1] for p in parts]


def _bits_dev(a):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def _both(kda, x, T, C):
    B, _, H, _ = x["q"].shape
    t_pad = -(-T // C) * C
    packed, (qw, kw, vw) = _packed(x, t_pad)
    g, b = dev(np.ascontiguousarray(x["gate"][:, :t_pad])), dev(np.ascontiguousarray(x["beta"][:, :t_pad]))
    st16, st32 = dev(x["state"]), dev(x["state"])
    o16 = torch.full((B, t_pad, H, 128), SENTINEL, device="cuda")
    o32 = torch.full((B, t_pad, H, 128), SENTINEL, device="cuda")
    kda.kda_chunk_prefill_bf16(_bits_dev(packed), g, b, st16, T, C, out=o16)
    kda.kda_chunk_prefill(dev(qw), dev(kw), dev(vw), g, b, st32, T, C, out=o32)
    torch.cuda.synchronize()
    return (o16, st16), (o32, st32), (qw, kw, vw)


@pytest.mark.parametrize("B,H,T,C,lo", [(1, 1, 64, 64, -5.0), (2, 3, 150, 64, -5.0), (1, 4, 77, 32, -5.0),
                                        (3, 2, 40, 16, -5.0), (1, 2, 200, 64, -30.0), (2, 5, 1000, 64, -0.5)])
def test_bf16_prefill_equals_fp32_on_widened_inputs(device, B, H, T, C, lo):
    import kda_gated_delta_core_amd as kda
    announce(f"kda_chunk_prefill_bf16 B={B} H={H} T={T} C={C} gates [{lo}, 0]")
    t_pad = -(-T // C) * C
    x = ki.make_batch(9400 + T + C, B, H, T, lo, 0.02, alloc_rows=t_pad, pad_value=float("nan"))
    (o16, s16), (o32, s32), _ = _both(kda, x, T, C)
    assert torch.equal(o16, o32), "out differs from kda_chunk_prefill on the widened inputs"
    assert torch.equal(s16, s32), "state differs from kda_chunk_prefill on the widened inputs"
    assert bool((o16[:, T:] == SENTINEL).all()), "rows >= T of out were written"


def test_bf16_prefill_full_size_matches_oracle(device):
    """The T=8192 H=32 C=64 workload with q, k, v rounded to BF16; the oracle on the widened values, every head."""
    import kda_gated_delta_core_amd as kda
    w = ki.WORKLOADS["prefill_h32_t8192_c64"]
    announce(f"kda_chunk_prefill_bf16 {w.name} seed={w.seed} (generating inputs)")
    x = ki.workload_inputs(w)
    (o16, s16), (o32, s32), (qw, kw, vw) = _both(kda, x, w.T, w.chunk)
    assert torch.equal(o16, o32) and torch.equal(s16, s32)
    o, s = host(o16), host(s16)
    T = w.T
    announce("oracle, all 32 heads")
    sl = lambda a: np.ascontiguousarray(a[:, :T])
    o_ref, s_ref, _, _ = oracle.serial(sl(qw), sl(kw), sl(vw), sl(x["gate"]), sl(x["beta"]), x["state"])
    assert_close("core", o[:, :T], o_ref)
    assert_close("state", s, s_ref)
    for h in range(w.heads):
        assert_close(f"h{h} core", o[:, :T, h], o_ref[:, :, h], quiet=True)
        assert_close(f"h{h} state", s[:, h], s_ref[:, h], quiet=True)


@pytest.mark.parametrize("C", [16, 32, 64])
def test_varlen_bf16_equals_fp32_varlen_on_widened_inputs(device, C):
    """kda_chunk_prefill_varlen_bf16: packed sequences (empty, one-token, ragged and multi-chunk ones, and
    rows after the last sequence), bit for bit equal to kda_chunk_prefill_varlen on the widened values."""
    import kda_gated_delta_core_amd as kda
    lens = [0, 1, 70, 130, 5, 200, 64]
    H = 3
    announce(f"kda_chunk_prefill_varlen_bf16 lens={lens} H={H} C={C}")
    x = ki.varlen_inputs(9450 + C, lens, H, -5.0, 0.02, pad_tokens=9)
    total = x["q"].shape[0]
    parts = [_bf16(x[n]) for n in ("q", "k", "v")]
    packed = np.ascontiguousarray(np.stack([p[0] for p in parts], axis=1))  # [total][3][H][128]
    qw, kw, vw = (p[1] for p in parts)
    g, b, cu = dev(x["gate"]), dev(x["beta"]), torch.from_numpy(x["cu_seqlens"]).cuda()
    st16, st32 = dev(x["state"]), dev(x["state"])
    o16 = torch.full((total, H, 128), SENTINEL, device="cuda")
    o32 = torch.full((total, H, 128), SENTINEL, device="cuda")
    kda.kda_chunk_prefill_varlen_bf16(_bits_dev(packed), g, b, st16, cu, C, out=o16)
    kda.kda_chunk_prefill_varlen(dev(qw), dev(kw), dev(vw), g, b, st32, cu, C, out=o32)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32), "out differs from kda_chunk_prefill_varlen on the widened inputs"
    assert torch.equal(st16, st32), "state differs from kda_chunk_prefill_varlen on the widened inputs"
    assert bool((o16[sum(lens):] == SENTINEL).all()), "rows after the last sequence were written"
    # and the oracle on the widened values, sequence by sequence
    o = host(o16)
    for s, (a, e) in enumerate(zip(x["cu_seqlens"][:-1], x["cu_seqlens"][1:])):
        if e == a:
            assert np.array_equal(host(st16)[s], x["state"][s]), "an empty sequence's state changed"
            continue
        sub = [np.ascontiguousarray(t[None, a:e]) for t in (qw, kw, vw, x["gate"], x["beta"])]
        o_ref, s_ref, _, _ = oracle.serial(*sub, x["state"][s:s + 1])
        assert_close(f"seq {s} out", o[None, a:e], o_ref)
        assert_close(f"seq {s} state", host(st16)[s:s + 1], s_ref)


_RNG = np.random.default_rng(20261204)
RANDOM = [(int(_RNG.integers(1, 4)), int(_RNG.integers(1, 9)), int(_RNG.integers(1, 400)),
           int(_RNG.choice([16, 32, 64])), float(_RNG.uniform(-20.0, 0.0)), int(_RNG.integers(0, 10 ** 6)))
          for _ in range(8)]


@pytest.mark.parametrize("B,H,T,C,lo,seed", RANDOM)
def test_bf16_prefill_random_shapes(device, B, H, T, C, lo, seed):
    """Seeded random batch, heads, length, chunk width and gate range: bit for bit the FP32 prefill on the
    widened values."""
    import kda_gated_delta_core_amd as kda
    announce(f"kda_chunk_prefill_bf16 B={B} H={H} T={T} C={C} gates [{lo:.1f}, 0] seed={seed}")
    t_pad = -(-T // C) * C
    x = ki.make_batch(seed, B, H, T, lo, 0.02, alloc_rows=t_pad, pad_value=float("nan"))
    (o16, s16), (o32, s32), _ = _both(kda, x, T, C)
    assert torch.equal(o16, o32) and torch.equal(s16, s32)
