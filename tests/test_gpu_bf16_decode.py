"""GPU parity of the BF16 decode forms (through the C ABI): kda_decode_front_end_bf16, whose BF16
conv_out is the front end's result rounded to nearest even, and kda_recurrent_step_bf16 /
kda_recurrent_k_bf16, which read q | k | v from such packed BF16 rows (workspace page, conv_out)."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testlib import SENTINEL, announce, assert_close, assert_within_one_ulp, dev, host

pytestmark = pytest.mark.gpu
D = 128
# the front end's FP32 error bound (a few units of 2^-24 relative, see the FP32 front-end tests)
FE_ATOL, FE_RTOL = 2e-6, 1e-6
# rounding to BF16 adds at most half a unit in the last place: 2^-8 of the value
BF16_HALF_ULP_REL = 2.0 ** -8


def _bits_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _bits_host(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _packed(x):
    """q, k, v [B][T][H][D] float32 -> BF16 bit patterns [B][T][3][H][D] and the widened q, k, v."""
    bits = np.stack([ki.to_bf16_bits(x[n]) for n in ("q", "k", "v")], axis=2)
    wide = [oracle.bf16_to_f64(bits[:, :, i]).astype(np.float32) for i in range(3)]
    return bits, wide


def _front_end_bf16(kda, x, heads, n_snap=0):
    B, T, C = x["qkv"].shape
    K = x["conv_w"].shape[1]
    st = torch.from_numpy(x["conv_state"]).cuda()
    snaps = torch.full((max(n_snap, 1), B, C, K), -7.0, device="cuda") if n_snap else None
    out = torch.full((B, T, C), -3.0, dtype=torch.bfloat16, device="cuda")
    kda.kda_decode_front_end_bf16(_bits_dev(x["qkv"]), _bits_dev(x["conv_w"]), st, heads, ki.L2_EPS,
                                  conv_out=out, conv_snapshots=snaps, n_snapshots=n_snap)
    torch.cuda.synchronize()
    return out, st, snaps


@pytest.mark.parametrize("B,T,H,K,n_snap", [(1, 1, 1, 4, 0), (3, 5, 2, 3, 2), (2, 4, 3, 1, 4), (64, 1, 32, 4, 0),
                                            (128, 4, 32, 4, 4)])
def test_front_end_bf16_matches_oracle(device, B, T, H, K, n_snap):
    import kda_gated_delta_core_amd as kda
    announce(f"kda_decode_front_end_bf16 B={B} T={T} H={H} K={K} n_snap={n_snap}")
    x = ki.front_end_inputs(400 + B + T + H + K, B, T, H, K)
    out, st, sn = _front_end_bf16(kda, x, H, n_snap)
    rq, rk, rv, rst, rsn = oracle.decode_front_end(x["qkv"], x["conv_w"], x["conv_state"], H, ki.L2_EPS, n_snap)
    ref = np.stack([rq, rk, rv], axis=2).reshape(B, T, 3 * H * D)
    got = oracle.bf16_to_f64(_bits_host(out))
    # each value is an FP32 result within the front end's bound, then rounded once to BF16
    err = np.abs(got - ref)
    bound = (BF16_HALF_ULP_REL + FE_RTOL) * np.abs(ref) + FE_ATOL
    print(f"    conv_out: max |err| / bound = {(err / bound).max():.3f}", flush=True)
    assert np.all(err <= bound)
    assert np.array_equal(host(st), rst)
    if n_snap:
        assert np.array_equal(host(sn)[:n_snap], rsn)


def test_front_end_bf16_rounds_the_fp32_front_end(device):
    """The header's statement: every BF16 value is the FP32 form's value rounded to nearest even,
    and the conv state and snapshots are the FP32 form's (checked here between the two forms; each
    form is checked against the oracle above and in the FP32 front-end tests)."""
    import kda_gated_delta_core_amd as kda
    B, T, H, K, n_snap = 5, 3, 4, 4, 3
    announce(f"kda_decode_front_end_bf16 vs kda_decode_front_end B={B} T={T} H={H}")
    x = ki.front_end_inputs(420, B, T, H, K)
    out, st, sn = _front_end_bf16(kda, x, H, n_snap)
    st32 = torch.from_numpy(x["conv_state"]).cuda()
    sn32 = torch.full_like(sn, -7.0)
    q, k, v = kda.kda_decode_front_end(_bits_dev(x["qkv"]), _bits_dev(x["conv_w"]), st32, H, ki.L2_EPS,
                                       conv_snapshots=sn32, n_snapshots=n_snap)
    torch.cuda.synchronize()
    fp32 = np.stack([host(q), host(k), host(v)], axis=2).reshape(B, T, 3 * H * D)
    assert np.array_equal(_bits_host(out), ki.to_bf16_bits(fp32))
    assert torch.equal(st, st32) and torch.equal(sn, sn32)


def _core_bf16(kda, bits, x, B, H, T, n_snap=0, n_slots=None):
    st = dev(x["state"])
    out = torch.full((B, T, H, D), SENTINEL, device="cuda")
    n_slots = n_snap if n_slots is None else n_slots
    snaps = torch.full((max(n_slots, 1), B, H, D, D), SENTINEL, device="cuda")
    if T == 1 and n_snap == 0:
        kda.kda_recurrent_step_bf16(_bits_dev(bits), dev(x["gate"]), dev(x["beta"]), st, out=out)
    else:
        kda.kda_recurrent_k_bf16(_bits_dev(bits), dev(x["gate"]), dev(x["beta"]), st, out=out,
                                 snapshots=snaps if n_snap else None, n_snapshots=n_snap)
    torch.cuda.synchronize()
    return out, st, snaps


@pytest.mark.parametrize("B,H,T,n_snap", [(1, 1, 1, 0), (3, 5, 1, 0), (64, 32, 1, 0), (2, 3, 4, 4), (1, 2, 7, 3)])
def test_recurrent_bf16_matches_oracle(device, B, H, T, n_snap):
    import kda_gated_delta_core_amd as kda
    w = ki.WORKLOADS["decode_k4_b128_h32"]
    announce(f"kda_recurrent_{'step' if T == 1 else 'k'}_bf16 seed={w.seed} B={B} H={H} T={T} n_snap={n_snap}")
    x = ki.make_batch(w.seed, B, H, T, w.gate_lo, w.state_std)
    bits, (q, k, v) = _packed(x)
    out, st, snaps = _core_bf16(kda, bits, x, B, H, T, n_snap, n_slots=n_snap + 1)
    o_ref, s_ref, sn_ref, _ = oracle.serial(q, k, v, x["gate"], x["beta"], x["state"], n_snap=n_snap)
    assert_close("out", host(out), o_ref)
    assert_close("state", host(st), s_ref)
    sn = host(snaps)
    for t in range(n_snap):
        assert_close(f"snapshot[{t}]", sn[t], sn_ref[t])
    if T > 1:
        assert np.all(sn[n_snap] == SENTINEL)  # the slot after the last snapshot is never written


def test_recurrent_bf16_equals_fp32_form_on_widened_inputs_bitwise(device):
    """The header's statement: the BF16 forms give the bits of the FP32 forms on the widened q, k, v."""
    import kda_gated_delta_core_amd as kda
    B, H, T = 6, 7, 5
    announce(f"kda_recurrent_k_bf16 vs kda_recurrent_k B={B} H={H} T={T}")
    x = ki.make_batch(431, B, H, T, -5.0, 0.02)
    bits, (q, k, v) = _packed(x)
    out_a, st_a, sn_a = _core_bf16(kda, bits, x, B, H, T, n_snap=T)
    st_b = dev(x["state"])
    sn_b = torch.full_like(sn_a, SENTINEL)
    out_b = kda.kda_recurrent_k(dev(q), dev(k), dev(v), dev(x["gate"]), dev(x["beta"]), st_b, snapshots=sn_b,
                                n_snapshots=T)
    y = dict(x, q=x["q"][:, :1], k=x["k"][:, :1], v=x["v"][:, :1], gate=x["gate"][:, :1], beta=x["beta"][:, :1])
    out_c, st_c, _ = _core_bf16(kda, bits[:, :1], y, B, H, 1)
    st_d = dev(x["state"])
    out_d = kda.kda_recurrent_step(dev(q[:, :1]), dev(k[:, :1]), dev(v[:, :1]), dev(y["gate"]), dev(y["beta"]), st_d)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(st_a, st_b) and torch.equal(sn_a, sn_b)
    assert torch.equal(out_c, out_d) and torch.equal(st_c, st_d)


def test_decode_k_bf16_equals_serial_steps_bitwise(device):
    """decode_k on BF16 rows at the full decode_k size (B=128, H=32, k=4, 4 snapshots) equals four
    kda_recurrent_step_bf16 calls bit for bit (layer page, decode_k), and the oracle on sampled
    sequences."""
    import kda_gated_delta_core_amd as kda
    w = ki.WORKLOADS["decode_k4_b128_h32"]
    B, H, T = w.batch, w.heads, w.T
    announce(f"kda_recurrent_k_bf16 T={T} vs {T} x kda_recurrent_step_bf16 B={B} H={H}")
    x = ki.make_batch(w.seed + 1, B, H, T, w.gate_lo, w.state_std)
    bits, wide = _packed(x)
    out_k, st_k, sn_k = _core_bf16(kda, bits, x, B, H, T, n_snap=T)
    st = dev(x["state"])
    g, b = dev(x["gate"]), dev(x["beta"])
    rows = _bits_dev(bits)
    for t in range(T):
        o = kda.kda_recurrent_step_bf16(rows[:, t:t + 1].contiguous(), g[:, t:t + 1].contiguous(),
                                        b[:, t:t + 1].contiguous(), st)
        torch.cuda.synchronize()
        assert torch.equal(o, out_k[:, t:t + 1]), t
        assert torch.equal(st, sn_k[t]), t
    assert torch.equal(st, st_k)
    sel = [0, 37, 127]
    q, k, v = (np.ascontiguousarray(a[sel]) for a in wide)
    o_ref, s_ref, sn_ref, _ = oracle.serial(q, k, v, x["gate"][sel], x["beta"][sel], x["state"][sel], n_snap=T)
    assert_close("out", host(out_k)[sel], o_ref)
    assert_close("state", host(st_k)[sel], s_ref)
    sn = host(sn_k)
    for t in range(T):
        assert_close(f"snapshot[{t}]", sn[t][sel], sn_ref[t])


def test_bf16_decode_chain(device):
    """front end (BF16 conv_out) -> kda_recurrent_k_bf16 -> gated RMSNorm, the decode chain of the module
    page, at the decode_k size with conv and state snapshots.  Each stage is held to its own bar on
    the previous stage's GPU output; the first stage also against the oracle chain."""
    import kda_gated_delta_core_amd as kda
    B, T, H, K, seed = ki.FRONT_END_WORKLOADS["front_end_b128_h32_k4_rows4"]
    announce(f"decode chain BF16 B={B} T={T} H={H} K={K}")
    x = ki.front_end_inputs(seed, B, T, H, K)
    conv_out, _, _ = _front_end_bf16(kda, x, H, n_snap=T)
    core = ki.make_batch(seed + 1, B, H, T, -5.0, 0.02)
    st = dev(core["state"])
    snaps = torch.full((T, B, H, D, D), SENTINEL, device="cuda")
    out = kda.kda_recurrent_k_bf16(conv_out, dev(core["gate"]), dev(core["beta"]), st, snapshots=snaps,
                                   n_snapshots=T)
    nx = ki.norm_inputs(seed + 2, B * T, H)
    y = kda.kda_gated_rmsnorm(out.view(B * T, H, D), _bits_dev(nx["out_gate"]), _bits_dev(nx["o_norm"]),
                              ki.NORM_EPS)
    torch.cuda.synchronize()
    # the core on the GPU's BF16 q, k, v
    qkv = oracle.bf16_to_f64(_bits_host(conv_out)).reshape(B, T, 3, H, D).astype(np.float32)
    o_ref, s_ref, sn_ref, _ = oracle.serial(qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2], core["gate"], core["beta"],
                                            core["state"], n_snap=T)
    assert_close("core out", host(out), o_ref)
    assert_close("core state", host(st), s_ref)
    for t in range(T):
        assert_close(f"snapshot[{t}]", host(snaps[t]), sn_ref[t])
    # the norm on the GPU's core output: within one BF16 unit in the last place of the exact value
    r = oracle.gated_rmsnorm(host(out).reshape(B * T, H, D), nx["out_gate"], nx["o_norm"], ki.NORM_EPS)
    assert_within_one_ulp("norm", oracle.bf16_to_f64(_bits_host(y)), r)
    # the q, k rows the front end hands over are unit vectors up to BF16 rounding (2^-9 per element)
    n = np.linalg.norm(qkv[:, :, :2].astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1.0) <= 4e-3)
