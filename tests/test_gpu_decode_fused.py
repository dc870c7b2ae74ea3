"""GPU parity of the decode step from the raw projections (kda_decode_fused_k / _step and their gated
forms: front end, recurrence and gated RMSNorm in one kernel), through the C ABI.  The fp64 oracle's
front end, gate and recurrence give the reference core rows and states; the conv state and its
snapshots are exact (they hold inputs only); y is held within one BF16 unit in the last place of the
oracle's norm of the call's own core rows; the k-row walk equals single steps bit for bit."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testlib import SENTINEL, announce, assert_close, assert_within_one_ulp, dev, host

pytestmark = pytest.mark.gpu
D = 128
LB = ki.GATE_LOWER_BOUND


def _bits_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _bits_host(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _inputs(seed, B, T, H, K):
    fe = ki.front_end_inputs(seed, B, T, H, K)
    x = ki.make_batch(seed + 1, B, H, T, -5.0, 0.02)
    nx = ki.norm_inputs(seed + 2, B * T, H)
    gx = ki.gate_inputs(seed + 3, B, T, H)
    return fe, x, nx["out_gate"].reshape(B, T, H, D), nx["o_norm"], gx


def _call(kda, fe, x, og, on, gx, H, gated, n_snap, out=None, want_core=True):
    B, T, C = fe["qkv"].shape
    K = fe["conv_w"].shape[1]
    cs = dev(fe["conv_state"])
    st = dev(x["state"])
    snaps = torch.full((max(n_snap, 1), B, H, D, D), SENTINEL, device="cuda") if n_snap else None
    csn = torch.full((max(n_snap, 1), B, C, K), SENTINEL, device="cuda") if n_snap else None
    common = dict(out=out, want_core=want_core)
    qkv, w, ogd, ond = _bits_dev(fe["qkv"]), _bits_dev(fe["conv_w"]), _bits_dev(og), _bits_dev(on)
    if gated:
        args = (qkv, w, cs, _bits_dev(gx["g_raw"]), dev(gx["beta_logit"]), dev(gx["dt_bias"]), dev(gx["a_log"]), LB,
                st, ogd, ond, H, ki.NORM_EPS, ki.L2_EPS)
        if T == 1 and not n_snap:
            y, o = kda.kda_decode_fused_step_gated(*args, **common)
        else:
            y, o = kda.kda_decode_fused_k_gated(*args, snapshots=snaps, conv_snapshots=csn, n_snapshots=n_snap,
                                                **common)
    else:
        args = (qkv, w, cs, dev(x["gate"]), dev(x["beta"]), st, ogd, ond, H, ki.NORM_EPS, ki.L2_EPS)
        if T == 1 and not n_snap:
            y, o = kda.kda_decode_fused_step(*args, **common)
        else:
            y, o = kda.kda_decode_fused_k(*args, snapshots=snaps, conv_snapshots=csn, n_snapshots=n_snap, **common)
    torch.cuda.synchronize()
    return y, o, st, cs, snaps, csn


def _oracle_gate_beta(x, gx, gated):
    if not gated:
        return x["gate"], x["beta"]
    g = oracle.kda_gate(gx["g_raw"], gx["dt_bias"], gx["a_log"], LB)
    return g.astype(np.float32), oracle.sigmoid(gx["beta_logit"]).astype(np.float32)


@pytest.mark.parametrize("B,T,H,K,n_snap,gated", [(64, 1, 32, 4, 0, False), (64, 1, 32, 4, 0, True),
                                                  (3, 5, 2, 3, 3, False), (2, 4, 3, 1, 4, True),
                                                  (17, 4, 9, 4, 2, True), (1, 1, 1, 2, 0, False),
                                                  (5, 3, 4, 2, 1, False), (128, 4, 32, 4, 4, True)])
def test_fused_decode_matches_oracle(device, B, T, H, K, n_snap, gated):
    _against_oracle(B, T, H, K, n_snap, gated, 9800 + 7 * B + T + K)


def _random_case(r):
    B, T, H, K = int(r.integers(1, 21)), int(r.integers(1, 7)), int(r.integers(1, 11)), int(r.integers(1, 5))
    return B, T, H, K, int(r.integers(0, T + 1)), bool(r.integers(0, 2)), int(r.integers(0, 10 ** 6))


_RNG = np.random.default_rng(20261203)
RANDOM = [_random_case(_RNG) for _ in range(8)]


@pytest.mark.parametrize("B,T,H,K,n_snap,gated,seed", RANDOM)
def test_fused_decode_random_shapes(device, B, T, H, K, n_snap, gated, seed):
    """Seeded random batch, rows, heads, conv width, snapshot count and gate form against the oracle."""
    _against_oracle(B, T, H, K, n_snap, gated, seed)


def _against_oracle(B, T, H, K, n_snap, gated, seed):
    import kda_gated_delta_core_amd as kda
    announce(f"kda_decode_fused{'_gated' if gated else ''} B={B} T={T} H={H} K={K} n_snap={n_snap} seed={seed}")
    fe, x, og, on, gx = _inputs(seed, B, T, H, K)
    out = torch.full((B, T, H, D), SENTINEL, device="cuda")
    y, o, st, cs, snaps, csn = _call(kda, fe, x, og, on, gx, H, gated, n_snap, out=out)
    rq, rk, rv, rcs, rcsn = oracle.decode_front_end(fe["qkv"], fe["conv_w"], fe["conv_state"], H, ki.L2_EPS, n_snap)
    gate, beta = _oracle_gate_beta(x, gx, gated)
    o_ref, s_ref, sn_ref, _ = oracle.serial(rq, rk, rv, gate, beta, x["state"], n_snap=n_snap)
    got = host(o)
    assert_close("core", got, o_ref)
    assert_close("state", host(st), s_ref)
    for t in range(n_snap):
        assert_close(f"snapshot[{t}]", host(snaps)[t], sn_ref[t])
    assert np.array_equal(host(cs), rcs), "conv state"
    if n_snap:
        assert np.array_equal(host(csn)[:n_snap], rcsn), "conv snapshots"
    y_ref = oracle.gated_rmsnorm(got.astype(np.float64), og, on, ki.NORM_EPS)
    assert_within_one_ulp("y", oracle.bf16_to_f64(_bits_host(y)), y_ref)


@pytest.mark.parametrize("gated", [False, True])
def test_fused_decode_against_separate_kernels(device, gated):
    """The conv state and its snapshots equal kda_decode_front_end's bit for bit; the core rows and
    state are within the tolerance of kda_decode_front_end (FP32) followed by the 4-slice core."""
    import kda_gated_delta_core_amd as kda
    B, T, H, K, n = 24, 4, 6, 4, 4
    announce(f"kda_decode_fused{'_gated' if gated else ''} vs separate kernels B={B} T={T} H={H}")
    fe, x, og, on, gx = _inputs(9850, B, T, H, K)
    y, o, st, cs, snaps, csn = _call(kda, fe, x, og, on, gx, H, gated, n)
    cs2 = dev(fe["conv_state"])
    csn2 = torch.empty((n, B, 3 * H * D, K), device="cuda")
    q, k, v = kda.kda_decode_front_end(_bits_dev(fe["qkv"]), _bits_dev(fe["conv_w"]), cs2, H, ki.L2_EPS,
                                       conv_snapshots=csn2, n_snapshots=n)
    st2 = dev(x["state"])
    snaps2 = torch.empty((n, B, H, D, D), device="cuda")
    if gated:
        o2 = kda.kda_recurrent_k_gated(q, k, v, _bits_dev(gx["g_raw"]), dev(gx["beta_logit"]), dev(gx["dt_bias"]),
                                       dev(gx["a_log"]), LB, st2, snapshots=snaps2, n_snapshots=n)
    else:
        o2 = kda.kda_recurrent_k(q, k, v, dev(x["gate"]), dev(x["beta"]), st2, snapshots=snaps2, n_snapshots=n)
    torch.cuda.synchronize()
    assert torch.equal(cs, cs2) and torch.equal(csn, csn2), "conv state / snapshots"
    assert_close("core vs separate", host(o), host(o2).astype(np.float64))
    assert_close("state vs separate", host(st), host(st2).astype(np.float64))
    for t in range(n):
        assert_close(f"snapshot[{t}] vs separate", host(snaps)[t], host(snaps2)[t].astype(np.float64))


@pytest.mark.parametrize("gated", [False, True])
def test_fused_decode_k_rows_equal_steps(device, gated):
    """T rows of the k-row form equal T single fused steps bit for bit (y, core rows, state, conv
    state); snapshot t is the state after step t; with out NULL, y is unchanged."""
    import kda_gated_delta_core_amd as kda
    B, T, H, K = 16, 4, 8, 3
    announce(f"kda_decode_fused{'_gated' if gated else ''} k rows vs steps B={B} T={T} H={H}")
    fe, x, og, on, gx = _inputs(9870, B, T, H, K)
    y, o, st, cs, snaps, csn = _call(kda, fe, x, og, on, gx, H, gated, T)
    st2, cs2 = dev(x["state"]), dev(fe["conv_state"])
    qkv, w, ogd, ond = _bits_dev(fe["qkv"]), _bits_dev(fe["conv_w"]), _bits_dev(og), _bits_dev(on)
    for t in range(T):
        sl = lambda a: a[:, t:t + 1].contiguous()
        if gated:
            yt, ot = kda.kda_decode_fused_step_gated(sl(qkv), w, cs2, sl(_bits_dev(gx["g_raw"])),
                                                     sl(dev(gx["beta_logit"])), dev(gx["dt_bias"]),
                                                     dev(gx["a_log"]), LB, st2, sl(ogd), ond, H, ki.NORM_EPS,
                                                     ki.L2_EPS)
        else:
            yt, ot = kda.kda_decode_fused_step(sl(qkv), w, cs2, sl(dev(x["gate"])), sl(dev(x["beta"])), st2, sl(ogd),
                                               ond, H, ki.NORM_EPS, ki.L2_EPS)
        torch.cuda.synchronize()
        assert torch.equal(yt, y[:, t:t + 1]) and torch.equal(ot, o[:, t:t + 1]), f"row {t}"
        assert torch.equal(st2, snaps[t]) and torch.equal(cs2, csn[t]), f"snapshot {t}"
    assert torch.equal(st2, st) and torch.equal(cs2, cs)
    y3, o3, st3, _, _, _ = _call(kda, fe, x, og, on, gx, H, gated, 0, want_core=False)
    assert o3 is None and torch.equal(y3, y) and torch.equal(st3, st)


@pytest.mark.parametrize("gated", [False, True])
def test_fused_decode_edges(device, gated):
    """Edge rows through the whole fused step: a sequence whose projections and conv state are all zero
    (q = k = v = 0, so the state only decays and the core rows and y are exactly 0); saturated gates and
    beta (gate 0 and -40 with beta 0 and 1 in the plain form; g_raw and beta logits at +-30 in the gated
    form); all against the oracle chain."""
    import kda_gated_delta_core_amd as kda
    B, T, H, K = 3, 3, 2, 4
    announce(f"kda_decode_fused{'_gated' if gated else ''} edges B={B} T={T} H={H}")
    fe, x, og, on, gx = _inputs(9890, B, T, H, K)
    fe["qkv"][0] = 0
    fe["conv_state"][0] = 0.0
    x["gate"][1, :, 0] = 0.0
    x["gate"][1, :, 1] = -40.0
    x["beta"][1, 0] = 0.0
    x["beta"][1, 1] = 1.0
    gx["g_raw"][1, :, 0] = ki.to_bf16_bits(np.float32(30.0))
    gx["g_raw"][1, :, 1] = ki.to_bf16_bits(np.float32(-30.0))
    gx["beta_logit"][1, 0] = 30.0
    gx["beta_logit"][1, 1] = -30.0
    out = torch.full((B, T, H, D), SENTINEL, device="cuda")
    y, o, st, cs, _, _ = _call(kda, fe, x, og, on, gx, H, gated, 0, out=out)
    rq, rk, rv, rcs, _ = oracle.decode_front_end(fe["qkv"], fe["conv_w"], fe["conv_state"], H, ki.L2_EPS)
    gate, beta = _oracle_gate_beta(x, gx, gated)
    o_ref, s_ref, _, _ = oracle.serial(rq, rk, rv, gate, beta, x["state"])
    got = host(o)
    assert not np.any(got[0]) and not np.any(oracle.bf16_to_f64(_bits_host(y))[0]), "zero sequence"
    assert_close("core", got, o_ref)
    assert_close("state", host(st), s_ref)
    assert np.array_equal(host(cs), rcs), "conv state"
    y_ref = oracle.gated_rmsnorm(got.astype(np.float64), og, on, ki.NORM_EPS)
    assert_within_one_ulp("y", oracle.bf16_to_f64(_bits_host(y)), y_ref)


@pytest.mark.timeout(600)
def test_fused_decode_state_past_4gib(device):
    """The whole-head kernel over 66,000 heads: the state spans 4.03 GiB, so the last heads' byte offsets
    pass 2^32; every head against the oracle."""
    B, H = 500, 132
    _against_oracle(B, 1, H, 4, 0, False, 9310)
