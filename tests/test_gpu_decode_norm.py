"""GPU parity of the BF16 decode forms with the gated RMSNorm fused in (kda_recurrent_k_bf16_norm,
kda_recurrent_step_bf16_norm), through the C ABI: the core rows and state against the fp64 oracle,
the normalised rows within one BF16 unit in the last place of the oracle's norm of those core rows,
and the k-row walk bit for bit equal to single steps."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testlib import SENTINEL, announce, assert_close, assert_within_one_ulp, dev, host

pytestmark = pytest.mark.gpu
D = 128


def _bits_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _bits_host(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _inputs(seed, B, T, H):
    x = ki.make_batch(seed, B, H, T, -5.0, 0.02)
    bits = np.stack([ki.to_bf16_bits(x[n]) for n in ("q", "k", "v")], axis=2)   # [B][T][3][H][D]
    wide = [oracle.bf16_to_f64(bits[:, :, i]).astype(np.float32) for i in range(3)]
    nx = ki.norm_inputs(seed + 1, B * T, H)
    return x, bits, wide, nx["out_gate"].reshape(B, T, H, D), nx["o_norm"]


@pytest.mark.parametrize("B,T,H,n_snap", [(64, 1, 32, 0), (3, 5, 2, 3), (1, 1, 1, 0), (17, 4, 9, 4)])
def test_decode_norm_matches_oracle(device, B, T, H, n_snap):
    import kda_gated_delta_core_amd as kda
    announce(f"kda_recurrent_k_bf16_norm B={B} T={T} H={H} n_snap={n_snap}")
    x, bits, wide, og, on = _inputs(9700 + B + T, B, T, H)
    st = dev(x["state"])
    out = torch.full((B, T, H, D), SENTINEL, device="cuda")
    snaps = torch.full((max(n_snap, 1), B, H, D, D), SENTINEL, device="cuda")
    y, _ = kda.kda_recurrent_k_bf16_norm(_bits_dev(bits), dev(x["gate"]), dev(x["beta"]), st, _bits_dev(og),
                                         _bits_dev(on), ki.NORM_EPS, out=out, snapshots=snaps if n_snap else None,
                                         n_snapshots=n_snap)
    torch.cuda.synchronize()
    o_ref, s_ref, sn_ref, _ = oracle.serial(wide[0], wide[1], wide[2], x["gate"], x["beta"], x["state"],
                                            n_snap=n_snap)
    o = host(out)
    assert_close("core", o, o_ref)
    assert_close("state", host(st), s_ref)
    for t in range(n_snap):
        assert_close(f"snapshot[{t}]", host(snaps)[t], sn_ref[t])
    # the norm of the core rows this call computed (its own FP32 output), exact in fp64
    y_ref = oracle.gated_rmsnorm(o.astype(np.float64), og, on, ki.NORM_EPS)
    assert_within_one_ulp("y", oracle.bf16_to_f64(_bits_host(y)), y_ref)


def test_decode_norm_k_rows_equal_steps_and_the_separate_norm(device):
    """T rows of the k-row form equal T single fused steps bit for bit; y agrees with kda_gated_rmsnorm
    of the same core rows to within one BF16 unit in the last place (equal almost everywhere); with out
    NULL the y rows are unchanged."""
    import kda_gated_delta_core_amd as kda
    B, T, H = 32, 4, 8
    announce(f"kda_recurrent_k_bf16_norm vs steps B={B} T={T} H={H}")
    x, bits, wide, og, on = _inputs(9720, B, T, H)
    qkv, g, b, ogd, ond = _bits_dev(bits), dev(x["gate"]), dev(x["beta"]), _bits_dev(og), _bits_dev(on)
    st = dev(x["state"])
    snaps = torch.empty((T, B, H, D, D), device="cuda")
    y, out = kda.kda_recurrent_k_bf16_norm(qkv, g, b, st, ogd, ond, ki.NORM_EPS, snapshots=snaps, n_snapshots=T)
    st2 = dev(x["state"])
    for t in range(T):
        sl = lambda a: a[:, t:t + 1].contiguous()
        yt, ot = kda.kda_recurrent_step_bf16_norm(sl(qkv), sl(g), sl(b), st2, sl(ogd), ond, ki.NORM_EPS)
        torch.cuda.synchronize()
        assert torch.equal(yt, y[:, t:t + 1]) and torch.equal(ot, out[:, t:t + 1]), f"row {t}"
        assert torch.equal(st2, snaps[t]), f"snapshot {t}"
    assert torch.equal(st2, st)
    sep = kda.kda_gated_rmsnorm(out.view(B * T, H, D), ogd.view(B * T, H, D), ond, ki.NORM_EPS)
    torch.cuda.synchronize()
    a, c = oracle.bf16_to_f64(_bits_host(y)).ravel(), oracle.bf16_to_f64(_bits_host(sep)).ravel()
    n_eq = int(np.sum(a == c))
    print(f"    fused y equal to the separate norm in {n_eq}/{a.size}", flush=True)
    assert n_eq >= 0.99 * a.size
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(c), 2.0 ** -133))) - 7)
    assert np.all(np.abs(a - c) <= ulp)
    st3 = dev(x["state"])
    y3, o3 = kda.kda_recurrent_k_bf16_norm(qkv, g, b, st3, ogd, ond, ki.NORM_EPS, want_core=False)
    torch.cuda.synchronize()
    assert o3 is None and torch.equal(y3, y) and torch.equal(st3, st)
