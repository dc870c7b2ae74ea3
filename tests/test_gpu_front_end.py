"""GPU parity of kda_decode_front_end (through the C ABI) with the fp64 oracle, and the front end
feeding the recurrent core."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testlib import announce, assert_close

pytestmark = pytest.mark.gpu
D = 128
# q, k, v carry the FP32 rounding of a <= 4-term conv sum and of the SiLU (a few units of 2^-24
# relative), so they are held far tighter than the core's bar
FE_ATOL, FE_RTOL = 2e-6, 1e-6


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _bits_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _run(kda, x, heads, eps, n_snap=0):
    qkv, w = _bits_dev(x["qkv"]), _bits_dev(x["conv_w"])
    st = torch.from_numpy(x["conv_state"]).cuda()
    B, T, C = x["qkv"].shape
    snaps = torch.full((max(n_snap, 1), B, C, w.shape[1]), -7.0, device="cuda") if n_snap else None
    q, k, v = kda.kda_decode_front_end(qkv, w, st, heads, eps, conv_snapshots=snaps, n_snapshots=n_snap)
    torch.cuda.synchronize()
    return q.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy(), st.cpu().numpy(), \
        (snaps.cpu().numpy() if snaps is not None else None)


@pytest.mark.parametrize("B,T,H,K,n_snap", [(1, 1, 1, 4, 0), (3, 5, 2, 3, 2), (2, 4, 3, 1, 4), (5, 2, 1, 2, 1),
                                            (64, 1, 32, 4, 0), (4, 4, 32, 4, 4)])
def test_front_end_matches_oracle(device, B, T, H, K, n_snap):
    import kda_gated_delta_core_amd as kda
    announce(f"kda_decode_front_end B={B} T={T} H={H} K={K} n_snap={n_snap}")
    x = ki.front_end_inputs(300 + B + T + H + K, B, T, H, K)
    q, k, v, st, sn = _run(kda, x, H, ki.L2_EPS, n_snap)
    rq, rk, rv, rst, rsn = oracle.decode_front_end(x["qkv"], x["conv_w"], x["conv_state"], H, ki.L2_EPS, n_snap)
    for name, g, r in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        assert_close(name, g, r, atol=FE_ATOL, rtol=FE_RTOL)
    assert np.array_equal(st, rst)  # the window holds inputs only: exact
    if n_snap:
        assert np.array_equal(sn[:n_snap], rsn)


def test_front_end_edges(device):
    """Zero input rows (q, k scale to 0 / sqrt(eps) = 0), large and tiny magnitudes, saturating SiLU."""
    import kda_gated_delta_core_amd as kda
    announce("kda_decode_front_end edges")
    B, T, H, K = 2, 3, 2, 4
    x = ki.front_end_inputs(350, B, T, H, K)
    qkv = x["qkv"].copy()
    C = 3 * H * D
    qkv[0, :, :] = 0
    st = x["conv_state"].copy()
    st[0] = 0.0
    big = ki.to_bf16_bits(np.float32(1e30))
    qkv[1, 0, :D] = big
    qkv[1, 1, D:2 * D] = ki.to_bf16_bits(np.float32(1e-30))
    qkv[1, 2, 2 * D:2 * D + 16] = ki.to_bf16_bits(np.float32(-100.0))
    qkv[1, 2, 2 * D + 16:2 * D + 32] = ki.to_bf16_bits(np.float32(100.0))
    y = dict(x, qkv=qkv, conv_state=st)
    q, k, v, s, _ = _run(kda, y, H, ki.L2_EPS)
    rq, rk, rv, rs, _ = oracle.decode_front_end(qkv, x["conv_w"], st, H, ki.L2_EPS)
    assert not np.any(q[0]) and not np.any(k[0]) and not np.any(v[0])
    for name, g, r in (("q", q, rq), ("k", k, rk)):
        assert_close(name, g, r, atol=FE_ATOL, rtol=FE_RTOL)
    # v is not normalised (values up to ~100 here): its error scales with its magnitude
    err = np.abs(v - rv) / (np.abs(rv) + 1.0)
    print(f"    v: max error / (|v| + 1) = {err.max():.3e}", flush=True)
    assert err.max() <= 4e-6
    assert np.array_equal(s, rs)


def test_front_end_feeds_the_recurrent_core(device):
    """front end -> kda_recurrent_k (gate, beta from the usual recipe) against the oracle chain."""
    import kda_gated_delta_core_amd as kda
    B, T, H, K = 3, 4, 2, 4
    announce(f"kda_decode_front_end + kda_recurrent_k B={B} T={T} H={H}")
    x = ki.front_end_inputs(360, B, T, H, K)
    core = ki.make_batch(361, B, H, T, -5.0, 0.02)
    q, k, v = kda.kda_decode_front_end(_bits_dev(x["qkv"]), _bits_dev(x["conv_w"]),
                                       torch.from_numpy(x["conv_state"]).cuda(), H, ki.L2_EPS)
    g, b = torch.from_numpy(core["gate"]).cuda(), torch.from_numpy(core["beta"]).cuda()
    st = torch.from_numpy(core["state"]).cuda()
    out = kda.kda_recurrent_k(q, k, v, g, b, st)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.decode_front_end(x["qkv"], x["conv_w"], x["conv_state"], H, ki.L2_EPS)
    # the core consumes the front end's FP32 outputs; the oracle chain feeds it its own fp64 ones
    ro, rs, _, _ = oracle.serial(rq.astype(np.float32), rk.astype(np.float32), rv.astype(np.float32),
                                 core["gate"], core["beta"], core["state"])
    assert_close("core out", out.cpu().numpy(), ro)
    assert_close("core state", st.cpu().numpy(), rs)


def test_rows_in_one_call_equal_single_row_calls_bitwise(device):
    """T rows in one call and T calls of one row give the same bits (the front-end half of the
    layer page's requirement that decode_k match k serial decodes exactly)."""
    import kda_gated_delta_core_amd as kda
    B, T, H, K = 3, 5, 2, 4
    announce(f"kda_decode_front_end T={T} vs {T} x T=1")
    x = ki.front_end_inputs(370, B, T, H, K)
    qkv, w = _bits_dev(x["qkv"]), _bits_dev(x["conv_w"])
    st_a = torch.from_numpy(x["conv_state"]).cuda()
    st_b = st_a.clone()
    qa, ka, va = kda.kda_decode_front_end(qkv, w, st_a, H, ki.L2_EPS)
    rows = []
    for t in range(T):
        rows.append(kda.kda_decode_front_end(qkv[:, t:t + 1].contiguous(), w, st_b, H, ki.L2_EPS))
    torch.cuda.synchronize()
    for i, a in enumerate((qa, ka, va)):
        assert torch.equal(a, torch.cat([r[i] for r in rows], dim=1))
    assert torch.equal(st_a, st_b)
