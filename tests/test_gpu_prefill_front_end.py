"""GPU parity of kda_prefill_front_end (through the C ABI): conv1d + SiLU + L2(q, k) over the tokens of a
prefill into the chunk-padded inputs of kda_chunk_prefill, against the fp64 oracle (the same token-by-token
front end the decode form is checked against), against the decode form bit for bit, and feeding the
chunked prefill."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testlib import SENTINEL, announce, assert_close, assert_within_one_ulp, host

pytestmark = pytest.mark.gpu
D = 128
# as for the decode form: FP32 rounding of a <= 4-term conv sum and of the SiLU
FE_ATOL, FE_RTOL = 2e-6, 1e-6


def _bits_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _run(kda, x, heads, chunk):
    B, T, C = x["qkv"].shape
    t_pad = -(-T // chunk) * chunk
    st = torch.from_numpy(x["conv_state"]).cuda()
    q, k, v = (torch.full((B, t_pad, heads, D), SENTINEL, device="cuda") for _ in range(3))
    kda.kda_prefill_front_end(_bits_dev(x["qkv"]), _bits_dev(x["conv_w"]), st, heads, chunk, ki.L2_EPS,
                              q=q, k=k, v=v)
    torch.cuda.synchronize()
    return host(q), host(k), host(v), host(st)


@pytest.mark.parametrize("B,T,H,K,chunk", [(1, 1, 1, 4, 64), (2, 37, 3, 4, 16), (1, 2, 2, 4, 32), (3, 16, 1, 3, 16),
                                           (1, 33, 2, 1, 64), (2, 5, 2, 2, 16), (1, 8192, 32, 4, 64)])
def test_prefill_front_end_matches_oracle(device, B, T, H, K, chunk):
    import kda_gated_delta_core_amd as kda
    announce(f"kda_prefill_front_end B={B} T={T} H={H} K={K} chunk={chunk}")
    x = ki.front_end_inputs(500 + B + T + H + K, B, T, H, K)
    q, k, v, st = _run(kda, x, H, chunk)
    rq, rk, rv, rst, _ = oracle.decode_front_end(x["qkv"], x["conv_w"], x["conv_state"], H, ki.L2_EPS)
    for name, g, r in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        assert_close(name, g[:, :T], r, atol=FE_ATOL, rtol=FE_RTOL)
        assert np.all(g[:, T:] == SENTINEL), f"{name}: a row >= T was written"
    assert np.array_equal(st, rst)  # the conv state only ever holds inputs: exact


@pytest.mark.parametrize("B,T,H,K", [(2, 50, 3, 4), (1, 3, 2, 4), (4, 100, 2, 2)])
def test_prefill_front_end_equals_decode_front_end_bitwise(device, B, T, H, K):
    """Every row and the final conv state equal what kda_decode_front_end gives walking the same T rows
    (the header's statement; each form is also checked against the oracle)."""
    import kda_gated_delta_core_amd as kda
    announce(f"kda_prefill_front_end vs kda_decode_front_end B={B} T={T} H={H} K={K}")
    x = ki.front_end_inputs(540 + T, B, T, H, K)
    q, k, v, st = _run(kda, x, H, 16)
    st_d = torch.from_numpy(x["conv_state"]).cuda()
    dq, dk, dv = kda.kda_decode_front_end(_bits_dev(x["qkv"]), _bits_dev(x["conv_w"]), st_d, H, ki.L2_EPS)
    torch.cuda.synchronize()
    for a, b in ((q, dq), (k, dk), (v, dv)):
        assert np.array_equal(a[:, :T], host(b))
    assert np.array_equal(st, host(st_d))


def test_prefill_front_end_then_decode_front_end_continues(device):
    """A prefill of T tokens, then decode rows from the advanced conv state, equal one walk of all the rows."""
    import kda_gated_delta_core_amd as kda
    B, T, R, H, K = 2, 45, 3, 2, 4
    announce(f"kda_prefill_front_end T={T} then {R} decode rows")
    x = ki.front_end_inputs(560, B, T + R, H, K)
    qkv, w = _bits_dev(x["qkv"]), _bits_dev(x["conv_w"])
    st = torch.from_numpy(x["conv_state"]).cuda()
    q, k, v = kda.kda_prefill_front_end(qkv[:, :T].contiguous(), w, st, H, 64, ki.L2_EPS)
    dq, dk, dv = kda.kda_decode_front_end(qkv[:, T:].contiguous(), w, st, H, ki.L2_EPS)
    st_all = torch.from_numpy(x["conv_state"]).cuda()
    aq, ak, av = kda.kda_decode_front_end(qkv, w, st_all, H, ki.L2_EPS)
    torch.cuda.synchronize()
    for p, d, a in ((q, dq, aq), (k, dk, ak), (v, dv, av)):
        assert torch.equal(p[:, :T], a[:, :T]) and torch.equal(d, a[:, T:])
    assert torch.equal(st, st_all)


def test_prefill_chain_front_end_core_norm(device):
    """front end -> kda_chunk_prefill -> kda_gated_rmsnorm at T=1000 H=8, each stage against the oracle on
    the previous stage's GPU output (the per-stage bars of the decode chain)."""
    import kda_gated_delta_core_amd as kda
    B, T, H, K, chunk = 2, 1000, 8, 4, 64
    announce(f"prefill chain B={B} T={T} H={H} K={K} chunk={chunk}")
    fx = ki.front_end_inputs(570, B, T, H, K)
    t_pad = -(-T // chunk) * chunk
    core = ki.make_batch(571, B, H, T, -5.0, 0.02, alloc_rows=t_pad)
    st_conv = torch.from_numpy(fx["conv_state"]).cuda()
    q, k, v = kda.kda_prefill_front_end(_bits_dev(fx["qkv"]), _bits_dev(fx["conv_w"]), st_conv, H, chunk, ki.L2_EPS)
    g, b = torch.from_numpy(core["gate"]).cuda(), torch.from_numpy(core["beta"]).cuda()
    st = torch.from_numpy(core["state"]).cuda()
    out = kda.kda_chunk_prefill(q, k, v, g, b, st, T, chunk)
    nx = ki.norm_inputs(572, B * T, H)
    y = kda.kda_gated_rmsnorm(out[:, :T].contiguous().view(B * T, H, D), _bits_dev(nx["out_gate"]),
                              _bits_dev(nx["o_norm"]), ki.NORM_EPS)
    torch.cuda.synchronize()
    rq, rk, rv, rst, _ = oracle.decode_front_end(fx["qkv"], fx["conv_w"], fx["conv_state"], H, ki.L2_EPS)
    gq, gk, gv = (host(a)[:, :T] for a in (q, k, v))
    assert_close("q", gq, rq, atol=FE_ATOL, rtol=FE_RTOL)
    assert_close("k", gk, rk, atol=FE_ATOL, rtol=FE_RTOL)
    assert np.array_equal(host(st_conv), rst)
    o_ref, s_ref, _, _ = oracle.serial(gq, gk, gv, core["gate"][:, :T], core["beta"][:, :T], core["state"])
    assert_close("core out", host(out)[:, :T], o_ref)
    assert_close("core state", host(st), s_ref)
    r = oracle.gated_rmsnorm(host(out)[:, :T].reshape(B * T, H, D), nx["out_gate"], nx["o_norm"], ki.NORM_EPS)
    assert_within_one_ulp("norm", oracle.bf16_to_f64(host(y.view(torch.int16)).view(np.uint16)), r)


def _varlen_fe_inputs(seed, lens, H, K, pad_tokens=5):
    total = sum(lens) + pad_tokens  # rows past the last sequence belong to none
    a = ki.front_end_inputs(seed, 1, total, H, K)
    st = ki.front_end_inputs(seed + 1, len(lens), 1, H, K)["conv_state"]  # one conv state per sequence
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return a["qkv"][0], a["conv_w"], st, cu


def _run_varlen(kda, qkv, w, st, cu, H):
    total = qkv.shape[0]
    q, k, v = (torch.full((total, H, D), SENTINEL, device="cuda") for _ in range(3))
    cst = torch.from_numpy(st).cuda()
    kda.kda_prefill_front_end_varlen(_bits_dev(qkv), _bits_dev(w), cst, torch.from_numpy(cu).cuda(), H, ki.L2_EPS,
                                     q=q, k=k, v=v)
    torch.cuda.synchronize()
    return host(q), host(k), host(v), host(cst)


@pytest.mark.parametrize("lens,H,K", [([5, 0, 70, 1, 33], 2, 4), ([1], 1, 4), ([0, 0, 64], 3, 3), ([100, 3, 0], 2, 2),
                                      ([31, 32, 33, 1, 0, 2], 1, 1)])
def test_prefill_front_end_varlen_matches_oracle(device, lens, H, K):
    import kda_gated_delta_core_amd as kda
    announce(f"kda_prefill_front_end_varlen lens={lens} H={H} K={K}")
    qkv, w, st, cu = _varlen_fe_inputs(580 + sum(lens), lens, H, K)
    q, k, v, cst = _run_varlen(kda, qkv, w, st, cu, H)
    for s, n in enumerate(lens):
        a, b = int(cu[s]), int(cu[s + 1])
        if n == 0:
            assert np.array_equal(cst[s], st[s])  # an empty sequence keeps its conv state
            continue
        rq, rk, rv, rst, _ = oracle.decode_front_end(qkv[None, a:b], w, st[s:s + 1], H, ki.L2_EPS)
        for name, g, r in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
            assert_close(f"seq {s} {name}", g[None, a:b], r, atol=FE_ATOL, rtol=FE_RTOL)
        assert np.array_equal(cst[s:s + 1], rst)
    end = int(cu[-1])
    assert np.all(q[end:] == SENTINEL) and np.all(k[end:] == SENTINEL) and np.all(v[end:] == SENTINEL)


def test_prefill_front_end_varlen_equals_dense_per_sequence_bitwise(device):
    """Each packed sequence gets the bits kda_prefill_front_end gives it alone (B=1)."""
    import kda_gated_delta_core_amd as kda
    lens, H, K = [40, 1, 0, 95, 7], 2, 4
    announce(f"kda_prefill_front_end_varlen vs kda_prefill_front_end per sequence lens={lens}")
    qkv, w, st, cu = _varlen_fe_inputs(590, lens, H, K)
    q, k, v, cst = _run_varlen(kda, qkv, w, st, cu, H)
    for s, n in enumerate(lens):
        if n == 0:
            continue
        a, b = int(cu[s]), int(cu[s + 1])
        x = {"qkv": qkv[None, a:b].copy(), "conv_w": w, "conv_state": st[s:s + 1].copy()}
        dq, dk, dv, dst = _run(kda, x, H, 16)
        for pk, d in ((q, dq), (k, dk), (v, dv)):
            assert np.array_equal(pk[a:b], d[0, :n]), s
        assert np.array_equal(cst[s], dst[0]), s


def test_varlen_prefill_chain(device):
    """Varlen front end -> kda_chunk_prefill_varlen against the oracle per sequence (the core on the GPU's
    q, k, v)."""
    import kda_gated_delta_core_amd as kda
    lens, H, K, C = [300, 0, 1, 129, 64], 4, 4, 64
    announce(f"varlen prefill chain lens={lens} H={H}")
    qkv, w, st, cu = _varlen_fe_inputs(600, lens, H, K, pad_tokens=0)
    q, k, v, _ = _run_varlen(kda, qkv, w, st, cu, H)
    core = ki.varlen_inputs(601, lens, H, -5.0, 0.02)
    d = {n: torch.from_numpy(core[n]).cuda() for n in ("gate", "beta", "state", "cu_seqlens")}
    out = kda.kda_chunk_prefill_varlen(torch.from_numpy(q).cuda(), torch.from_numpy(k).cuda(),
                                       torch.from_numpy(v).cuda(), d["gate"], d["beta"], d["state"], d["cu_seqlens"],
                                       C)
    torch.cuda.synchronize()
    got_o, got_s = host(out), host(d["state"])
    for s, n in enumerate(lens):
        if n == 0:
            assert np.array_equal(got_s[s], core["state"][s])
            continue
        a, b = int(cu[s]), int(cu[s + 1])
        sl = lambda arr: np.ascontiguousarray(arr[None, a:b])
        o_ref, s_ref, _, _ = oracle.serial(sl(q), sl(k), sl(v), sl(core["gate"]), sl(core["beta"]),
                                           core["state"][s:s + 1])
        assert_close(f"seq {s} out", got_o[None, a:b], o_ref)
        assert_close(f"seq {s} state", got_s[s:s + 1], s_ref)
