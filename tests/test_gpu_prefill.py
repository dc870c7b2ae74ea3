"""GPU parity of the chunked prefill against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import kda_inputs as ki
import oracle
from kda_testlib import SENTINEL, announce, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _prefill(kda, x, T, C, state=None, rows=None):
    """Run kda_chunk_prefill on host arrays x (rows >= T_pad ignored); returns (out, state, ws) tensors."""
    import torch
    B, _, H, _ = x["q"].shape
    t_pad = -(-T // C) * C
    v = lambda a: dev(a[:, :t_pad])
    st = dev(x["state"]) if state is None else state
    out = torch.full((B, t_pad, H, 128), SENTINEL, device="cuda")
    ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T, C), dtype=torch.uint8, device="cuda")
    kda.kda_chunk_prefill(v(x["q"]), v(x["k"]), v(x["v"]), v(x["gate"]), v(x["beta"]), st, T, C, out=out,
                          workspace=ws)
    torch.cuda.synchronize()
    return out, st, ws


def _unswizzle_a(buf, n_row_tiles, n_col_tiles):
    """Matrix from the A-tile order of the workspace records: tile (a, b), lane l, element e
    holds row 16a + l % 16, column 16b + 4 (l // 16) + e."""
    t = buf.reshape(n_row_tiles, n_col_tiles, 4, 16, 4)        # a, b, l//16, l%16, e
    return t.transpose(0, 3, 1, 2, 4).reshape(16 * n_row_tiles, 16 * n_col_tiles)


def _unswizzle_acc(buf, n_row_tiles):
    """Matrix [16 n_row_tiles][128] from accumulator tiles [X][j][lane][e]: row 16X + 4 (l // 16) + e,
    column 16j + l % 16."""
    t = buf.reshape(n_row_tiles, 8, 4, 16, 4)                  # X, j, l//16, l%16, e
    return t.transpose(0, 2, 4, 1, 3).reshape(16 * n_row_tiles, 128)


def _check_against_oracle(x, T, out, st, tag=""):
    o_ref, s_ref, _, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"], T=T)
    o = host(out)
    assert_close(f"{tag}core", o[:, :T], o_ref)
    assert_close(f"{tag}state", host(st), s_ref)
    assert np.all(o[:, T:] == SENTINEL), "rows >= T of out were written"


def test_prefill_small_workload(device):
    import kda_gated_delta_core_amd as kda
    w = ki.WORKLOADS["prefill_h2_t64_c16"]
    announce(f"kda_chunk_prefill {w.name} seed={w.seed}")
    x = ki.workload_inputs(w)
    out, st, _ = _prefill(kda, x, w.T, w.chunk)
    _check_against_oracle(x, w.T, out, st)


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 17, 64, 100, 130])
def test_prefill_ragged(device, T, C):
    import kda_gated_delta_core_amd as kda
    announce(f"kda_chunk_prefill ragged B=2 H=3 T={T} C={C}")
    t_pad = -(-T // C) * C
    x = ki.make_batch(2000 + T, 2, 3, T, -5.0, 0.02, alloc_rows=t_pad, pad_value=1e4)
    out, st, _ = _prefill(kda, x, T, C)
    _check_against_oracle(x, T, out, st)


def test_prefill_pad_values_are_ignored_bitwise(device):
    """positions >= T are ignored in-kernel whatever fills them (layer page, prefill_with_pad_fill)."""
    import torch
    import kda_gated_delta_core_amd as kda
    T, C = 100, 64
    announce(f"kda_chunk_prefill pad invariance T={T} C={C}")
    base = ki.make_batch(3001, 2, 3, T, -5.0, 0.02, alloc_rows=128, pad_value=0.0)
    results = []
    for pad in (0.0, 1e4, np.inf, -np.inf, np.nan):
        x = {n: a.copy() for n, a in base.items()}
        for n in ("q", "k", "v", "gate", "beta"):
            x[n][:, T:] = pad
        out, st, _ = _prefill(kda, x, T, C)
        results.append((out, st))
    for out, st in results[1:]:
        assert torch.equal(out, results[0][0])
        assert torch.equal(st, results[0][1])
    _check_against_oracle(base, T, *results[0])


def test_prefill_workspace_stages(device):
    """The chunk record the prepare kernel writes, stage by stage against the oracle's
    intermediates (workspace page: the numeric check runs one stage at a time)."""
    import kda_gated_delta_core_amd as kda
    T, C, H = 150, 64, 2
    announce(f"kda_chunk_prefill stages T={T} C={C}")
    x = ki.make_batch(4001, 1, H, T, -5.0, 0.02, alloc_rows=192, pad_value=np.nan)
    _, _, ws = _prefill(kda, x, T, C)
    rec_f = 5 * C * 128 + 128
    ws = host(ws).view(np.float32).reshape(H, -1, rec_f)
    for h, c in [(0, 0), (1, 1), (1, 2)]:
        n = min(C, T - c * C)
        stg = oracle.chunk_stages(x["q"], x["k"], x["v"], x["gate"], x["beta"], np.zeros((128, 128)), 0, h,
                                  c * C, n)
        rec = ws[h, c]
        blk = lambda i: rec[i * C * 128:(i + 1) * C * 128]
        W = _unswizzle_a(blk(0), C // 16, 8)
        U = _unswizzle_acc(blk(1), C // 16)
        P = _unswizzle_a(blk(2), C // 16, 8)
        R = _unswizzle_acc(blk(3), C // 16)
        KtT = _unswizzle_a(blk(4), 8, C // 16)
        gam = rec[5 * C * 128:]
        G = stg["G"]
        q = x["q"][0, c * C:c * C + n, h].astype(np.float64)
        k = x["k"][0, c * C:c * C + n, h].astype(np.float64)
        tag = f"h{h}c{c} "
        assert_close(tag + "W", W[:n], stg["W"])
        assert_close(tag + "U", U[:n], stg["U"])
        # the record holds P = e^G o Q - M W and R = M U (O = P S + R)
        assert_close(tag + "P", P[:n], np.exp(G) * q - stg["M"] @ stg["W"])
        assert_close(tag + "R", R[:n], stg["M"] @ stg["U"])
        assert_close(tag + "Ktil^T", KtT[:, :n], (np.exp(G[-1] - G) * k).T)
        # gamma = e^{G_last} is far below the fp32 range for most channels at these gates:
        # compare where the reference is representable, require exact zeros elsewhere
        g_ref = np.exp(G[-1])
        big = g_ref > 1e-30
        assert np.all(np.abs(gam[~big]) < 1e-30)
        if big.any():
            assert_close(tag + "gamma", gam[big], g_ref[big])
        for name, a in (("W", W[n:]), ("U", U[n:]), ("P", P[n:]), ("R", R[n:]), ("Kt", KtT[:, n:])):
            assert np.all(a == 0), f"{tag}{name} pad rows not zero"


def test_prefill_then_decode_equals_serial(device):
    import torch
    import kda_gated_delta_core_amd as kda
    T, n_dec, C, B, H = 200, 5, 64, 2, 3
    announce(f"kda_chunk_prefill T={T} then {n_dec} x kda_recurrent_step")
    x = ki.make_batch(5001, B, H, T + n_dec, -5.0, 0.02)
    pre = {n: np.ascontiguousarray(a[:, :T]) if n != "state" else a for n, a in x.items()}
    t_pad = -(-T // C) * C
    pre = {n: (np.concatenate([a, np.full((B, t_pad - T) + a.shape[2:], np.nan, np.float32)], 1)
               if n != "state" else a) for n, a in pre.items()}
    out, st, _ = _prefill(kda, pre, T, C)
    outs = [host(out)[:, :T]]
    for t in range(T, T + n_dec):
        sl = lambda a: dev(a[:, t:t + 1])
        o = torch.empty((B, 1, H, 128), device="cuda")
        kda.kda_recurrent_step(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["gate"]), sl(x["beta"]), st, out=o)
        outs.append(host(o))
    torch.cuda.synchronize()
    o_ref, s_ref, _, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"])
    assert_close("core", np.concatenate(outs, 1), o_ref)
    assert_close("state", host(st), s_ref)


def test_prefill_split_across_calls(device):
    import kda_gated_delta_core_amd as kda
    T1, T2, B, H = 96, 70, 1, 4
    announce(f"kda_chunk_prefill split {T1}+{T2}")
    x = ki.make_batch(6001, B, H, T1 + T2, -5.0, 0.02)
    a = {n: (np.ascontiguousarray(v[:, :T1]) if n != "state" else v) for n, v in x.items()}
    b2 = {n: (np.ascontiguousarray(v[:, T1:]) if n != "state" else v) for n, v in x.items()}
    b2 = {n: (np.concatenate([v, np.zeros((B, 96 - T2) + v.shape[2:], np.float32)], 1) if n != "state" else v)
          for n, v in b2.items()}
    out1, st, _ = _prefill(kda, a, T1, 32)
    out2, st, _ = _prefill(kda, b2, T2, 32, state=st)
    o_ref, s_ref, _, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"])
    assert_close("core", np.concatenate([host(out1)[:, :T1], host(out2)[:, :T2]], 1), o_ref)
    assert_close("state", host(st), s_ref)


def test_prefill_h32_t8192_full_size(device):
    """T=8192, H=32, C=64, pads (one extra chunk too) filled with 1e4; every head against the oracle."""
    import kda_gated_delta_core_amd as kda
    w = ki.WORKLOADS["prefill_h32_t8192_c64"]
    announce(f"kda_chunk_prefill {w.name} seed={w.seed} (generating inputs)")
    x = ki.workload_inputs(w)
    announce("running GPU prefill")
    out, st, _ = _prefill(kda, x, w.T, w.chunk)
    o, s = host(out), host(st)
    assert np.all(o[:, w.T:] == SENTINEL)
    announce("oracle, all 32 heads")
    o_ref, s_ref, _, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"], T=w.T)
    assert_close("core", o[:, :w.T], o_ref)
    assert_close("state", s, s_ref)
    for h in range(w.heads):  # no head passes on the strength of the others
        assert_close(f"h{h} core", o[:, :w.T, h], o_ref[:, :, h], quiet=True)
        assert_close(f"h{h} state", s[:, h], s_ref[:, h], quiet=True)


def test_prefill_h32_t8155_in_chunk_pads(device):
    """The T=8192 H=32 workload cut to T=8155: the last chunk holds 37 real rows and 27 pad rows of 1e4
    (plus the extra pad chunk), so the pad select inside a chunk is exercised at full size; every head
    against the oracle."""
    import kda_gated_delta_core_amd as kda
    w = ki.WORKLOADS["prefill_h32_t8192_c64"]
    T = 8155
    announce(f"kda_chunk_prefill {w.name} cut to T={T} seed={w.seed} (generating inputs)")
    x = ki.workload_inputs(w, T=T)
    assert x["q"].shape[1] > T and np.all(x["q"][:, T:] == w.pad_value)
    out, st, _ = _prefill(kda, x, T, w.chunk)
    o, s = host(out), host(st)
    assert np.all(o[:, T:] == SENTINEL)
    announce("oracle, all 32 heads")
    o_ref, s_ref, _, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"], T=T)
    assert_close("core", o[:, :T], o_ref)
    assert_close("state", s, s_ref)
    for h in range(w.heads):
        assert_close(f"h{h} core", o[:, :T, h], o_ref[:, :, h], quiet=True)
        assert_close(f"h{h} state", s[:, h], s_ref[:, h], quiet=True)


@pytest.mark.timeout(1200)
def test_prefill_b4_t32768_then_decode_full_size(device):
    """4 sequences x T=32768, H=32, C=64, gates in [-0.5, 0] (long memory), then 16 decode steps per
    sequence from the prefilled states (rows T.. of the same streams); the oracle walks every head of
    every sequence through all T + 16 rows."""
    import torch
    import kda_gated_delta_core_amd as kda
    w = ki.WORKLOADS["prefill_b4_h32_t32768_c64"]
    B, H, T = w.batch, w.heads, w.T
    announce(f"kda_chunk_prefill {w.name} seed={w.seed} (generating inputs)")
    x = ki.workload_inputs(w)
    announce("running GPU prefill")
    out, st, ws = _prefill(kda, x, T, w.chunk)
    del ws
    st_pre = host(st)
    announce(f"running {w.tail_steps} x kda_recurrent_step")
    rows = [ki.sequence_rows(w.seed, s, T, T + w.tail_steps, H, w.gate_lo) for s in range(B)]
    tail = {n: np.stack([r[n] for r in rows]) for n in ("q", "k", "v", "gate", "beta")}  # [B, steps, H(, D)]
    outs = []
    for j in range(w.tail_steps):
        sl = lambda a: dev(np.ascontiguousarray(a[:, j:j + 1]))
        o = torch.empty((B, 1, H, 128), device="cuda")
        kda.kda_recurrent_step(sl(tail["q"]), sl(tail["k"]), sl(tail["v"]), sl(tail["gate"]), sl(tail["beta"]), st,
                               out=o)
        outs.append(host(o))
    tail_out = np.concatenate(outs, 1)
    st_end = host(st)
    for b in range(B):
        announce(f"oracle sequence {b}, all {H} heads")
        sub = {n: np.ascontiguousarray(x[n][b:b + 1, :T]) for n in ("q", "k", "v", "gate", "beta")}
        o_ref, s_ref, _, _ = oracle.serial(sub["q"], sub["k"], sub["v"], sub["gate"], sub["beta"], x["state"][b:b + 1])
        del sub
        o_gpu = out[b:b + 1, :T].cpu().numpy()
        assert_close(f"b{b} core", o_gpu, o_ref)
        assert_close(f"b{b} state after prefill", st_pre[b:b + 1], s_ref)
        for h in range(H):
            assert_close(f"b{b} h{h} core", o_gpu[:, :, h], o_ref[:, :, h], quiet=True)
            assert_close(f"b{b} h{h} state after prefill", st_pre[b:b + 1, h], s_ref[:, h], quiet=True)
        del o_gpu, o_ref
        tsub = {n: np.ascontiguousarray(tail[n][b:b + 1]) for n in tail}
        o2, s2, _, _ = oracle.serial(tsub["q"], tsub["k"], tsub["v"], tsub["gate"], tsub["beta"], s_ref)
        assert_close(f"b{b} decode tail core", tail_out[b:b + 1], o2)
        assert_close(f"b{b} final state", st_end[b:b + 1], s2)
        for h in range(H):
            assert_close(f"b{b} h{h} decode tail core", tail_out[b:b + 1, :, h], o2[:, :, h], quiet=True)
            assert_close(f"b{b} h{h} final state", st_end[b:b + 1, h], s2[:, h], quiet=True)


@pytest.mark.parametrize("B,H,T", [(2, 32, 200), (3, 25, 130)])
def test_prefill_wide_column_groups(device, B, H, T):
    """Enough (sequence, head) pairs that, on a 256-CU part, the scan takes 32 value columns per
    workgroup (B*H*8 > 256 >= ... B*H*4); B*H = 75 also leaves a partly filled XCD group."""
    import kda_gated_delta_core_amd as kda
    C = 64
    announce(f"kda_chunk_prefill B={B} H={H} T={T} C={C}")
    x = ki.make_batch(7001 + B, B, H, T, -5.0, 0.02, alloc_rows=-(-T // C) * C, pad_value=float("nan"))
    out, st, _ = _prefill(kda, x, T, C)
    _check_against_oracle(x, T, out, st)


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("lo", [-9.0, -12.0, -20.0, -60.0])
def test_prefill_steep_gates(device, C, lo):
    """Gates steeper than the fast tables allow (below about -8.3): drawn on [lo, 0], channels at
    exactly lo on every row, channels with no decay, alternating rows, a head whose first chunk has
    mild gates (so one call takes both paths), -inf and -1e30 on a few channels, beta outside
    [0, 1].  Output and state finite and within the tolerance of the fp64 oracle, and the
    prefill's final state within the tolerance of the decode path walking the same rows."""
    import torch
    import kda_gated_delta_core_amd as kda
    B, H, T = 2, 3, 150
    announce(f"kda_chunk_prefill steep gates lo={lo} C={C}")
    t_pad = -(-T // C) * C
    x = ki.make_batch(8200 + C, B, H, T, lo, 0.02, alloc_rows=t_pad, pad_value=-1e30)
    mild = ki.make_batch(8300 + C, B, H, T, -5.0, 0.02)["gate"]
    x["gate"][0, :T, :, :16] = lo             # the steepest decay on every row
    x["gate"][0, :T, :, 16:32] = 0.0          # no decay
    x["gate"][1, :T:2, 1, :] = lo             # alternating steep / drawn rows
    x["gate"][1, :C, 2, :] = mild[1, :C, 2]   # a first chunk on the fast path, steep chunks after it
    x["gate"][1, :T, 0, 100:104] = -np.inf
    x["gate"][1, :T, 0, 104:108] = -1e30
    x["beta"][1, :T, 2] = 1.7
    x["beta"][0, :T, 1] = -0.3
    out, st, _ = _prefill(kda, x, T, C)
    _check_against_oracle(x, T, out, st)
    # the decode path over the same rows ends in the same state
    sl = lambda a: dev(np.ascontiguousarray(a[:, :T]))
    st2 = dev(x["state"])
    o2 = kda.kda_recurrent_k(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["gate"]), sl(x["beta"]), st2)
    torch.cuda.synchronize()
    assert_close("prefill vs decode state", host(st), host(st2))
    assert_close("prefill vs decode out", host(out)[:, :T], host(o2))


@pytest.mark.parametrize("C", [16, 64])
def test_prefill_gates_at_the_fast_bound(device, C):
    """Gates on both sides of the switch between the paths, by head: -8.0 on every row (the fast
    tables at 92 of their 96 bits of range, 8 x 8.0 x log2 e), -8.5 on every row (past the bound,
    steep path), and the two alternating; all within the tolerance of the oracle."""
    import kda_gated_delta_core_amd as kda
    B, H, T = 1, 4, 2 * C + 5
    announce(f"kda_chunk_prefill gates at the fast bound C={C}")
    t_pad = -(-T // C) * C
    x = ki.make_batch(8400 + C, B, H, T, -5.0, 0.02, alloc_rows=t_pad, pad_value=float("nan"))
    x["gate"][0, :T, 0] = -8.0
    x["gate"][0, :T, 1] = -8.5
    x["gate"][0, :T, 2] = -8.0
    x["gate"][0, :T:2, 2] = -8.5
    out, st, _ = _prefill(kda, x, T, C)
    _check_against_oracle(x, T, out, st)


@pytest.mark.parametrize("B,H,T,C", [(1, 1, 1, 64), (300, 1, 17, 16), (2, 129, 33, 32), (5, 7, 64, 64)])
def test_prefill_odd_shapes(device, B, H, T, C):
    """One head and one token; many sequences of one head; a head count that leaves the scan's
    8-head XCD groups and 8-column groups partly filled; whole chunks only."""
    import kda_gated_delta_core_amd as kda
    announce(f"kda_chunk_prefill odd shape B={B} H={H} T={T} C={C}")
    t_pad = -(-T // C) * C
    x = ki.make_batch(9100 + B + H, B, H, T, -5.0, 0.02, alloc_rows=t_pad, pad_value=float("nan"))
    out, st, _ = _prefill(kda, x, T, C)
    _check_against_oracle(x, T, out, st)


@pytest.mark.timeout(600)
def test_prefill_max_heads(device):
    """KDA_PREFILL_MAX_HEADS heads (the most the header allows) in one call, every head against the
    oracle."""
    import kda_gated_delta_core_amd as kda
    B, H, T, C = 1, 16384, 20, 16
    announce(f"kda_chunk_prefill max heads B={B} H={H} T={T} C={C}")
    t_pad = -(-T // C) * C
    x = ki.make_batch(9200, B, H, T, -5.0, 0.02, alloc_rows=t_pad)
    out, st, _ = _prefill(kda, x, T, C)
    o, s = host(out), host(st)
    assert np.all(o[:, T:] == SENTINEL)
    o_ref, s_ref, _, _ = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"], T=T)
    assert_close("core", o[:, :T], o_ref)
    assert_close("state", s, s_ref)
    # every head within the tolerance on its own (max-abs per head, rel-L2 per head)
    d = np.abs(o[:, :T].astype(np.float64) - o_ref).max(axis=(0, 1, 3))
    ds = np.abs(s.astype(np.float64) - s_ref).max(axis=(0, 2, 3))
    assert d.max() <= 1e-3 and ds.max() <= 1e-3, (int(d.argmax()), float(d.max()), int(ds.argmax()), float(ds.max()))
    num = np.linalg.norm((o[:, :T].astype(np.float64) - o_ref).transpose(2, 0, 1, 3).reshape(H, -1), axis=1)
    den = np.linalg.norm(o_ref.transpose(2, 0, 1, 3).reshape(H, -1), axis=1)
    assert np.all(num <= 1e-4 * den), int(np.argmax(num / den))


@pytest.mark.timeout(600)
def test_prefill_inputs_past_4gib(device):
    """65 sequences of 1,024 tokens at H=128: each input array spans 4.06 GiB, so the last sequence's
    q, k, v, gate and out rows lie past 2^32 bytes (its records past 21 GB).  That sequence holds the
    seeded inputs and is checked against the oracle on every head; the others hold zeros."""
    import torch
    import kda_gated_delta_core_amd as kda
    B, H, T, C = 65, 128, 1024, 64
    last = B - 1
    announce(f"kda_chunk_prefill B={B} H={H} T={T} C={C} (inputs {B * T * H * 512 / 2 ** 30:.2f} GiB each)")
    assert last * T * H * 512 >= 2 ** 32
    rows = ki.sequence_rows(9320, last, 0, T, H, -5.0)
    st0 = ki.initial_state(9320, last, H, 0.02)
    tens = {n: torch.zeros((B, T, H, 128), device="cuda") for n in ("q", "k", "v", "gate")}
    tens["beta"] = torch.zeros((B, T, H), device="cuda")
    for n in tens:
        tens[n][last].copy_(torch.from_numpy(rows[n]))
    st = torch.zeros((B, H, 128, 128), device="cuda")
    st[last].copy_(torch.from_numpy(st0))
    out = torch.full((B, T, H, 128), SENTINEL, device="cuda")
    ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T, C), dtype=torch.uint8, device="cuda")
    kda.kda_chunk_prefill(tens["q"], tens["k"], tens["v"], tens["gate"], tens["beta"], st, T, C, out=out,
                          workspace=ws)
    torch.cuda.synchronize()
    del ws, tens
    o, s = host(out[last:]), host(st[last:])
    o_ref, s_ref, _, _ = oracle.serial(*(rows[n][None] for n in ("q", "k", "v", "gate", "beta")), st0[None])
    assert_close("core", o, o_ref)
    assert_close("state", s, s_ref)
    for h in range(H):
        assert_close(f"h{h} core", o[:, :, h], o_ref[:, :, h], quiet=True)
        assert_close(f"h{h} state", s[:, h], s_ref[:, h], quiet=True)
    # the zero sequences stay zero: nothing leaked across the 2^32 boundary into them
    assert not bool(out[:last].abs().amax().item()) and not bool(st[:last].abs().amax().item())
