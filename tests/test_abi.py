"""CPU checks of the C ABI: the library loads, exports what include/kda.h declares,
and refuses bad arguments on the host before touching any buffer or the GPU.
None of these calls reaches a kernel launch."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import kda_gated_delta_core_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

# fake, never-dereferenced device addresses, far apart so no range overlaps
P = [0x10000000000 * (i + 1) for i in range(10)]


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return kda.load_library()


# The refusal tests pass fake, never-mapped device addresses: a check that regressed would launch a
# kernel on them.  They run only where no GPU is visible (counting devices does not initialise one).
no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="refusal tests use fake device addresses; run where no GPU is visible")


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(kda.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported
    assert not {e for e in exported if e.startswith("kda_")} - set(names)


def test_status_strings(lib):
    for code, tag in [(0, "KDA_OK"), (-1, "INVALID_ARG"), (-2, "UNSUPPORTED"), (-3, "WORKSPACE"), (-4, "HIP")]:
        assert tag in kda.kda_status_string(code)
    assert "unknown" in kda.kda_status_string(7)


def test_workspace_bytes():
    for B, H, T, C in [(1, 2, 64, 16), (1, 32, 8192, 64), (4, 32, 32768, 64), (3, 5, 100, 32), (2, 1, 1, 16)]:
        n = -(-T // C)
        rec = 5 * C * 128 + 128
        assert kda.kda_chunk_prefill_workspace_bytes(B, H, T, C) == B * H * n * rec * 4
    for bad in [(0, 1, 1, 16), (1, 0, 1, 16), (1, 1, 0, 16), (1, 1, 1, 8), (1, 1, 1, 128), (-1, 1, 1, 64)]:
        assert kda.kda_chunk_prefill_workspace_bytes(*bad) == 0
    assert kda.kda_chunk_prefill_workspace_bytes(1 << 20, 1 << 10, 1 << 20, 64) == 0  # overflow


def _prefill(lib, ptrs=None, B=1, H=2, T=64, C=16, ws=None, ws_bytes=None):
    p = list(ptrs or P[:7])
    need = kda.kda_chunk_prefill_workspace_bytes(B, H, T, C)
    return lib.kda_chunk_prefill(*p, B, H, T, C, P[7] if ws is None else ws,
                                 need if ws_bytes is None else ws_bytes, None)


@no_gpu
def test_prefill_refusals(lib):
    for i in range(7):
        p = list(P[:7])
        p[i] = None
        assert _prefill(lib, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    assert _prefill(lib, B=0) == kda.KDA_ERR_INVALID_ARG
    assert _prefill(lib, H=0) == kda.KDA_ERR_INVALID_ARG
    assert _prefill(lib, T=0) == kda.KDA_ERR_INVALID_ARG
    assert _prefill(lib, T=-5) == kda.KDA_ERR_INVALID_ARG
    for C in (0, 8, 48, 128):
        assert lib.kda_chunk_prefill(*P[:7], 1, 2, 64, C, P[7], 1 << 30, None) == kda.KDA_ERR_UNSUPPORTED
    assert _prefill(lib, ws_bytes=1000) == kda.KDA_ERR_WORKSPACE
    assert lib.kda_chunk_prefill(*P[:7], 1, 2, 64, 16, None, 1 << 30, None) == kda.KDA_ERR_WORKSPACE
    # out overlapping q, state overlapping out, workspace overlapping state
    p = list(P[:7])
    p[6] = P[0] + 64
    assert _prefill(lib, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    p = list(P[:7])
    p[5] = P[6] + 4
    assert _prefill(lib, ptrs=p) == kda.KDA_ERR_INVALID_ARG
    assert _prefill(lib, ws=P[5] + 128) == kda.KDA_ERR_INVALID_ARG
    # size overflow
    assert lib.kda_chunk_prefill(*P[:7], 1 << 20, 1 << 10, 1 << 20, 64, P[7], 1 << 62, None) == \
        kda.KDA_ERR_INVALID_ARG
    # more heads than the in-chunk offsets allow
    assert lib.kda_chunk_prefill(*P[:7], 1, 16385, 64, 16, P[7], 1 << 40, None) == kda.KDA_ERR_INVALID_ARG
    # more chunk records than the chunk index allows: 1024 x 16 x (2^16 + 1) chunks of 16 rows
    # (fake buffers 2^52 bytes apart, so only that limit can refuse the call)
    far = [(i + 1) << 52 for i in range(8)]
    args = (1 << 10, 1 << 4, (1 << 16) * 16 + 1, 16)
    assert kda.kda_chunk_prefill_workspace_bytes(*args) > 0
    assert lib.kda_chunk_prefill(*far[:7], *args, far[7], 1 << 62, None) == kda.KDA_ERR_INVALID_ARG
    args = (1 << 10, 1 << 4, (1 << 16) * 16, 16)  # exactly 2^30 records: accepted up to the launch
    assert lib.kda_chunk_prefill_workspace_bytes(*args) > 0


@no_gpu
def test_prefill_bf16_refusals(lib):
    f = lib.kda_chunk_prefill_bf16
    bad = kda.KDA_ERR_INVALID_ARG
    need = kda.kda_chunk_prefill_workspace_bytes(1, 2, 64, 16)
    # qkv, gate, beta, state, out
    for i in range(5):
        p = list(P[:5])
        p[i] = None
        assert f(*p, 1, 2, 64, 16, P[7], need, None) == bad, i
    for i in (0, 1, 3, 4):  # 16-byte alignment (beta: 4)
        p = list(P[:5])
        p[i] += 8
        assert f(*p, 1, 2, 64, 16, P[7], need, None) == bad, i
    p = list(P[:5])
    p[2] += 2
    assert f(*p, 1, 2, 64, 16, P[7], need, None) == bad
    assert f(*P[:5], 0, 2, 64, 16, P[7], need, None) == bad
    assert f(*P[:5], 1, 0, 64, 16, P[7], need, None) == bad
    assert f(*P[:5], 1, 2, 0, 16, P[7], need, None) == bad
    for C in (0, 8, 48, 128):
        assert f(*P[:5], 1, 2, 64, C, P[7], 1 << 30, None) == kda.KDA_ERR_UNSUPPORTED
    assert f(*P[:5], 1, 2, 64, 16, P[7], need - 1, None) == kda.KDA_ERR_WORKSPACE
    assert f(*P[:5], 1, 2, 64, 16, None, need, None) == kda.KDA_ERR_WORKSPACE
    # out over the packed rows (64 rows x 3 x 2 heads x 128 BF16 = 96 KiB), state over out, workspace over state
    p = list(P[:5])
    p[4] = P[0] + 90 * 1024
    assert f(*p, 1, 2, 64, 16, P[7], need, None) == bad
    p = list(P[:5])
    p[3] = P[4] + 4096
    assert f(*p, 1, 2, 64, 16, P[7], need, None) == bad
    assert f(*P[:5], 1, 2, 64, 16, P[3] + 128, need, None) == bad
    assert f(*P[:5], 1, 16385, 64, 16, P[7], 1 << 40, None) == bad  # heads past the in-chunk offsets
    assert f(*P[:5], 1 << 20, 1 << 10, 1 << 20, 64, P[7], 1 << 62, None) == bad  # size overflow


@no_gpu
def test_varlen_bf16_refusals(lib):
    f = lib.kda_chunk_prefill_varlen_bf16
    bad = kda.KDA_ERR_INVALID_ARG
    need = kda.kda_chunk_prefill_varlen_workspace_bytes(2, 2, 100, 16)
    # qkv, gate, beta, state, out, cu_seqlens
    for i in range(6):
        p = list(P[:6])
        p[i] = None
        assert f(*p, 2, 2, 100, 16, P[7], need, None) == bad, i
    for i, off in ((0, 8), (1, 8), (2, 2), (3, 8), (4, 8), (5, 2)):
        p = list(P[:6])
        p[i] += off
        assert f(*p, 2, 2, 100, 16, P[7], need, None) == bad, i
    assert f(*P[:6], 0, 2, 100, 16, P[7], need, None) == bad
    assert f(*P[:6], 2, 0, 100, 16, P[7], need, None) == bad
    assert f(*P[:6], 2, 2, 0, 16, P[7], need, None) == bad
    assert f(*P[:6], (1 << 20) + 1, 2, 100, 16, P[7], 1 << 40, None) == bad
    for C in (0, 8, 48, 128):
        assert f(*P[:6], 2, 2, 100, C, P[7], 1 << 30, None) == kda.KDA_ERR_UNSUPPORTED
    assert f(*P[:6], 2, 2, 100, 16, P[7], need - 1, None) == kda.KDA_ERR_WORKSPACE
    assert f(*P[:6], 2, 2, 100, 16, None, need, None) == kda.KDA_ERR_WORKSPACE
    p = list(P[:6])
    p[4] = P[0] + 1024  # out over the packed rows
    assert f(*p, 2, 2, 100, 16, P[7], need, None) == bad
    assert f(*P[:6], 2, 2, 100, 16, P[5], need, None) == bad  # workspace over cu_seqlens
    assert f(*P[:6], 2, 16385, 100, 16, P[7], 1 << 40, None) == bad


@no_gpu
def test_recurrent_refusals(lib):
    for i in range(7):
        p = list(P[:7])
        p[i] = None
        assert lib.kda_recurrent_step(*p, 4, 2, None) == kda.KDA_ERR_INVALID_ARG
        assert lib.kda_recurrent_k(*p, None, 0, 4, 2, 3, None) == kda.KDA_ERR_INVALID_ARG
    assert lib.kda_recurrent_step(*P[:7], 0, 2, None) == kda.KDA_ERR_INVALID_ARG
    assert lib.kda_recurrent_step(*P[:7], 2, 0, None) == kda.KDA_ERR_INVALID_ARG
    assert lib.kda_recurrent_k(*P[:7], None, 0, 4, 2, 0, None) == kda.KDA_ERR_INVALID_ARG   # k == 0
    assert lib.kda_recurrent_k(*P[:7], P[8], 4, 4, 2, 3, None) == kda.KDA_ERR_INVALID_ARG  # n_snap > T
    assert lib.kda_recurrent_k(*P[:7], P[8], -1, 4, 2, 3, None) == kda.KDA_ERR_INVALID_ARG
    assert lib.kda_recurrent_k(*P[:7], None, 2, 4, 2, 3, None) == kda.KDA_ERR_INVALID_ARG  # snapshots NULL
    # snapshots overlapping the state
    assert lib.kda_recurrent_k(*P[:7], P[5] + 256, 2, 4, 2, 3, None) == kda.KDA_ERR_INVALID_ARG
    # state overlapping an input
    p = list(P[:7])
    p[5] = P[2] + 16
    assert lib.kda_recurrent_step(*p, 4, 2, None) == kda.KDA_ERR_INVALID_ARG
    assert lib.kda_recurrent_k(*P[:7], None, 0, 1 << 20, 1 << 12, 1 << 20, None) == kda.KDA_ERR_INVALID_ARG


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 2, 128)
    b = torch.zeros(1, 1, 2)
    s = torch.zeros(1, 2, 128, 128)
    with pytest.raises(ValueError):
        kda.kda_recurrent_step(x, x, x, x, b, s, out=torch.zeros_like(x), stream=0)


@no_gpu
def test_gated_rmsnorm_refusals(lib):
    f = lib.kda_gated_rmsnorm
    ok = kda.KDA_ERR_INVALID_ARG
    for i in range(4):
        p = list(P[:4])
        p[i] = None
        assert f(*p, 4, 2, 1e-6, None) == ok
    assert f(*P[:4], 0, 2, 1e-6, None) == ok
    assert f(*P[:4], 4, 0, 1e-6, None) == ok
    assert f(*P[:4], -1, 2, 1e-6, None) == ok
    for eps in (0.0, -1e-6, 1e-31, float("nan"), float("inf")):
        assert f(*P[:4], 4, 2, eps, None) == ok, eps
    # out overlapping core, out_gate or o_norm
    for i in range(3):
        p = list(P[:4])
        p[3] = P[i] + 2
        assert f(*p, 4, 2, 1e-6, None) == ok
    # more vectors than the grid can hold: rows * heads = 2^34 (fake buffers 2^52 bytes apart)
    far = [(i + 1) << 52 for i in range(4)]
    assert f(*far, 1 << 20, 1 << 14, 1e-6, None) == ok


@no_gpu
def test_misaligned_pointers_are_refused(lib):
    bad = kda.KDA_ERR_INVALID_ARG
    for i in range(7):
        p = list(P[:7])
        p[i] += 4 if i != 4 else 2  # beta needs 4-byte alignment, the others 16-byte
        assert _prefill(lib, ptrs=p) == bad, i
        assert lib.kda_recurrent_k(*p, None, 0, 4, 2, 3, None) == bad, i
        assert lib.kda_recurrent_step(*p, 4, 2, None) == bad, i
    assert lib.kda_recurrent_k(*P[:7], P[8] + 8, 2, 4, 2, 3, None) == bad  # misaligned snapshots
    assert _prefill(lib, ws=P[7] + 8) == bad
    for i in range(4):
        p = list(P[:4])
        p[i] += 8
        assert lib.kda_gated_rmsnorm(*p, 4, 2, 1e-6, None) == bad, i


@no_gpu
def test_decode_front_end_refusals(lib):
    f = lib.kda_decode_front_end
    bad = kda.KDA_ERR_INVALID_ARG
    ok_args = (4, 2, 3, 4, 1e-6)  # batch, heads, T, conv_kernel, eps (n_snapshots 0)
    for i in range(6):
        p = list(P[:6])
        p[i] = None
        assert f(*p, None, 0, *ok_args, None) == bad, i
        p = list(P[:6])
        p[i] += 8
        assert f(*p, None, 0, *ok_args, None) == bad, i
    assert f(*P[:6], None, 0, 0, 2, 3, 4, 1e-6, None) == bad
    assert f(*P[:6], None, 0, 4, 0, 3, 4, 1e-6, None) == bad
    assert f(*P[:6], None, 0, 4, 2, 0, 4, 1e-6, None) == bad
    assert f(*P[:6], None, 0, 4, 16385, 3, 4, 1e-6, None) == bad
    assert f(*P[:6], None, 2, *ok_args, None) == bad           # snapshots NULL
    assert f(*P[:6], P[6], 4, *ok_args, None) == bad           # n_snapshots > T
    assert f(*P[:6], P[6], -1, *ok_args, None) == bad
    assert f(*P[:6], P[6] + 8, 1, *ok_args, None) == bad       # misaligned snapshots
    assert f(*P[:6], None, 0, 4, 2, 3, 0, 1e-6, None) == bad
    assert f(*P[:6], None, 0, 4, 2, 3, 5, 1e-6, None) == kda.KDA_ERR_UNSUPPORTED
    for eps in (0.0, -1.0, float("nan"), float("inf")):
        assert f(*P[:6], None, 0, 4, 2, 3, 4, eps, None) == bad
    # outputs overlapping an input or each other
    for i, j in ((3, 0), (4, 3), (2, 5), (5, 1)):
        p = list(P[:6])
        p[i] = p[j] + 16
        assert f(*p, None, 0, *ok_args, None) == bad, (i, j)


@no_gpu
def test_bf16_decode_refusals(lib):
    bad = kda.KDA_ERR_INVALID_ARG
    # kda_recurrent_k_bf16 / _step_bf16: qkv, gate, beta, state, out
    fk, fs = lib.kda_recurrent_k_bf16, lib.kda_recurrent_step_bf16
    for i in range(5):
        p = list(P[:5])
        p[i] = None
        assert fk(*p, None, 0, 4, 2, 3, None) == bad, i
        assert fs(*p, 4, 2, None) == bad, i
        p = list(P[:5])
        p[i] += 2 if i == 2 else 8  # beta needs 4-byte alignment, the others 16-byte
        assert fk(*p, None, 0, 4, 2, 3, None) == bad, i
        assert fs(*p, 4, 2, None) == bad, i
    assert fk(*P[:5], None, 0, 4, 2, 0, None) == bad            # k == 0
    assert fk(*P[:5], None, 0, 0, 2, 3, None) == bad
    assert fk(*P[:5], None, 0, 4, 0, 3, None) == bad
    assert fk(*P[:5], P[6], 4, 4, 2, 3, None) == bad            # n_snapshots > T
    assert fk(*P[:5], None, 2, 4, 2, 3, None) == bad            # snapshots NULL
    assert fk(*P[:5], P[6] + 8, 2, 4, 2, 3, None) == bad        # misaligned snapshots
    # out over the packed rows (3 * 2 bytes per q element), the state over out, snapshots over the state
    p = list(P[:5])
    p[4] = P[0] + 4 * 3 * 3 * 128 * 2 - 16  # B=4, H=3: the last 16 bytes of the rows
    assert fs(*p, 4, 3, None) == bad
    p = list(P[:5])
    p[3] = P[4] + 16
    assert fs(*p, 4, 2, None) == bad
    assert fk(*P[:5], P[3] + 256, 2, 4, 2, 3, None) == bad
    assert fk(*P[:5], None, 0, 1 << 20, 1 << 12, 1 << 20, None) == bad  # size overflow
    # kda_decode_front_end_bf16: qkv, conv_w, conv_state, conv_out
    f = lib.kda_decode_front_end_bf16
    ok_args = (4, 2, 3, 4, 1e-6)
    for i in range(4):
        p = list(P[:4])
        p[i] = None
        assert f(*p, None, 0, *ok_args, None) == bad, i
        p = list(P[:4])
        p[i] += 8
        assert f(*p, None, 0, *ok_args, None) == bad, i
    assert f(*P[:4], None, 0, 4, 2, 3, 5, 1e-6, None) == kda.KDA_ERR_UNSUPPORTED
    assert f(*P[:4], None, 0, 4, 2, 3, 4, 0.0, None) == bad
    assert f(*P[:4], None, 2, *ok_args, None) == bad            # snapshots NULL
    assert f(*P[:4], P[6], 4, *ok_args, None) == bad            # n_snapshots > T
    p = list(P[:4])
    p[3] = P[0] + 16                                            # conv_out over qkv
    assert f(*p, None, 0, *ok_args, None) == bad
    p = list(P[:4])
    p[3] = P[2] + 16                                            # conv_out over the conv state
    assert f(*p, None, 0, *ok_args, None) == bad
    assert f(*P[:4], P[3] + 16, 1, *ok_args, None) == bad       # snapshots over conv_out


@no_gpu
def test_prefill_front_end_refusals(lib):
    f = lib.kda_prefill_front_end
    bad = kda.KDA_ERR_INVALID_ARG
    ok_args = (4, 2, 37, 64, 4, 1e-6)  # batch, heads, T, chunk, conv_kernel, eps
    for i in range(6):
        p = list(P[:6])
        p[i] = None
        assert f(*p, *ok_args, None) == bad, i
        p = list(P[:6])
        p[i] += 8
        assert f(*p, *ok_args, None) == bad, i
    assert f(*P[:6], 0, 2, 37, 64, 4, 1e-6, None) == bad
    assert f(*P[:6], 4, 0, 37, 64, 4, 1e-6, None) == bad
    assert f(*P[:6], 4, 2, 0, 64, 4, 1e-6, None) == bad
    assert f(*P[:6], 4, 16385, 37, 64, 4, 1e-6, None) == bad
    assert f(*P[:6], 4, 2, 37, 64, 0, 1e-6, None) == bad
    assert f(*P[:6], 4, 2, 37, 48, 4, 1e-6, None) == kda.KDA_ERR_UNSUPPORTED
    assert f(*P[:6], 4, 2, 37, 64, 5, 1e-6, None) == kda.KDA_ERR_UNSUPPORTED
    for eps in (0.0, -1.0, float("nan"), float("inf")):
        assert f(*P[:6], 4, 2, 37, 64, 4, eps, None) == bad
    # q over the qkv rows, the conv state over v, k over q
    for i, j in ((3, 0), (2, 5), (4, 3)):
        p = list(P[:6])
        p[i] = p[j] + 16
        assert f(*p, *ok_args, None) == bad, (i, j)


@no_gpu
def test_prefill_front_end_varlen_refusals(lib):
    f = lib.kda_prefill_front_end_varlen
    bad = kda.KDA_ERR_INVALID_ARG
    ok_args = (3, 2, 100, 4, 1e-6)  # n_seqs, heads, total, conv_kernel, eps
    for i in range(7):
        p = list(P[:7])
        p[i] = None
        assert f(*p, *ok_args, None) == bad, i
        p = list(P[:7])
        p[i] += 2 if i == 6 else 8  # cu_seqlens needs 4-byte alignment, the rest 16
        assert f(*p, *ok_args, None) == bad, i
    assert f(*P[:7], 0, 2, 100, 4, 1e-6, None) == bad
    assert f(*P[:7], (1 << 20) + 1, 2, 100, 4, 1e-6, None) == bad
    assert f(*P[:7], 3, 0, 100, 4, 1e-6, None) == bad
    assert f(*P[:7], 3, 2, 0, 4, 1e-6, None) == bad
    assert f(*P[:7], 3, 2, 100, 0, 1e-6, None) == bad
    assert f(*P[:7], 3, 2, 100, 5, 1e-6, None) == kda.KDA_ERR_UNSUPPORTED
    assert f(*P[:7], 3, 2, 100, 4, 0.0, None) == bad
    for i, j in ((3, 0), (6, 2), (2, 5)):  # q over qkv, cu_seqlens inside the conv state, state over v
        p = list(P[:7])
        p[i] = p[j] + 16
        assert f(*p, *ok_args, None) == bad, (i, j)


@no_gpu
def test_varlen_refusals(lib):
    f = lib.kda_chunk_prefill_varlen
    bad = kda.KDA_ERR_INVALID_ARG
    need = kda.kda_chunk_prefill_varlen_workspace_bytes(3, 2, 100, 16)
    assert need > 0
    # records for heads * (total / chunk + n_seqs) chunks, then 2 (n_seqs + 1) int32 offsets
    rec = 5 * 16 * 128 + 128
    assert need == (-(-(2 * (100 // 16 + 3) * rec) // 64) * 64) * 4 + 2 * 4 * 4
    for bad_args in [(0, 2, 100, 16), (3, 0, 100, 16), (3, 2, 0, 16), (3, 2, 100, 8), ((1 << 20) + 1, 1, 100, 16)]:
        assert kda.kda_chunk_prefill_varlen_workspace_bytes(*bad_args) == 0
    args = lambda **kw: dict(dict(n=3, H=2, total=100, C=16, ws=P[9], wsb=need), **kw)

    def call(ptrs=None, **kw):
        a = args(**kw)
        p = list(P[:8]) if ptrs is None else ptrs
        return f(*p, a["n"], a["H"], a["total"], a["C"], a["ws"], a["wsb"], None)
    for i in range(8):
        p = list(P[:8])
        p[i] = None
        assert call(p) == bad, i
        p = list(P[:8])
        p[i] += 2 if i in (4, 7) else 4  # beta and cu_seqlens need 4-byte alignment, the rest 16
        assert call(p) == bad, i
    assert call(n=0) == bad
    assert call(H=0) == bad
    assert call(total=0) == bad
    assert call(C=48) == kda.KDA_ERR_UNSUPPORTED
    assert call(wsb=need - 1) == kda.KDA_ERR_WORKSPACE
    assert call(ws=None) == kda.KDA_ERR_WORKSPACE
    p = list(P[:8])
    p[6] = P[0] + 16  # out over q
    assert call(p) == bad
    p = list(P[:8])
    p[7] = P[5] + 16  # cu_seqlens inside the state
    assert call(p) == bad
    assert call(ws=P[6] + 64) == bad  # workspace over out


def test_library_allocates_copies_and_synchronises_nothing():
    """The library's only HIP imports are kernel registration, launch and device queries: no
    allocation, copy, fill or synchronisation can happen inside any entry point (module page: the
    forward calls allocate nothing)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", kda.LIB_PATH], capture_output=True, text=True).stdout
    hip = {line.split()[-1].split("@")[0] for line in out.splitlines() if "hip" in line.lower()}
    allowed = {"__hipPopCallConfiguration", "__hipPushCallConfiguration", "__hipRegisterFatBinary",
               "__hipRegisterFunction", "__hipUnregisterFatBinary", "hipDeviceGetAttribute", "hipGetDevice",
               "hipGetLastError", "hipLaunchKernel",
               # the static records array of kda_chunk_prefill_noalloc: registered, then looked up per device
               "__hipRegisterVar", "hipGetSymbolAddress",
               # the prepare's persistent grid: workgroups per compute unit, computed on the host
               "hipOccupancyMaxActiveBlocksPerMultiprocessor"}
    assert hip <= allowed, sorted(hip - allowed)
    for bad in ("Malloc", "Free", "Memcpy", "Memset", "Synchronize", "HostRegister"):
        assert not any(bad in name for name in hip), bad


@no_gpu
def test_prefill_noalloc_refusals(lib):
    f = lib.kda_chunk_prefill_noalloc
    for i in range(7):
        p = list(P[:7])
        p[i] = None
        assert f(*p, 1, 2, 64, 16, None) == kda.KDA_ERR_INVALID_ARG
    assert f(*P[:7], 0, 2, 64, 16, None) == kda.KDA_ERR_INVALID_ARG
    assert f(*P[:7], 1, 2, 0, 16, None) == kda.KDA_ERR_INVALID_ARG
    assert f(*P[:7], 1, 2, 64, 48, None) == kda.KDA_ERR_UNSUPPORTED
    p = list(P[:7])
    p[6] = P[0] + 64  # out overlapping q
    assert f(*p, 1, 2, 64, 16, None) == kda.KDA_ERR_INVALID_ARG
    # records beyond the static array: T=8192, H=32, C=64 needs 673 MB > 256 MiB
    assert kda.kda_chunk_prefill_workspace_bytes(1, 32, 8192, 64) > kda.STATIC_WORKSPACE_BYTES
    assert f(*P[:7], 1, 32, 8192, 64, None) == kda.KDA_ERR_WORKSPACE
    # the largest call that fits (1633 records of 164,352 B at C=64) is not refused for its size: its
    # size check passes and only the device lookup (no GPU here) can fail
    rec = 5 * 64 * 128 * 4 + 128 * 4
    n = kda.STATIC_WORKSPACE_BYTES // rec
    assert kda.kda_chunk_prefill_workspace_bytes(1, n, 64, 64) <= kda.STATIC_WORKSPACE_BYTES
    assert kda.kda_chunk_prefill_workspace_bytes(1, n + 1, 64, 64) > kda.STATIC_WORKSPACE_BYTES
    assert f(*P[:7], 1, n + 1, 64, 64, None) == kda.KDA_ERR_WORKSPACE


@no_gpu
def test_gated_refusals(lib):
    """the gate inputs of the gated entry points: null, misaligned, overlapping, or a lower bound that
    is positive or not finite"""
    q, k, v, g, b, dt, al, st, out, ws = P[:10]
    pf = lambda *a, lb=-5.0, ws_=ws: lib.kda_chunk_prefill_gated(*a, lb, st, out, 1, 2, 64, 16, ws_, 1 << 30, None)
    for i in range(7):
        a = [q, k, v, g, b, dt, al]
        a[i] = None
        assert pf(*a) == kda.KDA_ERR_INVALID_ARG, i
    assert pf(q, k, v, g + 4, b, dt, al) == kda.KDA_ERR_INVALID_ARG      # g_raw 8-byte aligned
    assert pf(q, k, v, g, b, dt + 8, al) == kda.KDA_ERR_INVALID_ARG      # dt_bias 16-byte aligned
    assert pf(q, k, v, g, b, dt, al, lb=0.5) == kda.KDA_ERR_INVALID_ARG
    assert pf(q, k, v, g, b, dt, al, lb=float("-inf")) == kda.KDA_ERR_INVALID_ARG
    assert pf(q, k, v, g, b, dt, al, lb=float("nan")) == kda.KDA_ERR_INVALID_ARG
    assert pf(q, k, v, g, b, out + 64, al) == kda.KDA_ERR_INVALID_ARG    # dt_bias inside out
    assert pf(q, k, v, g, b, dt, al, ws_=None) == kda.KDA_ERR_WORKSPACE
    rk = lambda *a, lb=-5.0: lib.kda_recurrent_k_gated(*a, lb, st, out, None, 0, 2, 3, 4, None)
    for i in range(7):
        a = [q, k, v, g, b, dt, al]
        a[i] = None
        assert rk(*a) == kda.KDA_ERR_INVALID_ARG, i
    assert rk(q, k, v, g, b, dt, al, lb=1.0) == kda.KDA_ERR_INVALID_ARG
    assert rk(q, k, v, g + 2, b, dt, al) == kda.KDA_ERR_INVALID_ARG
    assert rk(q, k, v, g, st + 4, dt, al) == kda.KDA_ERR_INVALID_ARG    # beta logits inside state
    assert lib.kda_recurrent_step_gated(q, k, v, None, b, dt, al, -5.0, st, out, 2, 3, None) == \
        kda.KDA_ERR_INVALID_ARG


@no_gpu
def test_decode_norm_refusals(lib):
    qkv, g, b, st, out, og, on, y, sn = P[:9]
    f = lambda *a, eps=1e-6, n=0, snp=None: lib.kda_recurrent_k_bf16_norm(*a[:7], eps, a[7], snp, n, 2, 3, 4, None)
    for i in (0, 1, 2, 3, 5, 6, 7):
        a = [qkv, g, b, st, out, og, on, y]
        a[i] = None
        assert f(*a) == kda.KDA_ERR_INVALID_ARG, i
    assert f(qkv, g, b, st, out, og, on, y, eps=0.0) == kda.KDA_ERR_INVALID_ARG
    assert f(qkv, g, b, st, out, og, on, y, eps=float("nan")) == kda.KDA_ERR_INVALID_ARG
    assert f(qkv, g, b, st, out, og, on, y, n=5, snp=sn) == kda.KDA_ERR_INVALID_ARG   # n_snapshots > T
    assert f(qkv, g, b, st, out, og, on, y, n=1) == kda.KDA_ERR_INVALID_ARG           # snapshots NULL
    assert f(qkv, g, b, st, out, og, on, st + 64) == kda.KDA_ERR_INVALID_ARG          # y inside state
    assert f(qkv, g, b, st, out, og, on, y + 2) == kda.KDA_ERR_INVALID_ARG            # y misaligned
    assert lib.kda_recurrent_step_bf16_norm(qkv, g, b, st, out, None, on, 1e-6, y, 2, 3, None) == \
        kda.KDA_ERR_INVALID_ARG


@no_gpu
def test_decode_fused_refusals(lib):
    Q = [0x10000000000 * (i + 1) for i in range(16)]
    bad = kda.KDA_ERR_INVALID_ARG
    x, w, cs, csn, g, b, st, sn, og, on, y, out = Q[:12]

    def f(*a, n=0, neps=1e-6, leps=1e-6, T=4, K=4):
        x_, w_, cs_, csn_, g_, b_, st_, sn_, og_, on_, y_, out_ = a
        return lib.kda_decode_fused_k(x_, w_, cs_, csn_, g_, b_, st_, sn_, n, og_, on_, neps, leps, y_, out_, 2, 3, T,
                                      K, None)
    ok = [x, w, cs, csn, g, b, st, sn, og, on, y, out]
    for i in (0, 1, 2, 4, 5, 6, 8, 9, 10):
        a = list(ok)
        a[i] = None
        assert f(*a) == bad, i
    for i in (0, 1, 2, 4, 6, 8, 9, 10, 11):
        a = list(ok)
        a[i] += 8
        assert f(*a) == bad, i
    assert f(*ok, neps=0.0) == bad
    assert f(*ok, leps=float("inf")) == bad
    assert f(*ok, n=5) == bad                                   # n_snapshots > T
    a = list(ok); a[3] = None
    assert f(*a, n=1) == bad                                    # conv snapshots NULL
    a = list(ok); a[7] = None
    assert f(*a, n=1) == bad                                    # state snapshots NULL
    assert f(*ok, K=0) == bad
    assert f(*ok, K=5) == kda.KDA_ERR_UNSUPPORTED
    assert f(*ok, T=0) == bad
    a = list(ok); a[10] = st + 64
    assert f(*a) == bad                                         # y inside state
    a = list(ok); a[2] = x
    assert f(*a) == bad                                         # conv state over the projections
    assert lib.kda_decode_fused_step(x, w, cs, None, b, st, og, on, 1e-6, 1e-6, y, out, 2, 3, 4, None) == bad
    assert lib.kda_decode_fused_step(x, w, cs, g, b, st, og, on, 1e-6, 1e-6, y, out, 2, 3, 7, None) == \
        kda.KDA_ERR_UNSUPPORTED
    gr, bl, dt, al = Q[12:16]
    fg = lib.kda_decode_fused_k_gated
    assert fg(x, w, cs, csn, None, bl, dt, al, -5.0, st, sn, 0, og, on, 1e-6, 1e-6, y, out, 2, 3, 4, 4, None) == bad
    assert fg(x, w, cs, csn, gr, bl, dt, al, 1.0, st, sn, 0, og, on, 1e-6, 1e-6, y, out, 2, 3, 4, 4, None) == bad
    assert fg(x, w, cs, csn, gr + 2, bl, dt, al, -5.0, st, sn, 0, og, on, 1e-6, 1e-6, y, out, 2, 3, 4, 4, None) == bad
    assert fg(x, w, cs, csn, gr, st + 4, dt, al, -5.0, st, sn, 0, og, on, 1e-6, 1e-6, y, out, 2, 3, 4, 4, None) == bad
    assert lib.kda_decode_fused_step_gated(x, w, cs, gr, bl, None, al, -5.0, st, og, on, 1e-6, 1e-6, y, out, 2, 3, 4,
                                           None) == bad


@no_gpu
def test_prefill_fused_gated_refusals(lib):
    Q = [0x10000000000 * (i + 1) for i in range(12)]
    bad = kda.KDA_ERR_INVALID_ARG
    x, w, cs, gr, bl, dt, al, st, out, ws = Q[:10]
    need = kda.kda_chunk_prefill_workspace_bytes(2, 3, 100, 64)
    f = lambda *a, lo=-5.0, C=64, K=4, eps=1e-6, wsb=need: lib.kda_chunk_prefill_fused_gated(
        *a[:7], lo, a[7], a[8], 2, 3, 100, C, K, eps, a[9], wsb, None)
    ok = [x, w, cs, gr, bl, dt, al, st, out, ws]
    for i in range(9):
        a = list(ok)
        a[i] = None
        assert f(*a) == bad, i
    assert f(*ok, lo=0.5) == bad
    assert f(*ok, lo=float("nan")) == bad
    assert f(*ok, eps=0.0) == bad
    assert f(*ok, C=48) == kda.KDA_ERR_UNSUPPORTED
    assert f(*ok, K=3) == kda.KDA_ERR_UNSUPPORTED
    assert f(*ok, wsb=need - 1) == kda.KDA_ERR_WORKSPACE
    a = list(ok); a[3] += 2
    assert f(*a) == bad                                        # g_raw misaligned
    a = list(ok); a[4] = st + 4
    assert f(*a) == bad                                        # beta logits inside state


@no_gpu
def test_transition_refusals(lib):
    f = lib.kda_chunk_prefill_transition
    bad = kda.KDA_ERR_INVALID_ARG
    need = kda.kda_chunk_prefill_workspace_bytes(1, 2, 64, 16)
    for i in range(7):
        p = list(P[:7])
        p[i] = None
        assert f(*p, 1, 2, 64, 16, P[7], need, None) == bad, i
        p = list(P[:7])
        p[i] += 8 if i != 4 else 2  # beta needs 4-byte alignment, the rest 16
        assert f(*p, 1, 2, 64, 16, P[7], need, None) == bad, i
    assert f(*P[:7], 0, 2, 64, 16, P[7], need, None) == bad
    assert f(*P[:7], 1, 0, 64, 16, P[7], need, None) == bad
    assert f(*P[:7], 1, 2, 0, 16, P[7], need, None) == bad
    assert f(*P[:7], 1, 2, 64, 48, P[7], 1 << 30, None) == kda.KDA_ERR_UNSUPPORTED
    assert f(*P[:7], 1, 2, 64, 16, P[7], need - 1, None) == kda.KDA_ERR_WORKSPACE
    assert f(*P[:7], 1, 2, 64, 16, None, need, None) == kda.KDA_ERR_WORKSPACE
    assert f(*P[:7], 1, 16385, 64, 16, P[7], 1 << 40, None) == bad
    for i, j in ((5, 0), (6, 5), (5, 6)):  # P over q, Q over P, P over Q
        p = list(P[:7])
        p[i] = p[j] + 64
        assert f(*p, 1, 2, 64, 16, P[7], need, None) == bad, (i, j)
    assert f(*P[:7], 1, 2, 64, 16, P[6] + 256, need, None) == bad  # workspace over Q

    g = lib.kda_state_transition_apply
    assert g(None, P[1], P[2], 1, 2, None) == bad
    assert g(P[0], P[1], None, 1, 2, None) == bad
    assert g(P[0] + 4, P[1], P[2], 1, 2, None) == bad
    assert g(P[0], P[1] + 4, P[2], 1, 2, None) == bad
    assert g(P[0], P[1], P[2] + 4, 1, 2, None) == bad
    assert g(P[0], P[1], P[2], 0, 2, None) == bad
    assert g(P[0], P[1], P[2], 1, 0, None) == bad
    assert g(P[0], P[1], P[0] + 256, 1, 2, None) == bad  # state over P
    assert g(P[0], P[1], P[1], 1, 2, None) == bad  # state is Q
    assert g(P[0], None, P[0], 1, 2, None) == bad  # state is P, Q absent
    assert g(P[0], P[1], P[2], 1 << 20, 1 << 12, None) == bad  # more states than one grid holds
    assert g(P[0], P[1], P[2], 1, (1 << 22) - 7, None) == bad  # one state past the grid limit


@no_gpu
def test_chunk_scan_refusals(lib):
    f = lib.kda_chunk_scan
    bad = kda.KDA_ERR_INVALID_ARG
    need = kda.kda_chunk_prefill_workspace_bytes(1, 2, 64, 16)
    ok = (1, 2, 64, 16)
    assert f(None, P[1], *ok, P[2], need, None) == bad
    assert f(P[0], None, *ok, P[2], need, None) == bad
    assert f(P[0], P[1], *ok, None, need, None) == kda.KDA_ERR_WORKSPACE
    assert f(P[0], P[1], *ok, P[2], need - 1, None) == kda.KDA_ERR_WORKSPACE
    for i in range(3):
        p = [P[0], P[1], P[2]]
        p[i] += 8
        assert f(p[0], p[1], *ok, p[2], need, None) == bad, i
    assert f(P[0], P[1], 0, 2, 64, 16, P[2], need, None) == bad
    assert f(P[0], P[1], 1, 0, 64, 16, P[2], need, None) == bad
    assert f(P[0], P[1], 1, 2, 0, 16, P[2], need, None) == bad
    assert f(P[0], P[1], 1, 2, 64, 8, P[2], 1 << 30, None) == kda.KDA_ERR_UNSUPPORTED
    assert f(P[0], P[1], 1, 16385, 64, 16, P[2], 1 << 40, None) == bad
    assert f(P[0], P[0] + 256, *ok, P[2], need, None) == bad  # out over state
    assert f(P[0], P[1], *ok, P[1] + 256, need, None) == bad  # workspace over out
    assert f(P[0], P[1], *ok, P[0] + 256, need, None) == bad  # workspace over state


def test_header_is_plain_c_and_links_from_c(tmp_path):
    """include/kda.h compiles as C99 and C++ on its own, and a C program links against the library and
    calls its host-only entry points (no GPU needed)."""
    src = tmp_path / "use_kda.c"
    src.write_text(
        '#include "kda.h"\n#include <stdio.h>\n#include <string.h>\n'
        "int main(void) {\n"
        "  size_t ws = kda_chunk_prefill_workspace_bytes(1, 32, 8192, 64);\n"
        '  if (ws != (size_t)1 * 32 * 128 * (5 * 64 * 128 + 128) * 4) { puts("bad size"); return 1; }\n'
        "  if (kda_chunk_prefill_workspace_bytes(1, 32, 8192, 48) != 0) return 2;\n"
        '  if (strstr(kda_status_string(KDA_ERR_WORKSPACE), "WORKSPACE") == NULL) return 3;\n'
        "  if (kda_recurrent_step(0, 0, 0, 0, 0, 0, 0, 1, 1, 0) != KDA_ERR_INVALID_ARG) return 4;\n"
        '  puts("ok");\n  return 0;\n}\n')
    inc = os.path.join(ROOT, "include")
    for std, comp in (("-std=c99", "gcc"), ("-std=c++17", "g++")):
        r = subprocess.run([comp, std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-x",
                            "c" if comp == "gcc" else "c++", "-I", inc, "-"], input='#include "kda.h"\n',
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
    exe = tmp_path / "use_kda"
    libdir = os.path.dirname(kda.LIB_PATH)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", inc, str(src), "-o", str(exe), "-L", libdir,
                        "-l:" + os.path.basename(kda.LIB_PATH), "-Wl,-rpath," + libdir], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)


@no_gpu
def test_fused_prefill_refusals(lib):
    f = lib.kda_chunk_prefill_fused
    bad = kda.KDA_ERR_INVALID_ARG
    need = kda.kda_chunk_prefill_workspace_bytes(1, 2, 64, 16)
    ok = (1, 2, 64, 16, 4, 1e-6)  # batch, heads, T, chunk, conv_kernel, l2_eps
    for i in range(7):
        p = list(P[:7])
        p[i] = None
        assert f(*p, *ok, P[7], need, None) == bad, i
        p = list(P[:7])
        p[i] += 8 if i != 4 else 2  # beta needs 4-byte alignment, the rest 16
        assert f(*p, *ok, P[7], need, None) == bad, i
    assert f(*P[:7], 0, 2, 64, 16, 4, 1e-6, P[7], need, None) == bad
    assert f(*P[:7], 1, 0, 64, 16, 4, 1e-6, P[7], need, None) == bad
    assert f(*P[:7], 1, 2, 0, 16, 4, 1e-6, P[7], need, None) == bad
    assert f(*P[:7], 1, 2, 64, 48, 4, 1e-6, P[7], 1 << 30, None) == kda.KDA_ERR_UNSUPPORTED
    for K in (1, 2, 3, 5):
        assert f(*P[:7], 1, 2, 64, 16, K, 1e-6, P[7], need, None) == kda.KDA_ERR_UNSUPPORTED, K
    assert f(*P[:7], 1, 2, 64, 16, 0, 1e-6, P[7], need, None) == bad
    assert f(*P[:7], 1, 2, 64, 16, 4, 0.0, P[7], need, None) == bad
    assert f(*P[:7], 1, 2, 64, 16, 4, float("nan"), P[7], need, None) == bad
    assert f(*P[:7], *ok, P[7], need - 1, None) == kda.KDA_ERR_WORKSPACE
    assert f(*P[:7], *ok, None, need, None) == kda.KDA_ERR_WORKSPACE
    # one sequence's BF16 rows must stay within 32-bit byte offsets: T * 3 * heads * 256 < 2^31
    far = [(i + 1) << 52 for i in range(8)]
    T = (1 << 31) // (3 * 16 * 256) + 1
    assert f(*far[:7], 1, 16, T, 64, 4, 1e-6, far[7], 1 << 62, None) == bad
    for i, j in ((6, 0), (5, 6), (2, 5), (2, 1)):  # out over qkv, state over out, conv state over state / conv_w
        p = list(P[:7])
        p[i] = p[j] + 64
        assert f(*p, *ok, P[7], need, None) == bad, (i, j)
    assert f(*P[:7], *ok, P[2] + 64, need, None) == bad  # workspace over the conv state


@no_gpu
def test_varlen_fused_prefill_refusals(lib):
    f = lib.kda_chunk_prefill_varlen_fused
    bad = kda.KDA_ERR_INVALID_ARG
    need = kda.kda_chunk_prefill_varlen_workspace_bytes(3, 2, 100, 16)
    ok = (3, 2, 100, 16, 4, 1e-6)  # n_seqs, heads, total, chunk, conv_kernel, l2_eps
    for i in range(8):
        p = list(P[:8])
        p[i] = None
        assert f(*p, *ok, P[8], need, None) == bad, i
        p = list(P[:8])
        p[i] += 8 if i not in (4, 7) else 2  # beta and cu_seqlens need 4-byte alignment, the rest 16
        assert f(*p, *ok, P[8], need, None) == bad, i
    assert f(*P[:8], 0, 2, 100, 16, 4, 1e-6, P[8], need, None) == bad
    assert f(*P[:8], (1 << 20) + 1, 2, 100, 16, 4, 1e-6, P[8], 1 << 40, None) == bad
    assert f(*P[:8], 3, 0, 100, 16, 4, 1e-6, P[8], need, None) == bad
    assert f(*P[:8], 3, 2, 0, 16, 4, 1e-6, P[8], need, None) == bad
    assert f(*P[:8], 3, 2, 100, 48, 4, 1e-6, P[8], 1 << 30, None) == kda.KDA_ERR_UNSUPPORTED
    assert f(*P[:8], 3, 2, 100, 16, 3, 1e-6, P[8], need, None) == kda.KDA_ERR_UNSUPPORTED
    assert f(*P[:8], 3, 2, 100, 16, 4, -1.0, P[8], need, None) == bad
    assert f(*P[:8], *ok, P[8], need - 1, None) == kda.KDA_ERR_WORKSPACE
    for i, j in ((6, 0), (7, 2), (5, 2)):  # out over qkv, cu_seqlens inside the conv state, state over conv state
        p = list(P[:8])
        p[i] = p[j] + 64
        assert f(*p, *ok, P[8], need, None) == bad, (i, j)
