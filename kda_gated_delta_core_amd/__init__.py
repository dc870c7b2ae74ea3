"""Python binding of the MI355X KDA gated delta-rule core.

Argument marshalling only: every step of the core runs in the HIP kernels of
``libkda_amd.so`` behind the C ABI of ``include/kda.h``.  The functions carry
the C names; tensors must be contiguous CUDA (HIP) tensors, float32 unless
the header says BF16 (then torch.bfloat16), in the layouts it documents.  PyTorch provides device memory and the stream
(the current torch stream unless one is given).  There is no CPU fallback: if
the library cannot be loaded every call raises.

Outputs the binding allocates (``out=None`` and the like) are allocated on the
current stream, like the result of any torch operation; a caller launching on
another stream keeps them alive until that stream is done, or passes its own.
A prefill workspace the binding allocates is allocated on the launch stream,
so its memory is reused only by work ordered after the call.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda_amd.so")
HEAD_DIM = 128

KDA_OK = 0
KDA_ERR_INVALID_ARG = -1
KDA_ERR_UNSUPPORTED = -2
KDA_ERR_WORKSPACE = -3
KDA_ERR_HIP = -4

EXPORTED = ("kda_status_string", "kda_chunk_prefill_workspace_bytes", "kda_chunk_prefill", "kda_recurrent_step",
            "kda_recurrent_k", "kda_gated_rmsnorm", "kda_decode_front_end",
            "kda_chunk_prefill_varlen_workspace_bytes", "kda_chunk_prefill_varlen", "kda_recurrent_k_bf16",
            "kda_recurrent_step_bf16", "kda_decode_front_end_bf16", "kda_prefill_front_end",
            "kda_prefill_front_end_varlen", "kda_chunk_prefill_transition", "kda_state_transition_apply", "kda_chunk_scan",
            "kda_chunk_prefill_fused", "kda_chunk_prefill_varlen_fused", "kda_chunk_prefill_noalloc",
            "kda_chunk_prefill_gated", "kda_recurrent_k_gated", "kda_recurrent_step_gated",
            "kda_recurrent_k_bf16_norm", "kda_recurrent_step_bf16_norm", "kda_decode_fused_k", "kda_decode_fused_step",
            "kda_decode_fused_k_gated", "kda_decode_fused_step_gated", "kda_chunk_prefill_fused_gated",
            "kda_chunk_prefill_bf16", "kda_chunk_prefill_varlen_bf16")
STATIC_WORKSPACE_BYTES = 256 << 20
GATED_RMSNORM_MIN_EPS = 1e-30

_lib = None


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {kda_status_string(status)} ({status})")
        self.status = status


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libkda_amd.so (building it first only if it does not exist)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(path)
    p, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.kda_status_string.argtypes = [i]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_chunk_prefill_workspace_bytes.argtypes = [i, i, i, i]
    lib.kda_chunk_prefill_workspace_bytes.restype = sz
    lib.kda_chunk_prefill.argtypes = [p] * 7 + [i] * 4 + [p, sz, p]
    lib.kda_chunk_prefill.restype = i
    lib.kda_chunk_prefill_noalloc.argtypes = [p] * 7 + [i] * 4 + [p]
    lib.kda_chunk_prefill_noalloc.restype = i
    f = ctypes.c_float
    lib.kda_chunk_prefill_gated.argtypes = [p] * 7 + [f, p, p] + [i] * 4 + [p, sz, p]
    lib.kda_chunk_prefill_gated.restype = i
    lib.kda_recurrent_k_gated.argtypes = [p] * 7 + [f, p, p, p] + [i] * 4 + [p]
    lib.kda_recurrent_k_gated.restype = i
    lib.kda_recurrent_step_gated.argtypes = [p] * 7 + [f, p, p] + [i, i, p]
    lib.kda_recurrent_step_gated.restype = i
    lib.kda_recurrent_k_bf16_norm.argtypes = [p] * 7 + [f, p, p] + [i] * 4 + [p]
    lib.kda_recurrent_k_bf16_norm.restype = i
    lib.kda_recurrent_step_bf16_norm.argtypes = [p] * 7 + [f, p] + [i, i, p]
    lib.kda_recurrent_step_bf16_norm.restype = i
    lib.kda_decode_fused_k.argtypes = [p] * 8 + [i] + [p] * 2 + [f, f, p, p] + [i] * 4 + [p]
    lib.kda_decode_fused_k.restype = i
    lib.kda_decode_fused_step.argtypes = [p] * 8 + [f, f, p, p] + [i] * 3 + [p]
    lib.kda_decode_fused_step.restype = i
    lib.kda_decode_fused_k_gated.argtypes = [p] * 8 + [f, p, p, i, p, p, f, f, p, p] + [i] * 4 + [p]
    lib.kda_decode_fused_k_gated.restype = i
    lib.kda_decode_fused_step_gated.argtypes = [p] * 7 + [f, p, p, p, f, f, p, p] + [i] * 3 + [p]
    lib.kda_decode_fused_step_gated.restype = i
    lib.kda_recurrent_step.argtypes = [p] * 7 + [i, i, p]
    lib.kda_recurrent_step.restype = i
    lib.kda_recurrent_k.argtypes = [p] * 8 + [i] * 4 + [p]
    lib.kda_recurrent_k.restype = i
    lib.kda_chunk_prefill_varlen_workspace_bytes.argtypes = [i, i, i, i]
    lib.kda_chunk_prefill_varlen_workspace_bytes.restype = sz
    lib.kda_chunk_prefill_varlen.argtypes = [p] * 8 + [i] * 4 + [p, sz, p]
    lib.kda_chunk_prefill_varlen_bf16.argtypes = [p] * 6 + [i] * 4 + [p, sz, p]
    lib.kda_chunk_prefill_varlen_bf16.restype = ctypes.c_int
    lib.kda_chunk_prefill_varlen.restype = i
    lib.kda_gated_rmsnorm.argtypes = [p] * 4 + [i, i, ctypes.c_float, p]
    lib.kda_gated_rmsnorm.restype = i
    lib.kda_decode_front_end.argtypes = [p] * 7 + [i] * 5 + [ctypes.c_float, p]
    lib.kda_decode_front_end.restype = i
    lib.kda_recurrent_k_bf16.argtypes = [p] * 6 + [i] * 4 + [p]
    lib.kda_recurrent_k_bf16.restype = i
    lib.kda_recurrent_step_bf16.argtypes = [p] * 5 + [i, i, p]
    lib.kda_chunk_prefill_bf16.argtypes = [p] * 5 + [i] * 4 + [p, sz, p]
    lib.kda_chunk_prefill_bf16.restype = i
    lib.kda_recurrent_step_bf16.restype = i
    lib.kda_decode_front_end_bf16.argtypes = [p] * 5 + [i] * 5 + [ctypes.c_float, p]
    lib.kda_decode_front_end_bf16.restype = i
    lib.kda_prefill_front_end.argtypes = [p] * 6 + [i] * 5 + [ctypes.c_float, p]
    lib.kda_prefill_front_end.restype = i
    lib.kda_prefill_front_end_varlen.argtypes = [p] * 7 + [i] * 4 + [ctypes.c_float, p]
    lib.kda_prefill_front_end_varlen.restype = i
    lib.kda_chunk_prefill_transition.argtypes = [p] * 7 + [i] * 4 + [p, sz, p]
    lib.kda_chunk_prefill_transition.restype = i
    lib.kda_state_transition_apply.argtypes = [p] * 3 + [i, i, p]
    lib.kda_state_transition_apply.restype = i
    lib.kda_chunk_scan.argtypes = [p, p] + [i] * 4 + [p, sz, p]
    lib.kda_chunk_scan.restype = i
    lib.kda_chunk_prefill_fused.argtypes = [p] * 7 + [i] * 5 + [ctypes.c_float, p, sz, p]
    lib.kda_chunk_prefill_fused.restype = i
    lib.kda_chunk_prefill_fused_gated.argtypes = [p] * 7 + [f] + [p] * 2 + [i] * 5 + [f, p, sz, p]
    lib.kda_chunk_prefill_fused_gated.restype = i
    lib.kda_chunk_prefill_varlen_fused.argtypes = [p] * 8 + [i] * 5 + [ctypes.c_float, p, sz, p]
    lib.kda_chunk_prefill_varlen_fused.restype = i
    if path == LIB_PATH:
        _lib = lib
    return lib


def kda_status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def kda_chunk_prefill_workspace_bytes(batch: int, heads: int, T: int, chunk: int) -> int:
    return int(load_library().kda_chunk_prefill_workspace_bytes(batch, heads, T, chunk))


def _stream_ptr(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _workspace(nbytes: int, device, stream) -> torch.Tensor:
    """A workspace the binding allocates for one call.  It is allocated on the stream the call is
    launched on: the caching allocator then hands its memory out again only to work ordered after
    this call on that stream, even though the tensor is dropped as soon as the call returns."""
    if stream is None:
        s = torch.cuda.current_stream(device)
    elif isinstance(stream, torch.cuda.Stream):
        s = stream
    else:
        s = torch.cuda.ExternalStream(int(stream), device=device)
    with torch.cuda.stream(s):
        return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _check(name: str, t: torch.Tensor, shape: tuple, dtype=torch.float32) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _vec_shapes(q: torch.Tensor):
    if q.dim() != 4 or q.shape[-1] != HEAD_DIM:
        raise ValueError(f"q must be [batch][rows][heads][{HEAD_DIM}]")
    B, rows, H, _ = q.shape
    return B, rows, H


def kda_recurrent_k(q, k, v, gate, beta, state, out=None, snapshots=None, n_snapshots: int = 0, stream=None):
    """Walk the rows of each sequence one at a time (decode_k).  Returns ``out``.

    q, k, v, gate: [B][T][H][128]; beta: [B][T][H]; state: [B][H][128][128] (in place);
    snapshots: [>= n_snapshots][B][H][128][128] receives the state after rows 0..n_snapshots-1.
    """
    B, T, H = _vec_shapes(q)
    vs = (B, T, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=q.device)
    args = [_check(n, t, vs) for n, t in (("q", q), ("k", k), ("v", v), ("gate", gate))]
    args.append(_check("beta", beta, (B, T, H)))
    args.append(_check("state", state, (B, H, HEAD_DIM, HEAD_DIM)))
    args.append(_check("out", out, vs))
    snap_ptr = None
    if n_snapshots:
        if snapshots is None or snapshots.dim() != 5 or snapshots.shape[0] < n_snapshots:
            raise ValueError("snapshots must be [>= n_snapshots][B][H][128][128]")
        snap_ptr = _check("snapshots", snapshots, (snapshots.shape[0], B, H, HEAD_DIM, HEAD_DIM))
    rc = load_library().kda_recurrent_k(*args, snap_ptr, int(n_snapshots), B, H, T, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_recurrent_k", rc)
    return out


def kda_recurrent_step(q, k, v, gate, beta, state, out=None, stream=None):
    """One decode token per sequence.  q, k, v, gate: [B][1][H][128]; beta: [B][1][H]."""
    B, rows, H = _vec_shapes(q)
    if rows != 1:
        raise ValueError("kda_recurrent_step takes one row per sequence")
    vs = (B, 1, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=q.device)
    args = [_check(n, t, vs) for n, t in (("q", q), ("k", k), ("v", v), ("gate", gate))]
    args.append(_check("beta", beta, (B, 1, H)))
    args.append(_check("state", state, (B, H, HEAD_DIM, HEAD_DIM)))
    args.append(_check("out", out, vs))
    rc = load_library().kda_recurrent_step(*args, B, H, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_recurrent_step", rc)
    return out


def _packed_qkv(qkv, gate):
    """Shapes of a BF16 q | k | v tensor, [B][T][3 H 128] or [B][T][3][H][128], against gate [B][T][H][128]."""
    B, T, H = _vec_shapes(gate)
    if not isinstance(qkv, torch.Tensor) or qkv.dim() not in (3, 5):
        raise ValueError("qkv must be [batch][T][3 * heads * 128] or [batch][T][3][heads][128]")
    shape = (B, T, 3 * H * HEAD_DIM) if qkv.dim() == 3 else (B, T, 3, H, HEAD_DIM)
    return B, T, H, _check("qkv", qkv, shape, torch.bfloat16)


def kda_recurrent_k_bf16(qkv, gate, beta, state, out=None, snapshots=None, n_snapshots: int = 0, stream=None):
    """kda_recurrent_k with BF16 q | k | v packed per token (the BF16 front end's conv_out).  Returns ``out``.

    qkv: bfloat16 [B][T][3 H 128] (or [B][T][3][H][128]); gate: [B][T][H][128]; beta: [B][T][H];
    state: [B][H][128][128] (in place); snapshots: [>= n_snapshots][B][H][128][128].
    """
    B, T, H, qkv_ptr = _packed_qkv(qkv, gate)
    vs = (B, T, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=gate.device)
    args = [qkv_ptr, _check("gate", gate, vs), _check("beta", beta, (B, T, H)),
            _check("state", state, (B, H, HEAD_DIM, HEAD_DIM)), _check("out", out, vs)]
    snap_ptr = None
    if n_snapshots:
        if snapshots is None or snapshots.dim() != 5 or snapshots.shape[0] < n_snapshots:
            raise ValueError("snapshots must be [>= n_snapshots][B][H][128][128]")
        snap_ptr = _check("snapshots", snapshots, (snapshots.shape[0], B, H, HEAD_DIM, HEAD_DIM))
    rc = load_library().kda_recurrent_k_bf16(*args, snap_ptr, int(n_snapshots), B, H, T, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_recurrent_k_bf16", rc)
    return out


def kda_recurrent_step_bf16(qkv, gate, beta, state, out=None, stream=None):
    """One decode token per sequence from BF16 q | k | v.  qkv: [B][1][3 H 128]; gate: [B][1][H][128]."""
    B, T, H, qkv_ptr = _packed_qkv(qkv, gate)
    if T != 1:
        raise ValueError("kda_recurrent_step_bf16 takes one row per sequence")
    vs = (B, 1, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=gate.device)
    args = [qkv_ptr, _check("gate", gate, vs), _check("beta", beta, (B, 1, H)),
            _check("state", state, (B, H, HEAD_DIM, HEAD_DIM)), _check("out", out, vs)]
    rc = load_library().kda_recurrent_step_bf16(*args, B, H, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_recurrent_step_bf16", rc)
    return out


def kda_chunk_prefill_bf16(qkv, gate, beta, state, T: int, chunk: int, out=None, workspace=None, stream=None):
    """kda_chunk_prefill with BF16 q | k | v packed per token.  Returns ``out``.

    qkv: bfloat16 [B][T_pad][3 H 128] (or [B][T_pad][3][H][128]); gate, out: [B][T_pad][H][128];
    beta: [B][T_pad][H]; state and workspace as kda_chunk_prefill.
    """
    if chunk not in (16, 32, 64):
        raise KdaError("kda_chunk_prefill_bf16", KDA_ERR_UNSUPPORTED)
    B, rows, H, qkv_ptr = _packed_qkv(qkv, gate)
    t_pad = -(-int(T) // chunk) * chunk
    if rows != t_pad:
        raise ValueError(f"inputs must hold T_pad = {t_pad} rows per sequence, got {rows}")
    vs = (B, t_pad, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=gate.device)
    need = kda_chunk_prefill_workspace_bytes(B, H, int(T), chunk)
    if workspace is None:
        workspace = _workspace(need, gate.device, stream)
    if not (workspace.device.type == "cuda" and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = load_library().kda_chunk_prefill_bf16(qkv_ptr, _check("gate", gate, vs), _check("beta", beta, (B, t_pad, H)),
                                               _check("state", state, (B, H, HEAD_DIM, HEAD_DIM)),
                                               _check("out", out, vs), B, H, int(T), chunk, workspace.data_ptr(),
                                               ws_bytes, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_chunk_prefill_bf16", rc)
    return out


def kda_chunk_prefill(q, k, v, gate, beta, state, T: int, chunk: int, out=None, workspace=None, stream=None):
    """Chunked prefill of T tokens per sequence.  Returns ``out``.

    q, k, v, gate, out: [B][T_pad][H][128] with T_pad = ceil(T/chunk)*chunk; beta: [B][T_pad][H];
    state: [B][H][128][128] (in place); workspace: a uint8 CUDA tensor of at least
    kda_chunk_prefill_workspace_bytes(B, H, T, chunk) bytes (allocated here when None).
    """
    B, rows, H = _vec_shapes(q)
    if chunk not in (16, 32, 64):
        raise KdaError("kda_chunk_prefill", KDA_ERR_UNSUPPORTED)
    t_pad = -(-int(T) // chunk) * chunk
    if rows != t_pad:
        raise ValueError(f"inputs must hold T_pad = {t_pad} rows per sequence, got {rows}")
    vs = (B, t_pad, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=q.device)
    need = kda_chunk_prefill_workspace_bytes(B, H, int(T), chunk)
    if workspace is None:
        workspace = _workspace(need, q.device, stream)
    if not (workspace.device.type == "cuda" and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    args = [_check(n, t, vs) for n, t in (("q", q), ("k", k), ("v", v), ("gate", gate))]
    args.append(_check("beta", beta, (B, t_pad, H)))
    args.append(_check("state", state, (B, H, HEAD_DIM, HEAD_DIM)))
    args.append(_check("out", out, vs))
    rc = load_library().kda_chunk_prefill(*args, B, H, int(T), chunk, workspace.data_ptr(), ws_bytes,
                                          _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_chunk_prefill", rc)
    return out


def kda_chunk_prefill_noalloc(q, k, v, gate, beta, state, T: int, chunk: int, out, stream=None):
    """kda_chunk_prefill with its chunk records in the library's static device array (no workspace,
    no allocation anywhere; ``out`` must be given).  At most STATIC_WORKSPACE_BYTES of records
    (kda_chunk_prefill_workspace_bytes); calls that may overlap on one GPU race on the array."""
    B, rows, H = _vec_shapes(q)
    if chunk not in (16, 32, 64):
        raise KdaError("kda_chunk_prefill_noalloc", KDA_ERR_UNSUPPORTED)
    t_pad = -(-int(T) // chunk) * chunk
    if rows != t_pad:
        raise ValueError(f"inputs must hold T_pad = {t_pad} rows per sequence, got {rows}")
    vs = (B, t_pad, H, HEAD_DIM)
    args = [_check(n, t, vs) for n, t in (("q", q), ("k", k), ("v", v), ("gate", gate))]
    args.append(_check("beta", beta, (B, t_pad, H)))
    args.append(_check("state", state, (B, H, HEAD_DIM, HEAD_DIM)))
    args.append(_check("out", out, vs))
    rc = load_library().kda_chunk_prefill_noalloc(*args, B, H, int(T), chunk, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_chunk_prefill_noalloc", rc)
    return out


def _gate_args(g_raw, beta_logit, dt_bias, a_log, B, rows, H):
    return [_check("g_raw", g_raw, (B, rows, H, HEAD_DIM), torch.bfloat16),
            _check("beta_logit", beta_logit, (B, rows, H)),
            _check("dt_bias", dt_bias, (H, HEAD_DIM)),
            _check("a_log", a_log, (H,))]


def kda_chunk_prefill_gated(q, k, v, g_raw, beta_logit, dt_bias, a_log, gate_lower_bound: float, state, T: int,
                            chunk: int, out=None, workspace=None, stream=None):
    """kda_chunk_prefill with gate = kda_gate(g_raw) and beta = sigmoid(beta_logit) formed inside the
    prefill.  g_raw: [B][T_pad][H][128] bfloat16; beta_logit: [B][T_pad][H]; dt_bias: [H][128];
    a_log: [H]; the rest as kda_chunk_prefill.  Returns ``out``."""
    B, rows, H = _vec_shapes(q)
    if chunk not in (16, 32, 64):
        raise KdaError("kda_chunk_prefill_gated", KDA_ERR_UNSUPPORTED)
    t_pad = -(-int(T) // chunk) * chunk
    if rows != t_pad:
        raise ValueError(f"inputs must hold T_pad = {t_pad} rows per sequence, got {rows}")
    vs = (B, t_pad, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=q.device)
    need = kda_chunk_prefill_workspace_bytes(B, H, int(T), chunk)
    if workspace is None:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    qkv = [_check(n, t, vs) for n, t in (("q", q), ("k", k), ("v", v))]
    g, b, dt, al = _gate_args(g_raw, beta_logit, dt_bias, a_log, B, t_pad, H)
    rc = load_library().kda_chunk_prefill_gated(*qkv, g, b, dt, al, float(gate_lower_bound),
                                                _check("state", state, (B, H, HEAD_DIM, HEAD_DIM)),
                                                _check("out", out, vs), B, H, int(T), chunk, workspace.data_ptr(),
                                                ws_bytes, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_chunk_prefill_gated", rc)
    return out


def kda_recurrent_k_gated(q, k, v, g_raw, beta_logit, dt_bias, a_log, gate_lower_bound: float, state, out=None,
                          snapshots=None, n_snapshots: int = 0, stream=None):
    """kda_recurrent_k with gate = kda_gate(g_raw) and beta = sigmoid(beta_logit) formed in the decode
    kernel.  g_raw: [B][T][H][128] bfloat16; beta_logit: [B][T][H]; dt_bias: [H][128]; a_log: [H]."""
    B, T, H = _vec_shapes(q)
    vs = (B, T, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=q.device)
    qkv = [_check(n, t, vs) for n, t in (("q", q), ("k", k), ("v", v))]
    g, b, dt, al = _gate_args(g_raw, beta_logit, dt_bias, a_log, B, T, H)
    snap_ptr = None
    if n_snapshots:
        if snapshots is None or snapshots.dim() != 5 or snapshots.shape[0] < n_snapshots:
            raise ValueError("snapshots must be [>= n_snapshots][B][H][128][128]")
        snap_ptr = _check("snapshots", snapshots, (snapshots.shape[0], B, H, HEAD_DIM, HEAD_DIM))
    rc = load_library().kda_recurrent_k_gated(*qkv, g, b, dt, al, float(gate_lower_bound),
                                              _check("state", state, (B, H, HEAD_DIM, HEAD_DIM)),
                                              _check("out", out, vs), snap_ptr, int(n_snapshots), B, H, T,
                                              _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_recurrent_k_gated", rc)
    return out


def kda_recurrent_step_gated(q, k, v, g_raw, beta_logit, dt_bias, a_log, gate_lower_bound: float, state, out=None,
                             stream=None):
    """One decode step with the gate and beta formed in the kernel (kda_recurrent_k_gated with T = 1)."""
    B, rows, H = _vec_shapes(q)
    if rows != 1:
        raise ValueError("kda_recurrent_step_gated takes one row per sequence")
    vs = (B, 1, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=q.device)
    qkv = [_check(n, t, vs) for n, t in (("q", q), ("k", k), ("v", v))]
    g, b, dt, al = _gate_args(g_raw, beta_logit, dt_bias, a_log, B, 1, H)
    rc = load_library().kda_recurrent_step_gated(*qkv, g, b, dt, al, float(gate_lower_bound),
                                                 _check("state", state, (B, H, HEAD_DIM, HEAD_DIM)),
                                                 _check("out", out, vs), B, H, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_recurrent_step_gated", rc)
    return out


def kda_chunk_prefill_transition(q, k, v, gate, beta, T: int, chunk: int, trans_p=None, trans_q=None,
                                 workspace=None, stream=None):
    """Segment transition of a prefill: (P, Q), [B][H][128][128] each, such that the prefill of these T
    tokens from any initial state S ends in P S + Q.  Inputs and workspace as kda_chunk_prefill.
    Returns (trans_p, trans_q)."""
    B, rows, H = _vec_shapes(q)
    if chunk not in (16, 32, 64):
        raise KdaError("kda_chunk_prefill_transition", KDA_ERR_UNSUPPORTED)
    t_pad = -(-int(T) // chunk) * chunk
    if rows != t_pad:
        raise ValueError(f"inputs must hold T_pad = {t_pad} rows per sequence, got {rows}")
    vs, ss = (B, t_pad, H, HEAD_DIM), (B, H, HEAD_DIM, HEAD_DIM)
    if trans_p is None:
        trans_p = torch.empty(ss, dtype=torch.float32, device=q.device)
    if trans_q is None:
        trans_q = torch.empty(ss, dtype=torch.float32, device=q.device)
    need = kda_chunk_prefill_workspace_bytes(B, H, int(T), chunk)
    if workspace is None:
        workspace = _workspace(need, q.device, stream)
    if not (workspace.device.type == "cuda" and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    args = [_check(n, t, vs) for n, t in (("q", q), ("k", k), ("v", v), ("gate", gate))]
    args.append(_check("beta", beta, (B, t_pad, H)))
    args.append(_check("trans_p", trans_p, ss))
    args.append(_check("trans_q", trans_q, ss))
    rc = load_library().kda_chunk_prefill_transition(*args, B, H, int(T), chunk, workspace.data_ptr(), ws_bytes,
                                                     _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_chunk_prefill_transition", rc)
    return trans_p, trans_q


def kda_chunk_scan(state, T: int, chunk: int, workspace, out=None, stream=None):
    """The scan half of kda_chunk_prefill alone, from the chunk records a preceding kda_chunk_prefill or
    kda_chunk_prefill_transition with the same (B, H, T, chunk) left in ``workspace``.  state:
    [B][H][128][128] (in place); out: [B][T_pad][H][128].  Returns ``out``."""
    if not isinstance(state, torch.Tensor) or state.dim() != 4:
        raise ValueError("state must be [batch][heads][128][128]")
    if chunk not in (16, 32, 64):
        raise KdaError("kda_chunk_scan", KDA_ERR_UNSUPPORTED)
    B, H = state.shape[0], state.shape[1]
    t_pad = -(-int(T) // chunk) * chunk
    vs = (B, t_pad, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=state.device)
    if not (isinstance(workspace, torch.Tensor) and workspace.device.type == "cuda" and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor holding the chunk records")
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = load_library().kda_chunk_scan(_check("state", state, (B, H, HEAD_DIM, HEAD_DIM)), _check("out", out, vs), B, H,
                                       int(T), chunk, workspace.data_ptr(), ws_bytes, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_chunk_scan", rc)
    return out


def kda_state_transition_apply(trans_p, trans_q, state, stream=None):
    """state <- trans_p @ state + trans_q in place (trans_q None: trans_p @ state), per (sequence, head);
    all [B][H][128][128] float32.  Returns ``state``."""
    if not isinstance(state, torch.Tensor) or state.dim() != 4:
        raise ValueError("state must be [batch][heads][128][128]")
    B, H = state.shape[0], state.shape[1]
    ss = (B, H, HEAD_DIM, HEAD_DIM)
    args = [_check("trans_p", trans_p, ss), None if trans_q is None else _check("trans_q", trans_q, ss),
            _check("state", state, ss)]
    rc = load_library().kda_state_transition_apply(*args, B, H, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_state_transition_apply", rc)
    return state


def kda_recurrent_k_bf16_norm(qkv, gate, beta, state, out_gate, o_norm, eps: float, y=None, out=None,
                              snapshots=None, n_snapshots: int = 0, want_core: bool = True, stream=None):
    """kda_recurrent_k_bf16 with the gated RMSNorm of every output row fused in.  Returns (y, out): y
    [B][T][H][128] bfloat16; out the FP32 core rows (None when want_core is False and out is None)."""
    B, T, H, qkv_ptr = _packed_qkv(qkv, gate)
    vs = (B, T, H, HEAD_DIM)
    if y is None:
        y = torch.empty(vs, dtype=torch.bfloat16, device=qkv.device)
    if out is None and want_core:
        out = torch.empty(vs, dtype=torch.float32, device=qkv.device)
    snap_ptr = None
    if n_snapshots:
        if snapshots is None or snapshots.dim() != 5 or snapshots.shape[0] < n_snapshots:
            raise ValueError("snapshots must be [>= n_snapshots][B][H][128][128]")
        snap_ptr = _check("snapshots", snapshots, (snapshots.shape[0], B, H, HEAD_DIM, HEAD_DIM))
    rc = load_library().kda_recurrent_k_bf16_norm(
        qkv_ptr, _check("gate", gate, vs),
        _check("beta", beta, (B, T, H)), _check("state", state, (B, H, HEAD_DIM, HEAD_DIM)),
        _check("out", out, vs) if out is not None else None, _check("out_gate", out_gate, vs, torch.bfloat16),
        _check("o_norm", o_norm, (HEAD_DIM,), torch.bfloat16), float(eps), _check("y", y, vs, torch.bfloat16),
        snap_ptr, int(n_snapshots), B, H, T, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_recurrent_k_bf16_norm", rc)
    return y, out


def kda_recurrent_step_bf16_norm(qkv, gate, beta, state, out_gate, o_norm, eps: float, y=None, out=None,
                                 want_core: bool = True, stream=None):
    """One BF16 decode step with the gated RMSNorm fused in (kda_recurrent_k_bf16_norm with T = 1)."""
    B, T, H, qkv_ptr = _packed_qkv(qkv, gate)
    if T != 1:
        raise ValueError("kda_recurrent_step_bf16_norm takes one row per sequence")
    vs = (B, 1, H, HEAD_DIM)
    if y is None:
        y = torch.empty(vs, dtype=torch.bfloat16, device=qkv.device)
    if out is None and want_core:
        out = torch.empty(vs, dtype=torch.float32, device=qkv.device)
    rc = load_library().kda_recurrent_step_bf16_norm(
        qkv_ptr, _check("gate", gate, vs),
        _check("beta", beta, (B, 1, H)), _check("state", state, (B, H, HEAD_DIM, HEAD_DIM)),
        _check("out", out, vs) if out is not None else None, _check("out_gate", out_gate, vs, torch.bfloat16),
        _check("o_norm", o_norm, (HEAD_DIM,), torch.bfloat16), float(eps), _check("y", y, vs, torch.bfloat16), B, H,
        _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_recurrent_step_bf16_norm", rc)
    return y, out


def _fused_args(qkv_proj, conv_w, conv_state, heads, out_gate, o_norm, y, out, snapshots, conv_snapshots,
                n_snapshots, want_core):
    if not isinstance(qkv_proj, torch.Tensor) or qkv_proj.dim() != 3:
        raise ValueError("qkv_proj must be [batch][T][3 * heads * 128]")
    B, T, C = qkv_proj.shape
    if C != 3 * heads * HEAD_DIM:
        raise ValueError(f"qkv_proj has {C} channels, expected 3 * {heads} * {HEAD_DIM}")
    if conv_w.dim() != 2:
        raise ValueError("conv_w must be [conv_dim][conv_kernel]")
    K = conv_w.shape[1]
    vs = (B, T, heads, HEAD_DIM)
    if y is None:
        y = torch.empty(vs, dtype=torch.bfloat16, device=qkv_proj.device)
    if out is None and want_core:
        out = torch.empty(vs, dtype=torch.float32, device=qkv_proj.device)
    snap_ptr = csnap_ptr = None
    if n_snapshots:
        if snapshots is None or snapshots.dim() != 5 or snapshots.shape[0] < n_snapshots:
            raise ValueError("snapshots must be [>= n_snapshots][B][H][128][128]")
        if conv_snapshots is None or conv_snapshots.dim() != 4 or conv_snapshots.shape[0] < n_snapshots:
            raise ValueError("conv_snapshots must be [>= n_snapshots][B][conv_dim][conv_kernel]")
        snap_ptr = _check("snapshots", snapshots, (snapshots.shape[0], B, heads, HEAD_DIM, HEAD_DIM))
        csnap_ptr = _check("conv_snapshots", conv_snapshots, (conv_snapshots.shape[0], B, C, K))
    head = [_check("qkv_proj", qkv_proj, (B, T, C), torch.bfloat16), _check("conv_w", conv_w, (C, K), torch.bfloat16),
            _check("conv_state", conv_state, (B, C, K))]
    tail = [_check("out_gate", out_gate, vs, torch.bfloat16), _check("o_norm", o_norm, (HEAD_DIM,), torch.bfloat16)]
    return B, T, K, vs, y, out, snap_ptr, csnap_ptr, head, tail


def kda_decode_fused_k(qkv_proj, conv_w, conv_state, gate, beta, state, out_gate, o_norm, heads: int,
                       norm_eps: float, l2_eps: float, y=None, out=None, snapshots=None, conv_snapshots=None,
                       n_snapshots: int = 0, want_core: bool = True, stream=None):
    """The decode walk from the raw projections in one kernel: front end, recurrence and gated RMSNorm.
    qkv_proj: bfloat16 [B][T][3 H 128]; conv_w, conv_state: as kda_decode_front_end; gate: [B][T][H][128];
    beta: [B][T][H]; state in place; out_gate: bfloat16 [B][T][H][128]; o_norm: bfloat16 [128].
    Returns (y, out): y bfloat16 [B][T][H][128]; out the FP32 core rows (None without want_core)."""
    B, T, K, vs, y, out, sp, cp, head, tail = _fused_args(qkv_proj, conv_w, conv_state, heads, out_gate, o_norm, y,
                                                          out, snapshots, conv_snapshots, n_snapshots, want_core)
    rc = load_library().kda_decode_fused_k(
        *head, cp, _check("gate", gate, vs), _check("beta", beta, (B, T, heads)),
        _check("state", state, (B, heads, HEAD_DIM, HEAD_DIM)), sp, int(n_snapshots), *tail, float(norm_eps),
        float(l2_eps), _check("y", y, vs, torch.bfloat16), _check("out", out, vs) if out is not None else None, B,
        heads, T, K, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_decode_fused_k", rc)
    return y, out


def kda_decode_fused_step(qkv_proj, conv_w, conv_state, gate, beta, state, out_gate, o_norm, heads: int,
                          norm_eps: float, l2_eps: float, y=None, out=None, want_core: bool = True, stream=None):
    """One decode step from the raw projections (kda_decode_fused_k with T = 1).  Returns (y, out)."""
    B, T, K, vs, y, out, _, _, head, tail = _fused_args(qkv_proj, conv_w, conv_state, heads, out_gate, o_norm, y,
                                                        out, None, None, 0, want_core)
    if T != 1:
        raise ValueError("kda_decode_fused_step takes one row per sequence")
    rc = load_library().kda_decode_fused_step(
        *head, _check("gate", gate, vs), _check("beta", beta, (B, 1, heads)),
        _check("state", state, (B, heads, HEAD_DIM, HEAD_DIM)), *tail, float(norm_eps), float(l2_eps),
        _check("y", y, vs, torch.bfloat16), _check("out", out, vs) if out is not None else None, B, heads, K,
        _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_decode_fused_step", rc)
    return y, out


def kda_decode_fused_k_gated(qkv_proj, conv_w, conv_state, g_raw, beta_logit, dt_bias, a_log, gate_lower_bound: float,
                             state, out_gate, o_norm, heads: int, norm_eps: float, l2_eps: float, y=None, out=None,
                             snapshots=None, conv_snapshots=None, n_snapshots: int = 0, want_core: bool = True,
                             stream=None):
    """kda_decode_fused_k with the gate and beta formed in the kernel from g_raw and beta_logit (as
    kda_recurrent_k_gated).  Returns (y, out)."""
    B, T, K, vs, y, out, sp, cp, head, tail = _fused_args(qkv_proj, conv_w, conv_state, heads, out_gate, o_norm, y,
                                                          out, snapshots, conv_snapshots, n_snapshots, want_core)
    g, b, dt, al = _gate_args(g_raw, beta_logit, dt_bias, a_log, B, T, heads)
    rc = load_library().kda_decode_fused_k_gated(
        *head, cp, g, b, dt, al, float(gate_lower_bound), _check("state", state, (B, heads, HEAD_DIM, HEAD_DIM)), sp,
        int(n_snapshots), *tail, float(norm_eps), float(l2_eps), _check("y", y, vs, torch.bfloat16),
        _check("out", out, vs) if out is not None else None, B, heads, T, K, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_decode_fused_k_gated", rc)
    return y, out


def kda_decode_fused_step_gated(qkv_proj, conv_w, conv_state, g_raw, beta_logit, dt_bias, a_log,
                                gate_lower_bound: float, state, out_gate, o_norm, heads: int, norm_eps: float,
                                l2_eps: float, y=None, out=None, want_core: bool = True, stream=None):
    """One gated decode step from the raw projections (kda_decode_fused_k_gated with T = 1)."""
    B, T, K, vs, y, out, _, _, head, tail = _fused_args(qkv_proj, conv_w, conv_state, heads, out_gate, o_norm, y,
                                                        out, None, None, 0, want_core)
    if T != 1:
        raise ValueError("kda_decode_fused_step_gated takes one row per sequence")
    g, b, dt, al = _gate_args(g_raw, beta_logit, dt_bias, a_log, B, 1, heads)
    rc = load_library().kda_decode_fused_step_gated(
        *head, g, b, dt, al, float(gate_lower_bound), _check("state", state, (B, heads, HEAD_DIM, HEAD_DIM)), *tail,
        float(norm_eps), float(l2_eps), _check("y", y, vs, torch.bfloat16),
        _check("out", out, vs) if out is not None else None, B, heads, K, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_decode_fused_step_gated", rc)
    return y, out


def kda_gated_rmsnorm(core, out_gate, o_norm, eps: float, out=None, stream=None):
    """Sigmoid-gated RMSNorm over the last (128-channel) dimension.  Returns ``out``.

    core: float32 [..., H, 128] (e.g. the [B][rows][H][128] output of the core);
    out_gate: bfloat16 of the same shape; o_norm: bfloat16 [128]; out: bfloat16 like out_gate.
    """
    if not isinstance(core, torch.Tensor) or core.dim() < 2 or core.shape[-1] != HEAD_DIM:
        raise ValueError(f"core must be [..., heads, {HEAD_DIM}]")
    shape = tuple(core.shape)
    H = shape[-2]
    rows = core.numel() // (H * HEAD_DIM) if H else 0
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=core.device)
    args = [_check("core", core, shape), _check("out_gate", out_gate, shape, torch.bfloat16),
            _check("o_norm", o_norm, (HEAD_DIM,), torch.bfloat16), _check("out", out, shape, torch.bfloat16)]
    rc = load_library().kda_gated_rmsnorm(*args, rows, H, float(eps), _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_gated_rmsnorm", rc)
    return out


def kda_decode_front_end(qkv, conv_w, conv_state, heads: int, l2_eps: float, q=None, k=None, v=None,
                         conv_snapshots=None, n_snapshots: int = 0, stream=None):
    """Conv1d update + SiLU + L2(q, k) over T rows per sequence.  Returns (q, k, v).

    qkv: bfloat16 [B][T][3 H 128]; conv_w: bfloat16 [3 H 128][K]; conv_state: float32 [B][3 H 128][K]
    (in place); q, k, v: float32 [B][T][H][128]; conv_snapshots: float32 [>= n][B][3 H 128][K].
    """
    if not isinstance(qkv, torch.Tensor) or qkv.dim() != 3:
        raise ValueError("qkv must be [batch][T][3 * heads * 128]")
    B, T, C = qkv.shape
    if C != 3 * heads * HEAD_DIM:
        raise ValueError(f"qkv has {C} channels, expected 3 * {heads} * {HEAD_DIM}")
    if conv_w.dim() != 2:
        raise ValueError("conv_w must be [conv_dim][conv_kernel]")
    K = conv_w.shape[1]
    vs = (B, T, heads, HEAD_DIM)
    q = torch.empty(vs, dtype=torch.float32, device=qkv.device) if q is None else q
    k = torch.empty(vs, dtype=torch.float32, device=qkv.device) if k is None else k
    v = torch.empty(vs, dtype=torch.float32, device=qkv.device) if v is None else v
    args = [_check("qkv", qkv, (B, T, C), torch.bfloat16), _check("conv_w", conv_w, (C, K), torch.bfloat16),
            _check("conv_state", conv_state, (B, C, K)), _check("q", q, vs), _check("k", k, vs), _check("v", v, vs)]
    snap_ptr = None
    if n_snapshots:
        if conv_snapshots is None or conv_snapshots.dim() != 4 or conv_snapshots.shape[0] < n_snapshots:
            raise ValueError("conv_snapshots must be [>= n_snapshots][B][conv_dim][conv_kernel]")
        snap_ptr = _check("conv_snapshots", conv_snapshots, (conv_snapshots.shape[0], B, C, K))
    rc = load_library().kda_decode_front_end(*args, snap_ptr, int(n_snapshots), B, heads, T, K, float(l2_eps),
                                             _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_decode_front_end", rc)
    return q, k, v


def kda_decode_front_end_bf16(qkv, conv_w, conv_state, heads: int, l2_eps: float, conv_out=None,
                              conv_snapshots=None, n_snapshots: int = 0, stream=None):
    """kda_decode_front_end with BF16 output in the input's layout.  Returns conv_out [B][T][3 H 128] bfloat16."""
    if not isinstance(qkv, torch.Tensor) or qkv.dim() != 3:
        raise ValueError("qkv must be [batch][T][3 * heads * 128]")
    B, T, C = qkv.shape
    if C != 3 * heads * HEAD_DIM:
        raise ValueError(f"qkv has {C} channels, expected 3 * {heads} * {HEAD_DIM}")
    if conv_w.dim() != 2:
        raise ValueError("conv_w must be [conv_dim][conv_kernel]")
    K = conv_w.shape[1]
    if conv_out is None:
        conv_out = torch.empty((B, T, C), dtype=torch.bfloat16, device=qkv.device)
    args = [_check("qkv", qkv, (B, T, C), torch.bfloat16), _check("conv_w", conv_w, (C, K), torch.bfloat16),
            _check("conv_state", conv_state, (B, C, K)), _check("conv_out", conv_out, (B, T, C), torch.bfloat16)]
    snap_ptr = None
    if n_snapshots:
        if conv_snapshots is None or conv_snapshots.dim() != 4 or conv_snapshots.shape[0] < n_snapshots:
            raise ValueError("conv_snapshots must be [>= n_snapshots][B][conv_dim][conv_kernel]")
        snap_ptr = _check("conv_snapshots", conv_snapshots, (conv_snapshots.shape[0], B, C, K))
    rc = load_library().kda_decode_front_end_bf16(*args, snap_ptr, int(n_snapshots), B, heads, T, K, float(l2_eps),
                                                  _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_decode_front_end_bf16", rc)
    return conv_out


def kda_prefill_front_end(qkv, conv_w, conv_state, heads: int, chunk: int, l2_eps: float, q=None, k=None, v=None,
                          stream=None):
    """Conv1d + SiLU + L2(q, k) over the T tokens of a prefill.  Returns (q, k, v).

    qkv: bfloat16 [B][T][3 H 128]; conv_w: bfloat16 [3 H 128][K]; conv_state: float32 [B][3 H 128][K]
    (advanced in place); q, k, v: float32 [B][T_pad][H][128], T_pad = ceil(T / chunk) * chunk (rows >= T
    are not written), ready for kda_chunk_prefill(..., T, chunk).
    """
    if not isinstance(qkv, torch.Tensor) or qkv.dim() != 3:
        raise ValueError("qkv must be [batch][T][3 * heads * 128]")
    B, T, C = qkv.shape
    if C != 3 * heads * HEAD_DIM:
        raise ValueError(f"qkv has {C} channels, expected 3 * {heads} * {HEAD_DIM}")
    if chunk not in (16, 32, 64):
        raise KdaError("kda_prefill_front_end", KDA_ERR_UNSUPPORTED)
    if conv_w.dim() != 2:
        raise ValueError("conv_w must be [conv_dim][conv_kernel]")
    K = conv_w.shape[1]
    t_pad = -(-int(T) // chunk) * chunk
    vs = (B, t_pad, heads, HEAD_DIM)
    q = torch.empty(vs, dtype=torch.float32, device=qkv.device) if q is None else q
    k = torch.empty(vs, dtype=torch.float32, device=qkv.device) if k is None else k
    v = torch.empty(vs, dtype=torch.float32, device=qkv.device) if v is None else v
    args = [_check("qkv", qkv, (B, T, C), torch.bfloat16), _check("conv_w", conv_w, (C, K), torch.bfloat16),
            _check("conv_state", conv_state, (B, C, K)), _check("q", q, vs), _check("k", k, vs), _check("v", v, vs)]
    rc = load_library().kda_prefill_front_end(*args, B, heads, T, chunk, K, float(l2_eps), _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_prefill_front_end", rc)
    return q, k, v


def kda_chunk_prefill_fused(qkv, conv_w, conv_state, gate, beta, state, chunk: int, l2_eps: float, out=None,
                            workspace=None, stream=None):
    """kda_prefill_front_end + kda_chunk_prefill with the front end fused into the prefill.  Returns ``out``.

    qkv: bfloat16 [B][T][3 H 128]; conv_w: bfloat16 [3 H 128][4]; conv_state: float32 [B][3 H 128][4]
    (advanced in place); gate: [B][T_pad][H][128]; beta: [B][T_pad][H]; state: [B][H][128][128] (in place);
    out: [B][T_pad][H][128]; workspace as kda_chunk_prefill.
    """
    if not isinstance(qkv, torch.Tensor) or qkv.dim() != 3:
        raise ValueError("qkv must be [batch][T][3 * heads * 128]")
    B, T, C = qkv.shape
    if chunk not in (16, 32, 64):
        raise KdaError("kda_chunk_prefill_fused", KDA_ERR_UNSUPPORTED)
    Bg, t_pad, H = _vec_shapes(gate)
    if Bg != B or C != 3 * H * HEAD_DIM or t_pad != -(-int(T) // chunk) * chunk:
        raise ValueError("qkv [B][T][3 H 128] and gate [B][T_pad][H][128] do not agree")
    if conv_w.dim() != 2:
        raise ValueError("conv_w must be [conv_dim][conv_kernel]")
    K = conv_w.shape[1]
    vs = (B, t_pad, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=qkv.device)
    need = kda_chunk_prefill_workspace_bytes(B, H, int(T), chunk)
    if workspace is None:
        workspace = _workspace(need, qkv.device, stream)
    if not (workspace.device.type == "cuda" and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    args = [_check("qkv", qkv, (B, T, C), torch.bfloat16), _check("conv_w", conv_w, (C, K), torch.bfloat16),
            _check("conv_state", conv_state, (B, C, K)), _check("gate", gate, vs), _check("beta", beta, (B, t_pad, H)),
            _check("state", state, (B, H, HEAD_DIM, HEAD_DIM)), _check("out", out, vs)]
    rc = load_library().kda_chunk_prefill_fused(*args, B, H, int(T), chunk, K, float(l2_eps), workspace.data_ptr(),
                                                ws_bytes, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_chunk_prefill_fused", rc)
    return out


def kda_chunk_prefill_fused_gated(qkv, conv_w, conv_state, g_raw, beta_logit, dt_bias, a_log,
                                  gate_lower_bound: float, state, chunk: int, l2_eps: float, out=None, workspace=None,
                                  stream=None):
    """kda_chunk_prefill_fused with the gate and beta formed in the prepare from g_raw ([B][T_pad][H][128]
    bfloat16) and beta_logit ([B][T_pad][H]) as kda_chunk_prefill_gated forms them.  Returns ``out``."""
    if not isinstance(qkv, torch.Tensor) or qkv.dim() != 3:
        raise ValueError("qkv must be [batch][T][3 * heads * 128]")
    B, T, C = qkv.shape
    if chunk not in (16, 32, 64):
        raise KdaError("kda_chunk_prefill_fused_gated", KDA_ERR_UNSUPPORTED)
    if not isinstance(g_raw, torch.Tensor) or g_raw.dim() != 4:
        raise ValueError("g_raw must be [B][T_pad][H][128]")
    Bg, t_pad, H = g_raw.shape[0], g_raw.shape[1], g_raw.shape[2]
    if Bg != B or C != 3 * H * HEAD_DIM or t_pad != -(-int(T) // chunk) * chunk:
        raise ValueError("qkv [B][T][3 H 128] and g_raw [B][T_pad][H][128] do not agree")
    if conv_w.dim() != 2:
        raise ValueError("conv_w must be [conv_dim][conv_kernel]")
    K = conv_w.shape[1]
    vs = (B, t_pad, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=qkv.device)
    need = kda_chunk_prefill_workspace_bytes(B, H, int(T), chunk)
    if workspace is None:
        workspace = _workspace(need, qkv.device, stream)
    if not (workspace.device.type == "cuda" and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    g, b, dt, al = _gate_args(g_raw, beta_logit, dt_bias, a_log, B, t_pad, H)
    rc = load_library().kda_chunk_prefill_fused_gated(
        _check("qkv", qkv, (B, T, C), torch.bfloat16), _check("conv_w", conv_w, (C, K), torch.bfloat16),
        _check("conv_state", conv_state, (B, C, K)), g, b, dt, al, float(gate_lower_bound),
        _check("state", state, (B, H, HEAD_DIM, HEAD_DIM)), _check("out", out, vs), B, H, int(T), chunk, K,
        float(l2_eps), workspace.data_ptr(), ws_bytes, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_chunk_prefill_fused_gated", rc)
    return out


def kda_chunk_prefill_varlen_fused(qkv, conv_w, conv_state, gate, beta, state, cu_seqlens, chunk: int, l2_eps: float,
                                   out=None, workspace=None, stream=None):
    """kda_prefill_front_end_varlen + kda_chunk_prefill_varlen with the front end fused into the prefill.
    Returns ``out``.

    qkv: bfloat16 [total][3 H 128]; conv_w: bfloat16 [3 H 128][4]; conv_state: float32 [n][3 H 128][4] (in
    place); gate: [total][H][128]; beta: [total][H]; state: [n][H][128][128] (in place); cu_seqlens: int32
    CUDA tensor [n + 1]; out: [total][H][128].
    """
    if not isinstance(qkv, torch.Tensor) or qkv.dim() != 2:
        raise ValueError("qkv must be [total_tokens][3 * heads * 128]")
    total, C = qkv.shape
    if chunk not in (16, 32, 64):
        raise KdaError("kda_chunk_prefill_varlen_fused", KDA_ERR_UNSUPPORTED)
    if not isinstance(gate, torch.Tensor) or gate.dim() != 3 or gate.shape[0] != total:
        raise ValueError("gate must be [total_tokens][heads][128]")
    H = gate.shape[1]
    if C != 3 * H * HEAD_DIM:
        raise ValueError(f"qkv has {C} channels, expected 3 * {H} * {HEAD_DIM}")
    if not (isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.dtype == torch.int32 and cu_seqlens.dim() == 1
            and cu_seqlens.is_cuda and cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous int32 CUDA tensor [n + 1]")
    n = cu_seqlens.shape[0] - 1
    K = conv_w.shape[1] if conv_w.dim() == 2 else 0
    vs = (total, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=qkv.device)
    need = kda_chunk_prefill_varlen_workspace_bytes(n, H, total, chunk)
    if workspace is None:
        workspace = _workspace(need, qkv.device, stream)
    if not (workspace.device.type == "cuda" and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    args = [_check("qkv", qkv, (total, C), torch.bfloat16), _check("conv_w", conv_w, (C, K), torch.bfloat16),
            _check("conv_state", conv_state, (n, C, K)), _check("gate", gate, vs), _check("beta", beta, (total, H)),
            _check("state", state, (n, H, HEAD_DIM, HEAD_DIM)), _check("out", out, vs), cu_seqlens.data_ptr()]
    rc = load_library().kda_chunk_prefill_varlen_fused(*args, n, H, total, chunk, K, float(l2_eps),
                                                       workspace.data_ptr(), ws_bytes, _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_chunk_prefill_varlen_fused", rc)
    return out


def kda_prefill_front_end_varlen(qkv, conv_w, conv_state, cu_seqlens, heads: int, l2_eps: float, q=None, k=None,
                                 v=None, stream=None):
    """kda_prefill_front_end over packed sequences.  Returns (q, k, v), each float32 [total][H][128].

    qkv: bfloat16 [total][3 H 128]; conv_state: float32 [n][3 H 128][K] (one per sequence, advanced in place);
    cu_seqlens: int32 CUDA tensor [n + 1] of token offsets.
    """
    if not isinstance(qkv, torch.Tensor) or qkv.dim() != 2:
        raise ValueError("qkv must be [total_tokens][3 * heads * 128]")
    total, C = qkv.shape
    if C != 3 * heads * HEAD_DIM:
        raise ValueError(f"qkv has {C} channels, expected 3 * {heads} * {HEAD_DIM}")
    if not (isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 2):
        raise ValueError("cu_seqlens must be a 1-d tensor of n_seqs + 1 offsets")
    n = cu_seqlens.numel() - 1
    if conv_w.dim() != 2:
        raise ValueError("conv_w must be [conv_dim][conv_kernel]")
    K = conv_w.shape[1]
    vs = (total, heads, HEAD_DIM)
    q = torch.empty(vs, dtype=torch.float32, device=qkv.device) if q is None else q
    k = torch.empty(vs, dtype=torch.float32, device=qkv.device) if k is None else k
    v = torch.empty(vs, dtype=torch.float32, device=qkv.device) if v is None else v
    args = [_check("qkv", qkv, (total, C), torch.bfloat16), _check("conv_w", conv_w, (C, K), torch.bfloat16),
            _check("conv_state", conv_state, (n, C, K)), _check("q", q, vs), _check("k", k, vs), _check("v", v, vs),
            _check("cu_seqlens", cu_seqlens, (n + 1,), torch.int32)]
    rc = load_library().kda_prefill_front_end_varlen(*args, n, heads, total, K, float(l2_eps), _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_prefill_front_end_varlen", rc)
    return q, k, v


def kda_chunk_prefill_varlen_workspace_bytes(n_seqs: int, heads: int, total_tokens: int, chunk: int) -> int:
    return int(load_library().kda_chunk_prefill_varlen_workspace_bytes(n_seqs, heads, total_tokens, chunk))


def kda_chunk_prefill_varlen_bf16(qkv, gate, beta, state, cu_seqlens, chunk: int, out=None, workspace=None,
                                  stream=None):
    """kda_chunk_prefill_varlen with BF16 q | k | v packed per token.  Returns ``out``.

    qkv: bfloat16 [total][3 H 128] (or [total][3][H][128]); gate, out: [total][H][128]; the rest as
    kda_chunk_prefill_varlen.
    """
    if not isinstance(gate, torch.Tensor) or gate.dim() != 3 or gate.shape[-1] != HEAD_DIM:
        raise ValueError(f"gate must be [total_tokens][heads][{HEAD_DIM}]")
    total, H, _ = gate.shape
    if not isinstance(qkv, torch.Tensor) or qkv.dim() not in (2, 4):
        raise ValueError("qkv must be [total][3 * heads * 128] or [total][3][heads][128]")
    qshape = (total, 3 * H * HEAD_DIM) if qkv.dim() == 2 else (total, 3, H, HEAD_DIM)
    if not (isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 2):
        raise ValueError("cu_seqlens must be a 1-d tensor of n_seqs + 1 offsets")
    n = cu_seqlens.numel() - 1
    vs = (total, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=gate.device)
    need = kda_chunk_prefill_varlen_workspace_bytes(n, H, total, chunk)
    if workspace is None:
        workspace = _workspace(need, gate.device, stream)
    if not (workspace.device.type == "cuda" and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    args = [_check("qkv", qkv, qshape, torch.bfloat16), _check("gate", gate, vs), _check("beta", beta, (total, H)),
            _check("state", state, (n, H, HEAD_DIM, HEAD_DIM)), _check("out", out, vs),
            _check("cu_seqlens", cu_seqlens, (n + 1,), torch.int32)]
    rc = load_library().kda_chunk_prefill_varlen_bf16(*args, n, H, total, chunk, workspace.data_ptr(),
                                                      workspace.numel() * workspace.element_size(),
                                                      _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_chunk_prefill_varlen_bf16", rc)
    return out


def kda_chunk_prefill_varlen(q, k, v, gate, beta, state, cu_seqlens, chunk: int, out=None, workspace=None,
                             stream=None):
    """Chunked prefill of packed sequences of their own lengths.  Returns ``out``.

    q, k, v, gate, out: [total][H][128]; beta: [total][H]; state: [n_seqs][H][128][128] (in place);
    cu_seqlens: int32 CUDA tensor [n_seqs + 1] of token offsets.
    """
    if not isinstance(q, torch.Tensor) or q.dim() != 3 or q.shape[-1] != HEAD_DIM:
        raise ValueError(f"q must be [total_tokens][heads][{HEAD_DIM}]")
    total, H, _ = q.shape
    if not (isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.dim() == 1 and cu_seqlens.numel() >= 2):
        raise ValueError("cu_seqlens must be a 1-d tensor of n_seqs + 1 offsets")
    n = cu_seqlens.numel() - 1
    vs = (total, H, HEAD_DIM)
    if out is None:
        out = torch.empty(vs, dtype=torch.float32, device=q.device)
    need = kda_chunk_prefill_varlen_workspace_bytes(n, H, total, chunk)
    if workspace is None:
        workspace = _workspace(need, q.device, stream)
    if not (workspace.device.type == "cuda" and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    args = [_check(nm, t, vs) for nm, t in (("q", q), ("k", k), ("v", v), ("gate", gate))]
    args.append(_check("beta", beta, (total, H)))
    args.append(_check("state", state, (n, H, HEAD_DIM, HEAD_DIM)))
    args.append(_check("out", out, vs))
    args.append(_check("cu_seqlens", cu_seqlens, (n + 1,), torch.int32))
    rc = load_library().kda_chunk_prefill_varlen(*args, n, H, total, chunk, workspace.data_ptr(),
                                                 workspace.numel() * workspace.element_size(), _stream_ptr(stream))
    if rc != KDA_OK:
        raise KdaError("kda_chunk_prefill_varlen", rc)
    return out

