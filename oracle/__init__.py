"""fp64 CPU oracle of the KDA gated delta-rule core (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this package.  It wraps ``kda_oracle.c`` through ctypes and
takes / returns numpy arrays; see that file's header for the exact recurrence,
the chunked form and every layout.

``gated_rmsnorm`` (the sigmoid-gated RMSNorm that follows the core) is plain
numpy in fp64.

Parity status: pinned.  tests/test_oracle_pins.py checks it against closed
forms, exact rational brute force on tiny inputs and invariants of the method
(state untouched at beta=0/gate=0, the delta-rule fixed point S^T k = v at
beta=1, per-row exponential averages for basis keys, decay-before-update order
on a scalar head, chunked == serial, pad independence, linearity, column
equivariance, continuation).  gated_rmsnorm is pinned against torch's own
rms_norm and sigmoid in fp64, closed forms (one-hot rows, gate 0 and +-inf),
scale invariance and unit mean square (tests/test_oracle_norm_pins.py).
``transition`` (the prefill's final state as an affine map P S + Q of its initial state) is pinned
against the state the recurrence reaches from random initial states, the explicit product of the
per-row factors, the matrix determinant lemma, composition of segments and the beta = 0 closed form
(tests/test_oracle_transition_pins.py).
``sigmoid`` is pinned against torch.sigmoid in fp64 and closed forms; ``kda_gate`` (a reading of a
step whose formula the pages do not print: parity unpinned against the pages) is pinned against
closed forms of that reading, its bounds and the per-head / per-channel broadcast of its parameters
(tests/test_oracle_gate_pins.py).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


def _load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        lib = ctypes.CDLL(path)
        i = ctypes.c_int
        lib.kda_oracle_serial.argtypes = [_f32p] * 5 + [_f64p, _f64p, ctypes.c_void_p] + [i] * 7
        lib.kda_oracle_serial.restype = i
        lib.kda_oracle_chunked.argtypes = [_f32p] * 5 + [_f64p, _f64p] + [i] * 7
        lib.kda_oracle_chunked.restype = i
        lib.kda_oracle_chunk_stages.argtypes = [_f32p] * 5 + [i] * 8 + [_f64p, _f64p] + [ctypes.c_void_p] * 7
        lib.kda_oracle_chunk_stages.restype = i
        lib.kda_oracle_threads.argtypes = [i]
        lib.kda_oracle_threads.restype = i
        _lib = lib
    return _lib


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _shape(q, beta):
    if q.ndim != 4:
        raise ValueError("q/k/v/gate must be [B][rows][H][D]")
    B, rows, H, D = q.shape
    if beta.shape != (B, rows, H):
        raise ValueError("beta must be [B][rows][H]")
    return B, rows, H, D


def threads(requested: int = 0) -> int:
    return _load().kda_oracle_threads(requested)


def serial(q, k, v, gate, beta, state, T: int | None = None, n_snap: int = 0, nthreads: int = 0):
    """Token-by-token fp64 recurrence.

    Returns (out [B][T][H][D], state [B][H][D][D], snaps [n_snap][B][H][D][D] or None,
    threads used), all fp64.  ``state`` may be float32 or float64; it is not modified.
    """
    q, k, v, gate, beta = map(_f32, (q, k, v, gate, beta))
    B, rows, H, D = _shape(q, beta)
    T = rows if T is None else T
    st = np.array(state, dtype=np.float64, order="C", copy=True)
    if st.shape != (B, H, D, D):
        raise ValueError("state must be [B][H][D][D]")
    out = np.zeros((B, T, H, D), dtype=np.float64)
    snaps = np.zeros((n_snap, B, H, D, D), dtype=np.float64) if n_snap > 0 else None
    sp = snaps.ctypes.data if snaps is not None else None
    rc = _load().kda_oracle_serial(q, k, v, gate, beta, st, out, sp, n_snap, B, H, D, T, rows, nthreads)
    if rc < 1:
        raise ValueError("kda_oracle_serial rejected its arguments")
    return out, st, snaps, rc


def chunked(q, k, v, gate, beta, state, chunk: int, T: int | None = None, nthreads: int = 0):
    """Chunked (WY/UT) fp64 form; returns (out, state, threads used)."""
    q, k, v, gate, beta = map(_f32, (q, k, v, gate, beta))
    B, rows, H, D = _shape(q, beta)
    T = rows if T is None else T
    st = np.array(state, dtype=np.float64, order="C", copy=True)
    out = np.zeros((B, T, H, D), dtype=np.float64)
    rc = _load().kda_oracle_chunked(q, k, v, gate, beta, st, out, B, H, D, T, rows, chunk, nthreads)
    if rc < 1:
        raise ValueError("kda_oracle_chunked rejected its arguments")
    return out, st, rc


def chunk_stages(q, k, v, gate, beta, S0, b: int, h: int, t0: int, n: int) -> dict:
    """Intermediates of one chunk (rows [t0, t0+n) of (b, h)) from incoming state S0 [D][D]."""
    q, k, v, gate, beta = map(_f32, (q, k, v, gate, beta))
    B, rows, H, D = _shape(q, beta)
    S = np.array(S0, dtype=np.float64, order="C", copy=True)
    res = {
        "O": np.zeros((n, D)), "G": np.zeros((n, D)), "A": np.zeros((n, n)), "Tinv": np.zeros((n, n)),
        "W": np.zeros((n, D)), "U": np.zeros((n, D)), "M": np.zeros((n, n)), "Delta": np.zeros((n, D)),
    }
    rc = _load().kda_oracle_chunk_stages(
        q, k, v, gate, beta, B, H, D, rows, b, h, t0, n, S, res["O"], res["G"].ctypes.data,
        res["A"].ctypes.data, res["Tinv"].ctypes.data, res["W"].ctypes.data, res["U"].ctypes.data,
        res["M"].ctypes.data, res["Delta"].ctypes.data)
    if rc != 0:
        raise ValueError("kda_oracle_chunk_stages rejected its arguments")
    res["S"] = S
    return res


def transition(q, k, v, gate, beta, T: int | None = None, nthreads: int = 0):
    """The final state of a prefill as an affine function of its initial state (kernels page,
    chunk_scan: the state update of each chunk is linear in the incoming state plus a term from
    the chunk's values).  Returns (P [B][H][D][D], Q [B][H][D][D]), fp64, such that for every
    initial state S [D (key)][D (value)] the recurrence over the T rows ends in P @ S + Q.

    Each row maps S to diag(alpha) S + beta k (v - (diag(alpha) S)^T k)^T, which is the linear map
    (I - beta k k^T) diag(alpha) applied to S plus beta k v^T.  So P is the recurrence started
    from the identity with every v set to 0 (a key-by-key state, one column per key), and Q is the
    recurrence started from the zero state."""
    q, k, v, gate, beta = map(_f32, (q, k, v, gate, beta))
    B, rows, H, D = _shape(q, beta)
    eye = np.broadcast_to(np.eye(D), (B, H, D, D))
    _, P, _, _ = serial(q, k, np.zeros_like(v), gate, beta, eye, T=T, nthreads=nthreads)
    _, Q, _, _ = serial(q, k, v, gate, beta, np.zeros((B, H, D, D)), T=T, nthreads=nthreads)
    return P, Q


def apply_transition(P, Q, S) -> np.ndarray:
    """P @ S + Q per (sequence, head), fp64: the state a segment with transition (P, Q) ends in when
    it starts from S (Q None: P @ S).  With S = Q1 and (P, Q) = (P2, Q2) it composes two segments,
    and with S = P1 and Q None it gives the composed P2 P1."""
    out = np.matmul(np.asarray(P, dtype=np.float64), np.asarray(S, dtype=np.float64))
    return out if Q is None else out + np.asarray(Q, dtype=np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    """BF16 bit patterns to float64: a BF16 value is the upper 16 bits of an IEEE float32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def sigmoid(x) -> np.ndarray:
    """1 / (1 + e^-x) in fp64 (workspace page, field beta: the core takes beta already passed through a
    sigmoid; module page, pipeline line: beta = sigmoid(b_proj(h))).  Written as e^x / (1 + e^x) for
    negative x so that neither sign overflows; sigmoid(+inf) = 1, sigmoid(-inf) = 0, NaN stays NaN."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def kda_gate(g_raw_bits, dt_bias, a_log, lower_bound: float) -> np.ndarray:
    """The gate, fp64, from its inputs (workspace page, field gate: the bounded log-decay kda_gate
    produces; field g_raw: f_b(f_a(h)), [T, heads * head_dim] BF16, what kda_gate consumes; config
    page, Glm5NextKdaWeights::dt_bias [heads * head_dim] F32 and a_log [heads] F32, and
    Glm5NextKdaConfig::gate_lower_bound).  The pages print no formula; the reading taken is

        gate[b, t, h, i] = lower_bound * sigmoid(exp(a_log[h]) * (g_raw[b, t, h, i] + dt_bias[h, i]))

    a per-channel bias, a per-head positive rate exp(a_log) and a sigmoid that bounds the log-decay
    to (lower_bound, 0) for lower_bound < 0.  Parity unpinned against the pages (no printed formula
    or value); the pins check this reading.  g_raw_bits: BF16 patterns [B][T][H][D]; dt_bias
    [H][D] (or [H * D]); a_log [H]; lower_bound widened from float32 as the C ABI takes it."""
    g = bf16_to_f64(g_raw_bits)
    B, T, H, D = g.shape
    dt = np.asarray(dt_bias, dtype=np.float64).reshape(H, D)
    rate = np.exp(np.asarray(a_log, dtype=np.float64).reshape(H))
    lo = float(np.float32(lower_bound))
    return lo * sigmoid(rate[None, None, :, None] * (g + dt[None, None]))


def gated_rmsnorm(core, out_gate_bits, o_norm_bits, eps: float) -> np.ndarray:
    """Sigmoid-gated RMSNorm, fp64 (module page, pipeline line: RMSNorm with weight o_norm, gated by
    a sigmoid of g_b(g_a(h)); workspace page, fields out_gate and o_norm_out; config page,
    Glm5NextKdaWeights::o_norm [head_dim]; config page, rms_norm_eps).  For every vector x over the last axis of
    core: x / sqrt(mean(x^2) + eps) * w * sigmoid(g).  eps is widened from float32, the precision
    the C ABI takes it in."""
    x = np.asarray(core, dtype=np.float64)
    w = bf16_to_f64(o_norm_bits)
    g = bf16_to_f64(out_gate_bits)
    e = float(np.float32(eps))
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + e) * w * sig


def decode_front_end(qkv_bits, conv_w_bits, conv_state, heads: int, l2_eps: float, n_snap: int = 0):
    """The decode front end, fp64, token by token (module page, pipeline line: conv1d and SiLU on
    q, k, v, then L2 on q and k alone; the conv state holds conv_kernel slots that move one place
    toward the oldest before each convolution.  Workspace page, qkv_proj [T, conv_dim] BF16, one row of q, k and
    v channels a token; config page, Glm5NextKdaWeights::conv [conv_dim, conv_kernel] BF16 (depthwise, no bias),
    conv_state_elems [conv_dim, conv_kernel] FP32, l2_eps added to the sum of squares inside the square root).

    qkv_bits [B][T][3 H D] and conv_w_bits [3 H D][K] are BF16 patterns, conv_state [B][3 H D][K]
    (not modified).  Per token: the K slots shift left by one and the new input enters the last
    slot; y = sum_k w[k] * slot[k] (slot K-1 newest, the causal convolution); y = y * sigmoid(y);
    the q and k parts are scaled per head by 1 / sqrt(sum y^2 + eps).  Returns q, k, v
    [B][T][H][D], the final conv state [B][3 H D][K] and the states after rows 0..n_snap-1
    [n_snap][B][3 H D][K], all fp64."""
    x = bf16_to_f64(qkv_bits)
    w = bf16_to_f64(conv_w_bits)
    s = np.array(conv_state, dtype=np.float64, copy=True)
    B, T, C = x.shape
    D = C // (3 * heads)
    e = float(np.float32(l2_eps))
    outs = np.zeros((3, B, T, heads, D))
    snaps = np.zeros((n_snap, B, C, s.shape[-1]))
    for t in range(T):
        s[:, :, :-1] = s[:, :, 1:].copy()
        s[:, :, -1] = x[:, t]
        y = np.sum(s * w[None], axis=-1)
        with np.errstate(over="ignore"):
            y = y / (1.0 + np.exp(-y))
        y = y.reshape(B, 3, heads, D)
        for part in range(3):
            yp = y[:, part]
            if part < 2:
                yp = yp / np.sqrt(np.sum(yp * yp, axis=-1, keepdims=True) + e)
            outs[part, :, t] = yp
        if t < n_snap:
            snaps[t] = s
    return outs[0], outs[1], outs[2], s, snaps
