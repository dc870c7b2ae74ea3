"""Seeded synthetic inputs for the KDA gated delta-rule core.

This module only draws random numbers and lays them out; it holds none of the
recurrence's arithmetic.  Both the HIP path (through its tests and the bench)
and the fp64 oracle are fed from here, so the two always see the same bytes.

Recipe (one per workload, all values fp32 in the end):

* q, k : standard normal draws, then scaled to unit L2 norm over the
  head dimension as x / sqrt(sum x^2 + eps), eps = 1e-6 (the L2 form the
  config page gives for the block's front end, field ``l2_eps``), in fp64.
* v    : standard normal.
* gate : uniform on [lo, 0] (a per-channel log-decay; lo = -5 or -0.5).
* beta : sigmoid of a standard normal draw (the core receives beta already
  passed through a sigmoid, workspace page, field ``beta``).
* state: 0.02 * standard normal, or zeros.

Inputs of the gated RMSNorm that follows the core (norm_inputs):

* core     : standard normal, fp32, [rows][heads][D].
* out_gate : standard normal, rounded to BF16 (round to nearest even) and
  kept as 16-bit patterns (a projection output of unit scale).
* o_norm   : 1 + 0.1 * standard normal, BF16 patterns, [D] (a norm weight
  near one).

Packed variable-length batches (varlen_lengths, varlen_inputs): sequence
lengths drawn log-normally (so short and long sequences mix) and cut so they
sum to the total; the token rows are one make_batch stream cut at the
lengths, and each sequence has its own initial state.

Inputs of the decode front end (front_end_inputs), conv_dim = 3 * heads * D:

* qkv        : standard normal rounded to BF16, [B][T][conv_dim] (q | k | v).
* conv_w     : 0.5 * standard normal rounded to BF16, [conv_dim][K].
* conv_state : standard normal rounded to BF16 values, stored FP32,
  [B][conv_dim][K] (the window of past inputs it holds in use).

Every array is a pure function of (workload seed, array id, sequence, row
block): rows are drawn in blocks of ``ROW_BLOCK`` tokens from
``SeedSequence([seed, array_id, b, block])``, so a sequence can be generated
slab by slab, in parallel, and rows T..T+n of a longer draw continue a
shorter one exactly.

Memory layouts (token-major, heads inside):
  q, k, v, gate, out : [B][rows][H][D]
  beta               : [B][rows][H]
  state              : [B][H][D (key)][D (value)]
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

D = 128
ROW_BLOCK = 256
L2_EPS = 1e-6

# array ids inside a workload's seed space
ID_STATE, ID_Q, ID_K, ID_V, ID_GATE, ID_BETA = 0, 1, 2, 3, 4, 5
ID_CORE, ID_OUT_GATE, ID_O_NORM = 6, 7, 8
ID_QKV, ID_CONV_W, ID_CONV_STATE = 9, 10, 11
ID_G_RAW, ID_BETA_LOGIT, ID_DT_BIAS, ID_A_LOG = 12, 13, 14, 15
# gate_lower_bound of the gated workloads (the pages name the key, not its value): -5, the lower end of
# the workloads' gate range
GATE_LOWER_BOUND = -5.0
# (batch, rows, heads, conv_kernel, seed) of the decode front-end workloads: one decode step of the
# B=64 H=32 workload, and the k=4 rows of the B=128 decode_k workload
FRONT_END_WORKLOADS = {
    "front_end_b64_h32_k4": (64, 1, 32, 4, 1008),
    "front_end_b128_h32_k4_rows4": (128, 4, 32, 4, 1009),
}
# (batch, tokens, heads, conv_kernel, chunk, seed) of the prefill front-end workloads: the front end of
# the T=8192 H=32 C=64 prefill
PREFILL_FRONT_END_WORKLOADS = {
    "prefill_front_end_t8192_h32_k4": (1, 8192, 32, 4, 64, 1011),
}
# varlen prefill workloads: (total tokens, heads, chunk, mean sequence length, seed)
VARLEN_WORKLOADS = {
    "prefill_varlen_h32_t32768_c64": (32768, 32, 64, 2048, 1010),
}
# rms_norm_eps of the gated RMSNorm workloads (the pages name the config key, not its value)
NORM_EPS = 1e-6
# (rows, heads, seed) of the gated RMSNorm workloads: the output of the T=8192 prefill and of one
# B=64 decode step, both H=32
NORM_WORKLOADS = {
    "gated_rmsnorm_t8192_h32": (8192, 32, 1006),
    "gated_rmsnorm_b64_h32": (64, 32, 1007),
}


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: sizes, value distributions and seed."""

    name: str
    mode: str          # "prefill", "decode" or "decode_k"
    batch: int
    heads: int
    T: int             # tokens per sequence (rows walked, k for decode_k)
    chunk: int         # prefill chunk width (0 for the recurrent forms)
    gate_lo: float
    state_std: float   # 0.0 = zero initial state
    seed: int
    n_snap: int = 0
    pad_value: float | None = None   # fill of rows >= T (prefill only)
    pad_extra_rows: int = 0          # rows allocated beyond T_pad
    tail_steps: int = 0              # decode steps after the prefill


WORKLOADS = {
    # prefill, 1 sequence, H=2, T=64, C=16, zero state
    "prefill_h2_t64_c16": Workload("prefill_h2_t64_c16", "prefill", 1, 2, 64, 16, -5.0, 0.0, 1001),
    # single-token decode, B=64, H=32, 128 MiB state updated in place
    "decode_b64_h32": Workload("decode_b64_h32", "decode", 64, 32, 1, 0, -5.0, 0.02, 1002),
    # chunked prefill, T=8192, H=32, C=64, pad filled with 1e4 plus one extra chunk
    "prefill_h32_t8192_c64": Workload("prefill_h32_t8192_c64", "prefill", 1, 32, 8192, 64, -5.0, 0.02, 1003,
                                      pad_value=1e4, pad_extra_rows=64),
    # decode_k speculative verify, k=4 rows, B=128, H=32, 4 snapshots
    "decode_k4_b128_h32": Workload("decode_k4_b128_h32", "decode_k", 128, 32, 4, 0, -5.0, 0.02, 1004, n_snap=4),
    # long-context prefill 4 x 32768, slow decay, then 16 decode steps
    "prefill_b4_h32_t32768_c64": Workload("prefill_b4_h32_t32768_c64", "prefill", 4, 32, 32768, 64, -0.5, 0.02,
                                          1005, tail_steps=16),
}


def _rng(seed: int, array_id: int, b: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, array_id, b, block])))


def _block(seed: int, array_id: int, b: int, blk: int, n_prefix: int, width: int, kind: str) -> np.ndarray:
    """The first n_prefix rows of row block ``blk`` of one array, shape [n_prefix, width], fp32."""
    g = _rng(seed, array_id, b, blk)
    if kind == "normal":
        return g.standard_normal((n_prefix, width), dtype=np.float32)
    return g.random((n_prefix, width), dtype=np.float32)


def fill_rows(seed: int, b: int, r0: int, r1: int, heads: int, gate_lo: float, dst: dict) -> None:
    """Write rows [r0, r1) of sequence b into dst["q"|"k"|"v"|"gate"] ([r1-r0, H, D] views)
    and dst["beta"] ([r1-r0, H]), one row block at a time."""
    width = heads * D
    for blk in range(r0 // ROW_BLOCK, (r1 - 1) // ROW_BLOCK + 1):
        lo = max(r0, blk * ROW_BLOCK)
        hi = min(r1, (blk + 1) * ROW_BLOCK)
        n_prefix = hi - blk * ROW_BLOCK
        cut = slice(lo - blk * ROW_BLOCK, n_prefix)
        rows = slice(lo - r0, hi - r0)
        n = hi - lo
        for name, aid in (("q", ID_Q), ("k", ID_K)):
            x = _block(seed, aid, b, blk, n_prefix, width, "normal")[cut].astype(np.float64).reshape(n, heads, D)
            x /= np.sqrt((x * x).sum(-1, keepdims=True) + L2_EPS)
            dst[name][rows] = x
        dst["v"][rows] = _block(seed, ID_V, b, blk, n_prefix, width, "normal")[cut].reshape(n, heads, D)
        u = _block(seed, ID_GATE, b, blk, n_prefix, width, "uniform")[cut].astype(np.float64)
        dst["gate"][rows] = (gate_lo * u).reshape(n, heads, D)
        z = _block(seed, ID_BETA, b, blk, n_prefix, heads, "normal")[cut].astype(np.float64)
        dst["beta"][rows] = 1.0 / (1.0 + np.exp(-z))


def sequence_rows(seed: int, b: int, r0: int, r1: int, heads: int, gate_lo: float) -> dict:
    """q, k, v, gate [rows, H, D] and beta [rows, H] (fp32) for rows [r0, r1) of sequence b."""
    n = r1 - r0
    out = {name: np.empty((n, heads, D), dtype=np.float32) for name in ("q", "k", "v", "gate")}
    out["beta"] = np.empty((n, heads), dtype=np.float32)
    fill_rows(seed, b, r0, r1, heads, gate_lo, out)
    return out


def initial_state(seed: int, b: int, heads: int, std: float) -> np.ndarray:
    """[H, D, D] fp32 initial state of sequence b (zeros when std == 0)."""
    if std == 0.0:
        return np.zeros((heads, D, D), dtype=np.float32)
    g = _rng(seed, ID_STATE, b, 0)
    return (std * g.standard_normal((heads, D, D), dtype=np.float32)).astype(np.float32)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_batch(seed: int, batch: int, heads: int, rows: int, gate_lo: float, state_std: float,
               alloc_rows: int | None = None, pad_value: float | None = None, row0: int = 0,
               threads: int | None = None) -> dict:
    """A whole batch of inputs.

    ``rows`` token rows [row0, row0+rows) of each sequence are drawn; the arrays are
    allocated with ``alloc_rows`` >= rows rows per sequence, the rows past ``rows``
    filled with ``pad_value`` (NaN-free zeros when None).
    """
    alloc_rows = rows if alloc_rows is None else alloc_rows
    assert alloc_rows >= rows
    fill = 0.0 if pad_value is None else pad_value
    arrays = {
        name: np.full((batch, alloc_rows, heads, D), fill, dtype=np.float32) for name in ("q", "k", "v", "gate")
    }
    arrays["beta"] = np.full((batch, alloc_rows, heads), fill, dtype=np.float32)
    state = np.empty((batch, heads, D, D), dtype=np.float32)

    jobs = []
    for b in range(batch):
        for s in range(0, rows, ROW_BLOCK):
            jobs.append((b, s, min(rows, s + ROW_BLOCK)))

    def work(job):
        b, s, e = job
        fill_rows(seed, b, row0 + s, row0 + e, heads, gate_lo, {name: a[b, s:e] for name, a in arrays.items()})

    def work_state(b):
        state[b] = initial_state(seed, b, heads, state_std)

    with ThreadPoolExecutor(threads or default_threads()) as ex:
        list(ex.map(work, jobs))
        list(ex.map(work_state, range(batch)))
    arrays["state"] = state
    return arrays


def workload_inputs(w: Workload, batch: int | None = None, heads: int | None = None, T: int | None = None,
                    threads: int | None = None) -> dict:
    """Inputs of a workload, optionally at a reduced batch / heads / T (same seeds).

    Prefill inputs are allocated with T_pad = ceil(T/chunk)*chunk rows plus
    ``pad_extra_rows``; rows >= T hold ``pad_value``.
    """
    B = w.batch if batch is None else batch
    H = w.heads if heads is None else heads
    T_ = w.T if T is None else T
    if w.mode == "prefill":
        t_pad = -(-T_ // w.chunk) * w.chunk
        alloc = t_pad + w.pad_extra_rows
    else:
        alloc = T_
    return make_batch(w.seed, B, H, T_, w.gate_lo, w.state_std, alloc_rows=alloc, pad_value=w.pad_value,
                      threads=threads)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Finite fp32 values to BF16 bit patterns (uint16), rounding to nearest even."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32).astype(np.uint64)  # keeps the shape
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def norm_inputs(seed: int, rows: int, heads: int) -> dict:
    """core [rows][heads][D] fp32, out_gate [rows][heads][D] and o_norm [D] as BF16 bit patterns."""
    core = _rng(seed, ID_CORE, 0, 0).standard_normal((rows, heads, D), dtype=np.float32)
    g = _rng(seed, ID_OUT_GATE, 0, 0).standard_normal((rows, heads, D), dtype=np.float32)
    w = 1.0 + 0.1 * _rng(seed, ID_O_NORM, 0, 0).standard_normal(D, dtype=np.float32)
    return {"core": core, "out_gate": to_bf16_bits(g), "o_norm": to_bf16_bits(w.astype(np.float32))}


def front_end_inputs(seed: int, batch: int, rows: int, heads: int, conv_kernel: int) -> dict:
    """qkv [B][rows][3 H D] and conv_w [3 H D][K] as BF16 patterns, conv_state [B][3 H D][K] fp32."""
    C = 3 * heads * D
    qkv = np.empty((batch, rows, C), dtype=np.uint16)
    st = np.empty((batch, C, conv_kernel), dtype=np.float32)
    for b in range(batch):
        qkv[b] = to_bf16_bits(_rng(seed, ID_QKV, b, 0).standard_normal((rows, C), dtype=np.float32))
        s = to_bf16_bits(_rng(seed, ID_CONV_STATE, b, 0).standard_normal((C, conv_kernel), dtype=np.float32))
        st[b] = (s.astype(np.uint32) << 16).view(np.float32)
    w = 0.5 * _rng(seed, ID_CONV_W, 0, 0).standard_normal((C, conv_kernel), dtype=np.float32)
    return {"qkv": qkv, "conv_w": to_bf16_bits(w.astype(np.float32)), "conv_state": st}


def gate_inputs(seed: int, batch: int, rows: int, heads: int) -> dict:
    """Inputs of the gate and beta steps that precede the core: g_raw [B][rows][H][D] standard normal
    rounded to BF16 patterns (a projection output of unit scale), beta_logit [B][rows][H] standard
    normal (so beta = sigmoid of it has the distribution of the other workloads' beta), dt_bias [H][D]
    0.5 * standard normal, a_log [H] 0.5 * standard normal (rates exp(a_log) around 1).  With the
    lower bound -5 the gates then spread over (-5, 0) like the other workloads' U[-5, 0]."""
    g = np.empty((batch, rows, heads, D), dtype=np.uint16)
    bl = np.empty((batch, rows, heads), dtype=np.float32)
    for b in range(batch):
        g[b] = to_bf16_bits(_rng(seed, ID_G_RAW, b, 0).standard_normal((rows, heads, D), dtype=np.float32))
        bl[b] = _rng(seed, ID_BETA_LOGIT, b, 0).standard_normal((rows, heads), dtype=np.float32)
    dt = (0.5 * _rng(seed, ID_DT_BIAS, 0, 0).standard_normal((heads, D))).astype(np.float32)
    al = (0.5 * _rng(seed, ID_A_LOG, 0, 0).standard_normal(heads)).astype(np.float32)
    return {"g_raw": g, "beta_logit": bl, "dt_bias": dt, "a_log": al}


def varlen_lengths(seed: int, total: int, mean_len: int) -> list:
    """Sequence lengths (each >= 1) summing to total: log-normal draws around mean_len."""
    g = _rng(seed, 12, 0, 0)
    lens, acc = [], 0
    while acc < total:
        n = max(1, int(round(mean_len * float(np.exp(g.normal(-0.5, 1.0))))))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return lens


def varlen_inputs(seed: int, lengths: list, heads: int, gate_lo: float, state_std: float,
                  pad_tokens: int = 0, threads: int | None = None) -> dict:
    """Packed [total][H][D] inputs (beta [total][H]) of sequences of the given lengths, with
    cu_seqlens (int32 [n + 1]) and per-sequence states [n][H][D][D].  The token rows are one
    stream (sequence 0 of make_batch over all rows, cut at the lengths); state s is the state of
    sequence s of make_batch's recipe.  pad_tokens rows of zeros after the last sequence belong
    to none."""
    used = int(sum(lengths))
    x = make_batch(seed, 1, heads, max(used, 1), gate_lo, 0.0, alloc_rows=max(used, 1) + pad_tokens,
                   threads=threads)
    out = {name: np.ascontiguousarray(x[name][0, :used + pad_tokens]) for name in ("q", "k", "v", "gate", "beta")}
    out["state"] = np.stack([initial_state(seed, s, heads, state_std) for s in range(len(lengths))])
    out["cu_seqlens"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return out
