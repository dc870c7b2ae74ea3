#!/usr/bin/env python3
"""Throughput of the KDA gated delta-rule core on one MI355X.

Headline (the ``value`` of the JSON line): single-token decode of 64
sequences x 32 heads, FP32 128x128 key-major state per head updated in place
(kda_recurrent_step), in tokens/s.  One step = one call over the whole batch.
The same run also times the other workloads of the core and reports each
under ``workloads``:
  * decode: decode_k (k=4, 4 snapshots, B=128), the BF16 q | k | v forms, the gated form (gate and
    beta formed inside), the whole step from the raw projections in one kernel (kda_decode_fused_step,
    kda_decode_fused_k), and two chains replayed from one HIP graph (front end + core + gated RMSNorm
    as three kernels, and with the norm fused into the core);
  * prefill: T=8192 H=32 at chunk 64 / 32 / 16 (at 64 also split into the scan alone, kda_chunk_scan
    on the kept records, and the prepare as the rest of the call), 4 x 32768 followed by 16 decode
    steps, T=64 H=2, the gated form, BF16 q | k | v (kda_chunk_prefill_bf16), 23 packed sequences of
    mixed lengths (kda_chunk_prefill_varlen),
    the front end fused into the prepare (dense and packed), and the chain front end + prefill + norm;
  * the token-segment split's per-device pieces: the segment transition, the fold S <- P S + Q, and
    one device's share of the 4 x 32768 prefill cut into 8 segments (no exchange);
  * the front ends (decode and prefill, FP32 and BF16 outputs) and the gated RMSNorm on their own;
  * copy_ceiling: a plain 1 GiB device copy, the practical HBM ceiling beside the vendor's 8 TB/s.

Inputs are seeded synthetic tensors (kda_inputs) resident in HBM before the
timed region.  Decode states are rotated over buffers totalling >= 1 GiB so
the 256 MB Infinity Cache cannot hold them: every step reads and writes HBM.

``roofline`` describes the dominant kernel of the headline (the recurrent
kernel): algorithmic bytes per launch / average launch duration (one HIP event
pair on the launch stream around back-to-back launches), against 8 TB/s, with
the counter-measured traffic from the committed rocprofv3 summary while it
matches the kernel source, and the fraction of the plain copy's rate.
``cpu_baseline`` times the fp64 oracle on the host cores (rank 0, N=1) on the headline workload; the
same oracle is also timed beside the decode_k workload and the three prefill workloads (each
workload's ``cpu_oracle`` entry, with the threads it used and the sample it ran).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KDA core tokens/s + achieved HBM GB/s (decode) / MFMA % (prefill), 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense FP32 matrix, vendor figure
D = 128
STATE_BYTES = D * D * 4


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- algorithmic work
def decode_bytes(B: int, H: int, T: int = 1, n_snap: int = 0, qkv_bytes: int = 4) -> int:
    """State read + write (+ snapshot writes) + q, k, v reads (qkv_bytes per element: 4 FP32, 2 BF16)
    + gate read + out write + beta reads."""
    per_head = 2 * STATE_BYTES + n_snap * STATE_BYTES + T * (3 * D * qkv_bytes + D * 4 + D * 4 + 4)
    return B * H * per_head


def prefill_flops(B: int, H: int, T: int, C: int) -> float:
    """Per token-head: 6 d^2 (W S, Qhat S, Ktil^T Delta) + 5 C d (lower-triangular A, M, W, U,
    M Delta) + C^2 / 3 (triangular inverse)."""
    return float(B) * H * T * (6 * D * D + 5 * C * D + C * C / 3.0)


def transition_flops(B: int, H: int, T: int, C: int) -> float:
    """Per token-head of the segment transition: 4 d^2 for each of P and Q (W S, Ktil^T Delta) + 3 C d
    (lower-triangular A, W, U) + C^2 / 3 (triangular inverse).  The prepare also builds the output
    operands of the record, which the transition does not use; they are not counted."""
    return float(B) * H * T * (8 * D * D + 3 * C * D + C * C / 3.0)


def prefill_bytes(B: int, H: int, T: int) -> int:
    return B * H * (2 * STATE_BYTES + T * (4 * D * 4 + D * 4 + 4))


# ---------------------------------------------------------------- timing
class Timer:
    """K back-to-back launches between device synchronisations: wall clock for the step time,
    and one pair of HIP events on the launch stream around the K launches for the average
    launch duration (no event commands between launches, so the kernels run back to back).

    Before the W warm-up steps each workload runs untimed for at least PREWARM_S of wall time: after
    a switch of workload the device takes a few hundred milliseconds to settle (decode_k measured
    364 us per call after 5 warm-up calls, 299 us after 2000), and the timed steps are meant to see
    the steady state a serving loop runs in."""

    def __init__(self, torch, prewarm_s: float = 0.3):
        self.torch = torch
        self.PREWARM_S = prewarm_s

    def prewarm(self, fn):
        torch = self.torch
        t0, i = time.perf_counter(), 0
        while True:
            for _ in range(8):
                fn(i)
                i += 1
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= self.PREWARM_S or i >= 100000:
                return i

    def run(self, fn, steps: int, warmup: int):
        torch = self.torch
        if self.PREWARM_S > 0:
            self.prewarm(fn)
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            fn(warmup + i)
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return {
            "wall_s": wall,
            "s_per_step": wall / steps,
            "launch_avg_s": e0.elapsed_time(e1) * 1e-3 / steps,
        }


# ---------------------------------------------------------------- workloads
def _packed_bf16(torch, ki, x):
    """q, k, v of a workload rounded to BF16 and packed per token as [B][T][3][H][D] on the device."""
    import numpy as np
    bits = np.stack([ki.to_bf16_bits(x[n]) for n in ("q", "k", "v")], axis=2)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def bench_decode(torch, kda, ki, steps, warmup, timer, bf16=False):
    w = ki.WORKLOADS["decode_b64_h32"]
    B, H = w.batch, w.heads
    x = ki.workload_inputs(w)
    dev = lambda a: torch.from_numpy(a).cuda()
    q, k, v, g, b = (dev(x[n]) for n in ("q", "k", "v", "gate", "beta"))
    qkv = _packed_bf16(torch, ki, x) if bf16 else None
    n_buf = max(2, -(-(1 << 30) // (B * H * STATE_BYTES)))  # >= 1 GiB of states
    states = [dev(x["state"]) for _ in range(n_buf)]
    out = torch.empty((B, 1, H, D), device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        if bf16:
            kda.kda_recurrent_step_bf16(qkv, g, b, states[i % n_buf], out=out, stream=stream)
        else:
            kda.kda_recurrent_step(q, k, v, g, b, states[i % n_buf], out=out, stream=stream)

    r = timer.run(step, steps, warmup)
    nbytes = decode_bytes(B, H, qkv_bytes=2 if bf16 else 4)
    return w, r, nbytes, n_buf


def decode_bytes_gated(B: int, H: int, T: int = 1) -> int:
    """The gated decode step: state read + write, q, k, v read, g_raw read (BF16), out written, beta logit
    read, and dt_bias + a_log read once per call."""
    return B * H * (2 * STATE_BYTES + T * (3 * D * 4 + D * 2 + D * 4 + 4)) + H * (D * 4 + 4)


def bench_decode_gated(torch, kda, ki, steps, warmup, timer):
    """kda_recurrent_step_gated at B=64 H=32: the gate (kda_gate of BF16 g_raw) and beta (sigmoid of the
    logit) formed in the decode kernel; states rotated over >= 1 GiB as for the plain step."""
    import numpy as np
    w = ki.WORKLOADS["decode_b64_h32"]
    B, H = w.batch, w.heads
    x = ki.workload_inputs(w)
    gx = ki.gate_inputs(1013, B, 1, H)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v = (dev(x[n]) for n in ("q", "k", "v"))
    g = torch.from_numpy(gx["g_raw"].view(np.int16)).view(torch.bfloat16).cuda()
    bl, dt, al = dev(gx["beta_logit"]), dev(gx["dt_bias"]), dev(gx["a_log"])
    n_buf = max(2, -(-(1 << 30) // (B * H * STATE_BYTES)))
    states = [dev(x["state"]) for _ in range(n_buf)]
    out = torch.empty((B, 1, H, D), device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        kda.kda_recurrent_step_gated(q, k, v, g, bl, dt, al, ki.GATE_LOWER_BOUND, states[i % n_buf], out=out,
                                     stream=stream)

    r = timer.run(step, steps, warmup)
    return w, r, decode_bytes_gated(B, H)


def bench_prefill_gated(torch, kda, ki, steps, warmup, timer):
    """kda_chunk_prefill_gated at T=8192 H=32 C=64: the T=8192 prefill workload's q, k, v and state with
    the gate inputs of its shape (gate and beta formed in the prepare)."""
    import numpy as np
    w = ki.WORKLOADS["prefill_h32_t8192_c64"]
    B, H, T, C = w.batch, w.heads, w.T, w.chunk
    t_pad = -(-T // C) * C
    x = ki.workload_inputs(w)
    gx = ki.gate_inputs(1012, B, t_pad, H)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v = (dev(x[n][:, :t_pad]) for n in ("q", "k", "v"))
    g = torch.from_numpy(gx["g_raw"].view(np.int16)).view(torch.bfloat16).cuda()
    bl, dt, al = dev(gx["beta_logit"]), dev(gx["dt_bias"]), dev(gx["a_log"])
    st = dev(x["state"])
    out = torch.empty((B, t_pad, H, D), device="cuda")
    ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T, C), dtype=torch.uint8, device="cuda")

    def step(i):
        kda.kda_chunk_prefill_gated(q, k, v, g, bl, dt, al, ki.GATE_LOWER_BOUND, st, T, C, out=out, workspace=ws)

    return w, timer.run(step, steps, warmup)


def bench_prefill_bf16(torch, kda, ki, steps, warmup, timer):
    """kda_chunk_prefill_bf16 at T=8192 H=32 C=64: the T=8192 prefill workload with q, k, v rounded to BF16
    and packed per token."""
    import numpy as np
    w = ki.WORKLOADS["prefill_h32_t8192_c64"]
    B, H, T, C = w.batch, w.heads, w.T, w.chunk
    t_pad = -(-T // C) * C
    x = ki.workload_inputs(w)
    qkv = _packed_bf16(torch, ki, {n: np.ascontiguousarray(x[n][:, :t_pad]) for n in ("q", "k", "v")})
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    g, b, st = dev(x["gate"][:, :t_pad]), dev(x["beta"][:, :t_pad]), dev(x["state"])
    out = torch.empty((B, t_pad, H, D), device="cuda")
    ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T, C), dtype=torch.uint8, device="cuda")

    def step(i):
        kda.kda_chunk_prefill_bf16(qkv, g, b, st, T, C, out=out, workspace=ws)

    return w, timer.run(step, steps, warmup)


def bench_decode_k(torch, kda, ki, steps, warmup, timer, bf16=False):
    w = ki.WORKLOADS["decode_k4_b128_h32"]
    B, H, T = w.batch, w.heads, w.T
    x = ki.workload_inputs(w)
    dev = lambda a: torch.from_numpy(a).cuda()
    q, k, v, g, b = (dev(x[n]) for n in ("q", "k", "v", "gate", "beta"))
    qkv = _packed_bf16(torch, ki, x) if bf16 else None
    n_buf = max(2, -(-(1 << 30) // (B * H * STATE_BYTES)))
    states = [dev(x["state"]) for _ in range(n_buf)]
    snaps = torch.empty((w.n_snap, B, H, D, D), device="cuda")
    out = torch.empty((B, T, H, D), device="cuda")

    def step(i):
        if bf16:
            kda.kda_recurrent_k_bf16(qkv, g, b, states[i % n_buf], out=out, snapshots=snaps, n_snapshots=w.n_snap)
        else:
            kda.kda_recurrent_k(q, k, v, g, b, states[i % n_buf], out=out, snapshots=snaps, n_snapshots=w.n_snap)

    r = timer.run(step, steps, warmup)
    return w, r, decode_bytes(B, H, T, w.n_snap, qkv_bytes=2 if bf16 else 4)


def norm_bytes(rows: int, heads: int) -> int:
    """Algorithmic bytes of one gated RMSNorm call: FP32 core read, BF16 gate read, BF16 output
    written (512 + 256 + 256 per (token, head)) and the BF16 weight read once."""
    return rows * heads * (4 * D + 2 * D + 2 * D) + 2 * D


def bench_norm(torch, kda, ki, name, steps, warmup, timer):
    rows, heads, seed = ki.NORM_WORKLOADS[name]
    x = ki.norm_inputs(seed, rows, heads)
    bits = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).cuda()
    core0, gate0, w = torch.from_numpy(x["core"]).cuda(), bits(x["out_gate"]), bits(x["o_norm"])
    # buffer sets rotated over >= 1 GiB so the 256 MB Infinity Cache cannot serve them
    n_set = max(2, -(-(1 << 30) // (norm_bytes(rows, heads))))
    sets = [(core0.clone(), gate0.clone(), torch.empty_like(gate0)) for _ in range(n_set)]
    stream = torch.cuda.current_stream()

    def step(i):
        c, g, o = sets[i % n_set]
        kda.kda_gated_rmsnorm(c, g, w, ki.NORM_EPS, out=o, stream=stream)

    r = timer.run(step, steps, warmup)
    return r, norm_bytes(rows, heads), n_set


def front_end_bytes(B: int, T: int, H: int, K: int, n_snap: int, out_bytes: int = 4) -> int:
    """Algorithmic bytes of one decode front-end call: BF16 qkv read, q, k, v written (out_bytes per
    element: 4 FP32, 2 BF16), the FP32 conv state read and written, snapshots written, BF16 conv
    weights read once."""
    C = 3 * H * D
    return B * T * C * (2 + out_bytes) + B * C * K * 4 * (2 + n_snap) + C * K * 2


def bench_front_end(torch, kda, ki, name, steps, warmup, timer, bf16=False):
    B, T, H, K, seed = ki.FRONT_END_WORKLOADS[name]
    n_snap = T if T > 1 else 0
    x = ki.front_end_inputs(seed, B, T, H, K)
    bits = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).cuda()
    qkv0, w, st0 = bits(x["qkv"]), bits(x["conv_w"]), torch.from_numpy(x["conv_state"]).cuda()
    vs = (B, T, H, D)
    per_set = front_end_bytes(B, T, H, K, n_snap, 2 if bf16 else 4)
    n_set = max(2, -(-(1 << 30) // per_set))
    sets = []
    for _ in range(n_set):
        snaps = torch.empty((n_snap, B, 3 * H * D, K), device="cuda") if n_snap else None
        if bf16:
            outs = (torch.empty_like(qkv0), None, None)
        else:
            outs = tuple(torch.empty(vs, device="cuda") for _ in range(3))
        sets.append((qkv0.clone(), st0.clone(), *outs, snaps))
    stream = torch.cuda.current_stream()

    def step(i):
        qkv, st, q, k, v, snaps = sets[i % n_set]
        if bf16:
            kda.kda_decode_front_end_bf16(qkv, w, st, H, ki.L2_EPS, conv_out=q, conv_snapshots=snaps,
                                          n_snapshots=n_snap, stream=stream)
        else:
            kda.kda_decode_front_end(qkv, w, st, H, ki.L2_EPS, q=q, k=k, v=v, conv_snapshots=snaps,
                                     n_snapshots=n_snap, stream=stream)

    r = timer.run(step, steps, warmup)
    return r, per_set, n_set, B * T


def prefill_front_end_bytes(B: int, T: int, H: int, K: int) -> int:
    """Algorithmic bytes of one prefill front-end call: BF16 qkv read, FP32 q, k, v rows < T written, the
    FP32 conv state read and written, BF16 conv weights read once."""
    C = 3 * H * D
    return B * T * C * (2 + 4) + 2 * B * C * K * 4 + C * K * 2


def bench_prefill_front_end(torch, kda, ki, name, steps, warmup, timer):
    B, T, H, K, chunk, seed = ki.PREFILL_FRONT_END_WORKLOADS[name]
    x = ki.front_end_inputs(seed, B, T, H, K)
    bits = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).cuda()
    qkv0, w, st0 = bits(x["qkv"]), bits(x["conv_w"]), torch.from_numpy(x["conv_state"]).cuda()
    t_pad = -(-T // chunk) * chunk
    per_set = prefill_front_end_bytes(B, T, H, K)
    n_set = max(2, -(-(1 << 30) // per_set))
    sets = [(qkv0.clone(), st0.clone(), *(torch.empty((B, t_pad, H, D), device="cuda") for _ in range(3)))
            for _ in range(n_set)]
    stream = torch.cuda.current_stream()

    def step(i):
        qkv, st, q, k, v = sets[i % n_set]
        kda.kda_prefill_front_end(qkv, w, st, H, chunk, ki.L2_EPS, q=q, k=k, v=v, stream=stream)

    r = timer.run(step, steps, warmup)
    return r, per_set, n_set, B * T


def fused_decode_bytes(B: int, H: int, K: int, T: int = 1, n_snap: int = 0) -> int:
    """The decode walk from the raw projections in one kernel: BF16 qkv_proj read, FP32 conv state read
    and written (and n_snap conv snapshots written), state read and written (and n_snap snapshots), FP32
    gate and beta read, BF16 out_gate read and BF16 y written per row, and the BF16 conv weights and norm
    weight read once."""
    C = 3 * H * D
    return (B * T * C * 2 + B * C * K * 4 * (2 + n_snap) + B * H * (2 + n_snap) * STATE_BYTES
            + B * T * H * (D * 4 + 4 + D * 2 + D * 2) + C * K * 2 + 2 * D)


def bench_decode_fused_k(torch, kda, ki, steps, warmup, timer):
    """kda_decode_fused_k at B=128 H=32, 4 rows with 4 snapshots of both states (the decode_k workload from
    the raw projections), states rotated over >= 1 GiB."""
    w = ki.WORKLOADS["decode_k4_b128_h32"]
    B, H, T, n = w.batch, w.heads, w.T, w.n_snap
    K = 4
    x = ki.workload_inputs(w)
    fx = ki.front_end_inputs(41, B, T, H, K)
    nx = ki.norm_inputs(42, B * T, H)
    bits = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).cuda()
    qkv, cw = bits(fx["qkv"]), bits(fx["conv_w"])
    og, on = bits(nx["out_gate"]).view(B, T, H, D), bits(nx["o_norm"])
    g, b = torch.from_numpy(x["gate"]).cuda(), torch.from_numpy(x["beta"]).cuda()
    n_set = max(2, -(-(1 << 30) // (B * H * STATE_BYTES)))
    sts = [torch.from_numpy(x["state"]).cuda() for _ in range(n_set)]
    cst = torch.from_numpy(fx["conv_state"]).cuda()
    snaps = torch.empty((n, B, H, D, D), device="cuda")
    csn = torch.empty((n, B, 3 * H * D, K), device="cuda")
    y = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    r = timer.run(lambda i: kda.kda_decode_fused_k(qkv, cw, cst, g, b, sts[i % n_set], og, on, H, ki.NORM_EPS,
                                                   ki.L2_EPS, y=y, snapshots=snaps, conv_snapshots=csn,
                                                   n_snapshots=n, want_core=False), steps, warmup)
    return r, B * T, fused_decode_bytes(B, H, K, T, n), n_set


def bench_decode_chain(torch, kda, ki, reps, fused=False, whole=False):
    """The decode step of the block on BF16 q | k | v: front end -> kda_recurrent_step_bf16 -> gated RMSNorm
    at B=64 H=32, captured as one HIP graph of 8 steps, each on its own state set (8 x 128 MiB of recurrent
    state, so replays stream HBM), replayed back to back.  fused: front end -> kda_recurrent_step_bf16_norm
    (the norm inside the decode kernel, the FP32 core rows not stored).  whole: kda_decode_fused_step
    (front end, core and norm in one kernel, the core rows not stored).  Returns (us per step, bytes per
    step)."""
    w = ki.WORKLOADS["decode_b64_h32"]
    B, H = w.batch, w.heads
    FB, FT, FH, K, fseed = ki.FRONT_END_WORKLOADS["front_end_b64_h32_k4"]
    rows, nh, nseed = ki.NORM_WORKLOADS["gated_rmsnorm_b64_h32"]
    assert (FB, FT, FH) == (B, 1, H) and (rows, nh) == (B, H)
    x = ki.workload_inputs(w)
    fx = ki.front_end_inputs(fseed, B, 1, H, K)
    nx = ki.norm_inputs(nseed, rows, H)
    bits = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).cuda()
    qkv, cw, og, on = bits(fx["qkv"]), bits(fx["conv_w"]), bits(nx["out_gate"]), bits(nx["o_norm"])
    g, b = torch.from_numpy(x["gate"]).cuda(), torch.from_numpy(x["beta"]).cuda()
    n_set = 8
    sets = [dict(cst=torch.from_numpy(fx["conv_state"]).cuda(), st=torch.from_numpy(x["state"]).cuda(),
                 co=torch.empty((B, 1, 3 * H * D), dtype=torch.bfloat16, device="cuda"),
                 out=torch.empty((B, 1, H, D), device="cuda"),
                 y=torch.empty((B, H, D), dtype=torch.bfloat16, device="cuda")) for _ in range(n_set)]

    def chain(z):
        if whole:
            kda.kda_decode_fused_step(qkv, cw, z["cst"], g, b, z["st"], og.view(B, 1, H, D), on, H, ki.NORM_EPS,
                                      ki.L2_EPS, y=z["y"].view(B, 1, H, D), want_core=False)
            return
        kda.kda_decode_front_end_bf16(qkv, cw, z["cst"], H, ki.L2_EPS, conv_out=z["co"])
        if fused:
            kda.kda_recurrent_step_bf16_norm(z["co"], g, b, z["st"], og.view(B, 1, H, D), on, ki.NORM_EPS,
                                             y=z["y"].view(B, 1, H, D), want_core=False)
        else:
            kda.kda_recurrent_step_bf16(z["co"], g, b, z["st"], out=z["out"])
            kda.kda_gated_rmsnorm(z["out"].view(B, H, D), og, on, ki.NORM_EPS, out=z["y"])

    for z in sets:
        chain(z)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for z in sets:
            chain(z)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:  # untimed, past the device's settling after a switch of workload
        for _ in range(4):
            graph.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * n_set)
    if whole:
        nbytes = fused_decode_bytes(B, H, K)
    elif fused:  # the core rows stay on chip: the norm reads only its gate and weight and writes y
        nbytes = (front_end_bytes(B, 1, H, K, 0, out_bytes=2) + decode_bytes(B, H, qkv_bytes=2) - B * H * D * 4
                  + B * H * D * 4 + 2 * D)
    else:
        nbytes = (front_end_bytes(B, 1, H, K, 0, out_bytes=2) + decode_bytes(B, H, qkv_bytes=2) + norm_bytes(B, H))
    return us, nbytes


def bench_prefill_chain(torch, kda, ki, steps, warmup, timer, fused=False):
    """The prefill of the block at T=8192 H=32 C=64: prefill front end -> kda_chunk_prefill -> gated RMSNorm
    of the T rows, timed eagerly as one step.  fused: kda_chunk_prefill_fused (the front end inside the
    prefill) -> gated RMSNorm."""
    B, T, H, K, C, fseed = ki.PREFILL_FRONT_END_WORKLOADS["prefill_front_end_t8192_h32_k4"]
    w = ki.WORKLOADS["prefill_h32_t8192_c64"]
    rows, nh, nseed = ki.NORM_WORKLOADS["gated_rmsnorm_t8192_h32"]
    assert (B, T, H, C) == (w.batch, w.T, w.heads, w.chunk) and (rows, nh) == (T, H)
    t_pad = -(-T // C) * C
    fx = ki.front_end_inputs(fseed, B, T, H, K)
    x = ki.workload_inputs(w)
    nx = ki.norm_inputs(nseed, rows, H)
    bits = lambda a: torch.from_numpy(a.view("int16")).view(torch.bfloat16).cuda()
    qkv, cw, og, on = bits(fx["qkv"]), bits(fx["conv_w"]), bits(nx["out_gate"]), bits(nx["o_norm"])
    cst = torch.from_numpy(fx["conv_state"]).cuda()
    g = torch.from_numpy(x["gate"][:, :t_pad].copy()).cuda()
    b = torch.from_numpy(x["beta"][:, :t_pad].copy()).cuda()
    st = torch.from_numpy(x["state"]).cuda()
    q, k, v, out = (torch.empty((B, t_pad, H, D), device="cuda") for _ in range(4))
    ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T, C), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        if fused:
            kda.kda_chunk_prefill_fused(qkv, cw, cst, g, b, st, C, ki.L2_EPS, out=out, workspace=ws, stream=stream)
        else:
            kda.kda_prefill_front_end(qkv, cw, cst, H, C, ki.L2_EPS, q=q, k=k, v=v, stream=stream)
            kda.kda_chunk_prefill(q, k, v, g, b, st, T, C, out=out, workspace=ws, stream=stream)
        kda.kda_gated_rmsnorm(out[0, :T], og, on, ki.NORM_EPS, out=y, stream=stream)

    return timer.run(step, steps, warmup), B * T


def bench_prefill_front_end_varlen(torch, kda, ki, name, steps, warmup, timer, K=4):
    """kda_prefill_front_end_varlen over the packed sequences of a varlen prefill workload."""
    import numpy as np
    total, H, C, mean_len, seed = ki.VARLEN_WORKLOADS[name]
    lens = ki.varlen_lengths(seed, total, mean_len)
    fx = ki.front_end_inputs(seed, 1, total, H, K)
    st0 = ki.front_end_inputs(seed + 1, len(lens), 1, H, K)["conv_state"]
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view("int16")).view(torch.bfloat16).cuda()
    qkv, w = bits(fx["qkv"][0]), bits(fx["conv_w"])
    st = torch.from_numpy(st0).cuda()
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    q, k, v = (torch.empty((total, H, D), device="cuda") for _ in range(3))
    stream = torch.cuda.current_stream()

    def step(i):
        kda.kda_prefill_front_end_varlen(qkv, w, st, cu, H, ki.L2_EPS, q=q, k=k, v=v, stream=stream)

    r = timer.run(step, steps, warmup)
    Cd = 3 * H * D
    nbytes = total * Cd * 6 + 2 * len(lens) * Cd * K * 4 + Cd * K * 2
    return r, nbytes, total


def bench_varlen(torch, kda, ki, name, steps, warmup, timer):
    total, H, C, mean_len, seed = ki.VARLEN_WORKLOADS[name]
    lens = ki.varlen_lengths(seed, total, mean_len)
    x = ki.varlen_inputs(seed, lens, H, -5.0, 0.02)
    d = {n: torch.from_numpy(x[n]).cuda() for n in ("q", "k", "v", "gate", "beta", "state", "cu_seqlens")}
    out = torch.empty_like(d["q"])
    ws = torch.empty(kda.kda_chunk_prefill_varlen_workspace_bytes(len(lens), H, total, C), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        kda.kda_chunk_prefill_varlen(d["q"], d["k"], d["v"], d["gate"], d["beta"], d["state"], d["cu_seqlens"], C,
                                     out=out, workspace=ws, stream=stream)

    r = timer.run(step, steps, warmup)
    return r, lens, H, C


def bench_varlen_fused(torch, kda, ki, name, steps, warmup, timer, K=4):
    """kda_chunk_prefill_varlen_fused (front end inside the prefill) over a varlen prefill workload, with the
    front end inputs of the varlen front end workload."""
    import numpy as np
    total, H, C, mean_len, seed = ki.VARLEN_WORKLOADS[name]
    lens = ki.varlen_lengths(seed, total, mean_len)
    x = ki.varlen_inputs(seed, lens, H, -5.0, 0.02)
    fx = ki.front_end_inputs(seed, 1, total, H, K)
    cst = torch.from_numpy(ki.front_end_inputs(seed + 1, len(lens), 1, H, K)["conv_state"]).cuda()
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view("int16")).view(torch.bfloat16).cuda()
    qkv, w = bits(fx["qkv"][0]), bits(fx["conv_w"])
    d = {n: torch.from_numpy(x[n]).cuda() for n in ("gate", "beta", "state", "cu_seqlens")}
    out = torch.empty((total, H, D), device="cuda")
    ws = torch.empty(kda.kda_chunk_prefill_varlen_workspace_bytes(len(lens), H, total, C), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def step(i):
        kda.kda_chunk_prefill_varlen_fused(qkv, w, cst, d["gate"], d["beta"], d["state"], d["cu_seqlens"], C,
                                           ki.L2_EPS, out=out, workspace=ws, stream=stream)

    return timer.run(step, steps, warmup), lens


def bench_prefill(torch, kda, ki, name, steps, warmup, timer, chunk=None):
    """kda_chunk_prefill on workload `name` (chunk: another chunk width on the same inputs)."""
    w = ki.WORKLOADS[name]
    B, H, T, C = w.batch, w.heads, w.T, chunk or w.chunk
    t_pad = -(-T // C) * C
    dev = lambda a: torch.from_numpy(a).cuda()
    tens = {}
    # generate one sequence at a time and move it to the GPU (bounded host memory)
    for n in ("q", "k", "v", "gate"):
        tens[n] = torch.empty((B, t_pad, H, D), device="cuda")
    tens["beta"] = torch.empty((B, t_pad, H), device="cuda")
    state0 = torch.empty((B, H, D, D), device="cuda")
    for s in range(B):
        part = _sequence(ki, w, s, T, t_pad)
        for n in tens:
            tens[n][s].copy_(dev(part[n][0]))
        state0[s].copy_(dev(part["state"][0]))
    state = state0.clone()
    out = torch.empty((B, t_pad, H, D), device="cuda")
    ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T, C), dtype=torch.uint8, device="cuda")

    def step(i):
        kda.kda_chunk_prefill(tens["q"], tens["k"], tens["v"], tens["gate"], tens["beta"], state, T, C, out=out,
                              workspace=ws)

    r = timer.run(step, steps, warmup)
    extra = {}
    if C == 64 and T >= 1024:
        # the call's two kernels apart: kda_chunk_scan alone from the records the last call left in the
        # workspace gives the scan's time; the prepare's is the rest of the call
        def scan_step(i):
            kda.kda_chunk_scan(state, T, C, ws, out=out)

        rs = timer.run(scan_step, steps, 3)
        scan_s = rs["launch_avg_s"]
        prep_s = max(r["launch_avg_s"] - scan_s, 1e-9)
        scan_fl = 6.0 * D * D * B * H * T
        prep_bytes = 4 * B * t_pad * H * D * 4 + B * t_pad * H * 4 + ws.numel()  # inputs read, records written
        extra = {"scan_ms": scan_s * 1e3, "scan_mfma_frac": scan_fl / scan_s / 1e12 / MFMA_F32_PEAK_TFLOPS,
                 "prepare_ms": prep_s * 1e3, "prepare_GB_per_s": prep_bytes / prep_s / 1e9,
                 "prepare_hbm_frac": prep_bytes / prep_s / 1e9 / HBM_PEAK_GBS}
    if w.tail_steps:
        # decode steps continuing from the prefill's final state (rows T.. of the same streams)
        state.copy_(state0)
        step(0)
        tail = _tail_inputs(ki, w, torch)
        o = torch.empty((B, 1, H, D), device="cuda")

        def dstep(i):
            j = i % w.tail_steps
            kda.kda_recurrent_step(*(tail[n][j] for n in ("q", "k", "v", "gate", "beta")), state, out=o)

        rt = timer.run(dstep, w.tail_steps, 0)
        # The wall time per step above is bound by the Python binding's per-call work at this
        # size; the device time per step comes from the same steps captured once in a HIP graph
        # and replayed back to back.
        graph_us = None
        try:
            state.copy_(state0)
            step(0)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for j in range(w.tail_steps):
                    dstep(j)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            graph_us = e0.elapsed_time(e1) * 1e3 / (5 * w.tail_steps)
        except Exception as exc:  # capture unavailable: report the wall rate only
            log(f"tail graph timing skipped: {exc}")
        extra.update({"tail_steps": w.tail_steps, "tail_us_per_step": rt["s_per_step"] * 1e6,
                      "tail_graph_us_per_step": graph_us, "tail_tokens_per_s": B / rt["s_per_step"]})
    return w, r, extra


def bench_transition(torch, kda, ki, name, T, steps, warmup, timer, n_fold=-1):
    """kda_chunk_prefill_transition over the first T tokens of every sequence of workload `name`.
    n_fold >= 0: a device's whole share of a split sequence instead: its transition (records kept),
    n_fold folds of earlier segments' pairs into the state, then kda_chunk_scan from the kept records."""
    w = ki.WORKLOADS[name]
    B, H, C = w.batch, w.heads, w.chunk
    t_pad = -(-T // C) * C
    tens = {n: torch.empty((B, t_pad, H, D), device="cuda") for n in ("q", "k", "v", "gate")}
    tens["beta"] = torch.empty((B, t_pad, H), device="cuda")
    for s in range(B):
        part = _sequence(ki, w, s, T, t_pad)
        for n in tens:
            tens[n][s].copy_(torch.from_numpy(part[n][0]).cuda())
    P = torch.empty((B, H, D, D), device="cuda")
    Q = torch.empty((B, H, D, D), device="cuda")
    ws = torch.empty(kda.kda_chunk_prefill_workspace_bytes(B, H, T, C), dtype=torch.uint8, device="cuda")

    state = torch.zeros((B, H, D, D), device="cuda")
    out = torch.empty((B, t_pad, H, D), device="cuda")

    def step(i):
        kda.kda_chunk_prefill_transition(tens["q"], tens["k"], tens["v"], tens["gate"], tens["beta"], T, C,
                                         trans_p=P, trans_q=Q, workspace=ws)
        if n_fold >= 0:
            for _ in range(n_fold):
                kda.kda_state_transition_apply(P, Q, state)
            kda.kda_chunk_scan(state, T, C, ws, out=out)

    return w, timer.run(step, steps, warmup)


def bench_transition_apply(torch, kda, B, H, steps, warmup, timer):
    """kda_state_transition_apply on B x H states in place (P = I / 2, so repeated folds stay bounded)."""
    P = (0.5 * torch.eye(D, device="cuda")).expand(B, H, D, D).contiguous()
    Q = torch.randn((B, H, D, D), device="cuda")
    S = torch.randn((B, H, D, D), device="cuda")
    return timer.run(lambda i: kda.kda_state_transition_apply(P, Q, S), steps, warmup)


def _sequence(ki, w, s, T, t_pad):
    import numpy as np
    arrays = {n: np.full((1, t_pad, w.heads, D), 0.0 if w.pad_value is None else w.pad_value, np.float32)
              for n in ("q", "k", "v", "gate")}
    arrays["beta"] = np.full((1, t_pad, w.heads), 0.0 if w.pad_value is None else w.pad_value, np.float32)
    from concurrent.futures import ThreadPoolExecutor
    jobs = [(r, min(T, r + ki.ROW_BLOCK)) for r in range(0, T, ki.ROW_BLOCK)]
    with ThreadPoolExecutor(ki.default_threads()) as ex:
        list(ex.map(lambda j: ki.fill_rows(w.seed, s, j[0], j[1], w.heads, w.gate_lo,
                                           {n: a[0, j[0]:j[1]] for n, a in arrays.items()}), jobs))
    arrays["state"] = ki.initial_state(w.seed, s, w.heads, w.state_std)[None]
    return arrays


def _tail_inputs(ki, w, torch):
    import numpy as np
    rows = [ki.sequence_rows(w.seed, s, w.T, w.T + w.tail_steps, w.heads, w.gate_lo) for s in range(w.batch)]
    tail = {}
    for n in ("q", "k", "v", "gate", "beta"):
        a = np.stack([r[n] for r in rows])            # [B, steps, H, (D)]
        tail[n] = [torch.from_numpy(np.ascontiguousarray(a[:, j:j + 1])).cuda() for j in range(w.tail_steps)]
    return tail


# ---------------------------------------------------------------- cpu baseline
def _oracle_rate(oracle, x, tokens: int, T: int | None = None, n_snap: int = 0):
    """One run of the fp64 oracle (as it stands) on x; returns (tokens/s, wall s, threads)."""
    t0 = time.perf_counter()
    _, _, _, threads = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"], T=T, n_snap=n_snap)
    el = time.perf_counter() - t0
    return tokens / el, el, threads


def cpu_baselines(ki, budget_s: float = 10.0):
    """The fp64 oracle (never tuned for this) timed on the host cores beside every configuration, on
    the same seeded inputs.  Returns (headline entry, {workload: entry}); input generation is not
    timed.  Each sample is bounded so the whole baseline stays within about half a minute."""
    import numpy as np
    import oracle
    res = {}

    cpu_model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu_model)
    except OSError:
        pass

    def entry(rate, threads, sample, unit="tokens/s"):
        return {"value": rate, "unit": unit, "cores": threads, "kind": "oracle",
                "sample": sample + f"; os.cpu_count()={os.cpu_count()}", "cpu": cpu_model}

    # decode B=64 H=32 (headline): repeated full decode steps until ~budget_s of wall time
    w = ki.WORKLOADS["decode_b64_h32"]
    x = ki.workload_inputs(w)
    state = x["state"].astype("float64")
    reps, t0, threads = 0, time.perf_counter(), 1
    while True:
        _, state, _, threads = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], state)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 100000:
            break
    res[w.name] = entry(w.batch * reps / el, threads,
                        f"{reps} full decode steps (B=64, H=32, one token each), {el:.1f} s wall on {threads} threads")
    # decode_k B=128 H=32 k=4 with 4 snapshots: the whole call
    w = ki.WORKLOADS["decode_k4_b128_h32"]
    x = ki.workload_inputs(w)
    rate, el, th = _oracle_rate(oracle, x, w.batch * w.T, n_snap=w.n_snap)
    res[w.name] = entry(rate, th, f"one whole call (B=128, H=32, 4 rows, 4 snapshots), {el:.2f} s wall on {th} threads")
    # prefill T=64 H=2: the whole call
    w = ki.WORKLOADS["prefill_h2_t64_c16"]
    x = ki.workload_inputs(w)
    rate, el, th = _oracle_rate(oracle, x, w.batch * w.T, T=w.T)
    res[w.name] = entry(rate, th, f"one whole call (T=64, H=2), {el:.4f} s wall on {th} threads")
    # prefill T=8192 H=32: the whole call (32 independent heads, so at most 32 threads)
    w = ki.WORKLOADS["prefill_h32_t8192_c64"]
    x = ki.workload_inputs(w)
    rate, el, th = _oracle_rate(oracle, x, w.batch * w.T, T=w.T)
    res[w.name] = entry(rate, th, f"one whole call (T=8192, H=32), {el:.1f} s wall on {th} threads")
    # prefill 4 x 32768 H=32: the first 4096 tokens of each sequence (an eighth of the call)
    w = ki.WORKLOADS["prefill_b4_h32_t32768_c64"]
    Ts = 4096
    rows = [ki.sequence_rows(w.seed, s, 0, Ts, w.heads, w.gate_lo) for s in range(w.batch)]
    x = {n: np.ascontiguousarray(np.stack([r[n] for r in rows])) for n in ("q", "k", "v", "gate", "beta")}
    x["state"] = np.stack([ki.initial_state(w.seed, s, w.heads, w.state_std) for s in range(w.batch)])
    rate, el, th = _oracle_rate(oracle, x, w.batch * Ts, T=Ts)
    res[w.name] = entry(rate, th, f"the first {Ts} tokens of each of the 4 sequences, all 32 heads, "
                                  f"{el:.1f} s wall on {th} threads")
    return res


# ---------------------------------------------------------------- traffic from committed counters
def committed_traffic(kernel_src: str, profile: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    sha = hashlib.sha256(open(os.path.join(ROOT, kernel_src), "rb").read()).hexdigest()[:16]
    if fields.get("kernel_source_sha256_16") != sha:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default="", help="comma list of workloads to time (default: all)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--copy-probe", action="store_true", help="time a plain 1 GiB device copy kernel (1 GiB read + 1 GiB written per launch) and exit")
    ap.add_argument("--reps", type=int, default=0, help="override the repetitions of every workload (profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the core needs no collective and "
                                   "--gpus above 1 is not supported", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import kda_gated_delta_core_amd as kda
    import kda_inputs as ki

    kda.load_library()
    timer = Timer(torch, prewarm_s=0.0 if args.reps else 0.3)  # (profiling runs: only the counted calls)
    if args.copy_probe:
        n = 1 << 28  # 1 GiB of fp32
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        # an elementwise kernel (not a runtime blit) so counter collection sees it as a dispatch
        r = timer.run(lambda i: torch.mul(src, 1.0, out=dst), args.reps or 20, 0 if args.reps else 3)
        log(f"copy probe: 1 GiB read + 1 GiB write per launch, {2 * n * 4 / r['launch_avg_s'] / 1e9:.1f} GB/s")
        return

    only = set(filter(None, args.only.split(",")))
    want = lambda n: not only or n in only
    workloads = {}

    headline = None
    if want("decode_b64_h32"):
        log("decode_b64_h32")
        w, r, nbytes, n_buf = bench_decode(torch, kda, ki, args.reps or args.steps, args.warmup, timer)
        gbs = nbytes / r["launch_avg_s"] / 1e9
        headline = (w, r, nbytes, n_buf, gbs)
        workloads[w.name] = {"tokens_per_s": w.batch / r["s_per_step"], "us_per_step": r["s_per_step"] * 1e6,
                             "kernel_us": r["launch_avg_s"] * 1e6, "GB_per_s": gbs,
                             "hbm_frac": gbs / HBM_PEAK_GBS, "state_buffers_rotated": n_buf}
    if want("decode_k4_b128_h32"):
        log("decode_k4_b128_h32")
        w, r, nbytes = bench_decode_k(torch, kda, ki, args.reps or max(10, args.steps // 2), args.warmup, timer)
        gbs = nbytes / r["launch_avg_s"] / 1e9
        workloads[w.name] = {"tokens_per_s": w.batch * w.T / r["s_per_step"], "us_per_call": r["s_per_step"] * 1e6,
                             "kernel_us": r["launch_avg_s"] * 1e6, "GB_per_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
    # the same two decode workloads reading BF16 q | k | v packed per token (the BF16 front end's output)
    if want("decode_bf16_b64_h32"):
        log("decode_bf16_b64_h32")
        w, r, nbytes, _ = bench_decode(torch, kda, ki, args.reps or args.steps, args.warmup, timer, bf16=True)
        gbs = nbytes / r["launch_avg_s"] / 1e9
        workloads["decode_bf16_b64_h32"] = {"tokens_per_s": w.batch / r["s_per_step"],
                                            "us_per_step": r["s_per_step"] * 1e6,
                                            "kernel_us": r["launch_avg_s"] * 1e6, "GB_per_s": gbs,
                                            "hbm_frac": gbs / HBM_PEAK_GBS}
    if want("decode_k4_bf16_b128_h32"):
        log("decode_k4_bf16_b128_h32")
        w, r, nbytes = bench_decode_k(torch, kda, ki, args.reps or max(10, args.steps // 2), args.warmup, timer,
                                      bf16=True)
        gbs = nbytes / r["launch_avg_s"] / 1e9
        workloads["decode_k4_bf16_b128_h32"] = {"tokens_per_s": w.batch * w.T / r["s_per_step"],
                                                "us_per_call": r["s_per_step"] * 1e6,
                                                "kernel_us": r["launch_avg_s"] * 1e6, "GB_per_s": gbs,
                                                "hbm_frac": gbs / HBM_PEAK_GBS}
    # the gate (kda_gate of BF16 g_raw) and beta (sigmoid of the logit) formed inside the core kernels
    if want("decode_gated_b64_h32"):
        log("decode_gated_b64_h32")
        w, r, nbytes = bench_decode_gated(torch, kda, ki, args.reps or args.steps, args.warmup, timer)
        gbs = nbytes / r["launch_avg_s"] / 1e9
        workloads["decode_gated_b64_h32"] = {"tokens_per_s": w.batch / r["s_per_step"],
                                             "us_per_step": r["s_per_step"] * 1e6,
                                             "kernel_us": r["launch_avg_s"] * 1e6, "GB_per_s": gbs,
                                             "hbm_frac": gbs / HBM_PEAK_GBS}
    if want("prefill_gated_h32_t8192_c64"):
        log("prefill_gated_h32_t8192_c64")
        w, r = bench_prefill_gated(torch, kda, ki, args.reps or 20, 0 if args.reps else 60, timer)
        tf = prefill_flops(w.batch, w.heads, w.T, w.chunk) / r["launch_avg_s"] / 1e12
        workloads["prefill_gated_h32_t8192_c64"] = {"tokens_per_s": w.batch * w.T / r["s_per_step"],
                                                    "ms_per_call": r["s_per_step"] * 1e3,
                                                    "call_ms": r["launch_avg_s"] * 1e3,
                                                    "algorithmic_TFLOP_per_s": tf,
                                                    "mfma_frac": tf / MFMA_F32_PEAK_TFLOPS}
    if want("prefill_bf16_h32_t8192_c64"):
        log("prefill_bf16_h32_t8192_c64")
        w, r = bench_prefill_bf16(torch, kda, ki, args.reps or 20, 0 if args.reps else 60, timer)
        tf = prefill_flops(w.batch, w.heads, w.T, w.chunk) / r["launch_avg_s"] / 1e12
        workloads["prefill_bf16_h32_t8192_c64"] = {"tokens_per_s": w.batch * w.T / r["s_per_step"],
                                                   "ms_per_call": r["s_per_step"] * 1e3,
                                                   "call_ms": r["launch_avg_s"] * 1e3,
                                                   "algorithmic_TFLOP_per_s": tf,
                                                   "mfma_frac": tf / MFMA_F32_PEAK_TFLOPS}
    # (timed calls, untimed warm-up calls): once the T=8192 prefill starts, its calls run up to 30%
    # slower for ~15 ms (a device-level transient: the first few calls are fast, then the time rises
    # and settles back over ~30 calls), so it gets 60 untimed calls before the timed ones
    for name, steps, warm in (("prefill_h32_t8192_c64", 20, 60), ("prefill_b4_h32_t32768_c64", 4, 3),
                              ("prefill_h2_t64_c16", 50, 10)):
        if not want(name):
            continue
        log(name)
        w, r, extra = bench_prefill(torch, kda, ki, name, args.reps or steps, 0 if args.reps else warm, timer)
        fl = prefill_flops(w.batch, w.heads, w.T, w.chunk)
        tf = fl / r["launch_avg_s"] / 1e12
        res = {"tokens_per_s": w.batch * w.T / r["s_per_step"], "ms_per_call": r["s_per_step"] * 1e3,
               "call_ms": r["launch_avg_s"] * 1e3, "algorithmic_TFLOP_per_s": tf,
               "mfma_frac": tf / MFMA_F32_PEAK_TFLOPS,
               "GB_per_s": prefill_bytes(w.batch, w.heads, w.T) / r["launch_avg_s"] / 1e9}
        res.update(extra)
        workloads[name] = res
    # the T=8192 workload at the narrower chunk widths (the same inputs, rows >= T still the pad)
    for C in (32, 16):
        name = f"prefill_h32_t8192_c{C}"
        if not want(name):
            continue
        log(name)
        w, r, _ = bench_prefill(torch, kda, ki, "prefill_h32_t8192_c64", args.reps or 20, 0 if args.reps else 60,
                                timer, chunk=C)
        tf = prefill_flops(w.batch, w.heads, w.T, C) / r["launch_avg_s"] / 1e12
        workloads[name] = {"tokens_per_s": w.batch * w.T / r["s_per_step"], "ms_per_call": r["s_per_step"] * 1e3,
                           "call_ms": r["launch_avg_s"] * 1e3, "algorithmic_TFLOP_per_s": tf,
                           "mfma_frac": tf / MFMA_F32_PEAK_TFLOPS}
    # segment transitions: a whole T=8192 prefill as one segment, and one device's share of the
    # 4 x 32768 prefill split into 8 token segments (4 sequences x 4096 tokens)
    for name, base, T, steps, warm in (("transition_h32_t8192_c64", "prefill_h32_t8192_c64", 8192, 20, 20),
                                       ("transition_b4_h32_t4096_c64", "prefill_b4_h32_t32768_c64", 4096, 10, 10)):
        if not want(name):
            continue
        log(name)
        w, r = bench_transition(torch, kda, ki, base, T, args.reps or steps, 0 if args.reps else warm, timer)
        tf = transition_flops(w.batch, w.heads, T, w.chunk) / r["launch_avg_s"] / 1e12
        workloads[name] = {"tokens_per_s": w.batch * T / r["s_per_step"], "ms_per_call": r["s_per_step"] * 1e3,
                           "call_ms": r["launch_avg_s"] * 1e3, "algorithmic_TFLOP_per_s": tf,
                           "mfma_frac": tf / MFMA_F32_PEAK_TFLOPS}
    if want("split_device_b4_h32_t4096_c64"):
        # the last of 8 devices sharing the 4 x 32768 prefill by token segments, without the exchange
        log("split_device_b4_h32_t4096_c64")
        w, r = bench_transition(torch, kda, ki, "prefill_b4_h32_t32768_c64", 4096, args.reps or 10,
                                0 if args.reps else 10, timer, n_fold=7)
        workloads["split_device_b4_h32_t4096_c64"] = {
            "ms_per_call": r["s_per_step"] * 1e3, "device_ms": r["launch_avg_s"] * 1e3,
            "steps": "transition (records kept) + 7 folds + kda_chunk_scan, one device's share; no exchange"}
    if want("transition_apply_b4_h32"):
        # the fold step for 4 sequences x 32 heads: a device folds the pairs of the segments before its own
        log("transition_apply_b4_h32")
        r = bench_transition_apply(torch, kda, 4, 32, args.reps or 100, args.warmup, timer)
        fl = 4 * 32 * 2.0 * D ** 3
        workloads["transition_apply_b4_h32"] = {"us_per_call": r["s_per_step"] * 1e6,
                                                "kernel_us": r["launch_avg_s"] * 1e6,
                                                "algorithmic_TFLOP_per_s": fl / r["launch_avg_s"] / 1e12}
    for name in ki.VARLEN_WORKLOADS:
        if not want(name):
            continue
        log(name)
        r, lens, H, C = bench_varlen(torch, kda, ki, name, args.reps or 20, 0 if args.reps else 20, timer)
        fl = sum(prefill_flops(1, H, n, C) for n in lens)
        tf = fl / r["launch_avg_s"] / 1e12
        workloads[name] = {"tokens_per_s": sum(lens) / r["s_per_step"], "ms_per_call": r["s_per_step"] * 1e3,
                           "call_ms": r["launch_avg_s"] * 1e3, "algorithmic_TFLOP_per_s": tf,
                           "mfma_frac": tf / MFMA_F32_PEAK_TFLOPS, "sequences": len(lens),
                           "min_len": min(lens), "max_len": max(lens)}
    for base in ki.FRONT_END_WORKLOADS:
        for bf16 in (False, True):
            name = base.replace("front_end_", "front_end_bf16_") if bf16 else base
            if not want(name):
                continue
            log(name)
            r, nbytes, n_set, tokens = bench_front_end(torch, kda, ki, base, args.reps or args.steps, args.warmup,
                                                       timer, bf16=bf16)
            gbs = nbytes / r["launch_avg_s"] / 1e9
            workloads[name] = {"tokens_per_s": tokens / r["s_per_step"], "us_per_call": r["s_per_step"] * 1e6,
                               "kernel_us": r["launch_avg_s"] * 1e6, "GB_per_s": gbs,
                               "hbm_frac": gbs / HBM_PEAK_GBS, "buffer_sets_rotated": n_set}
    for name in ki.VARLEN_WORKLOADS:
        fe_name = name.replace("prefill_varlen_", "prefill_front_end_varlen_").replace("_c64", "_k4")
        if not want(fe_name):
            continue
        log(fe_name)
        r, nbytes, tokens = bench_prefill_front_end_varlen(torch, kda, ki, name, args.reps or 50, args.warmup, timer)
        gbs = nbytes / r["launch_avg_s"] / 1e9
        workloads[fe_name] = {"tokens_per_s": tokens / r["s_per_step"], "us_per_call": r["s_per_step"] * 1e6,
                              "kernel_us": r["launch_avg_s"] * 1e6, "GB_per_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
    for name in ki.PREFILL_FRONT_END_WORKLOADS:
        if not want(name):
            continue
        log(name)
        r, nbytes, n_set, tokens = bench_prefill_front_end(torch, kda, ki, name, args.reps or 50, args.warmup, timer)
        gbs = nbytes / r["launch_avg_s"] / 1e9
        workloads[name] = {"tokens_per_s": tokens / r["s_per_step"], "us_per_call": r["s_per_step"] * 1e6,
                           "kernel_us": r["launch_avg_s"] * 1e6, "GB_per_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                           "buffer_sets_rotated": n_set}
    if want("decode_chain_bf16_b64_h32"):
        log("decode_chain_bf16_b64_h32")
        us, nbytes = bench_decode_chain(torch, kda, ki, args.reps or 50)
        workloads["decode_chain_bf16_b64_h32"] = {
            "tokens_per_s": 64 / (us * 1e-6), "us_per_step": us, "GB_per_s": nbytes / (us * 1e-6) / 1e9,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "steps": "front end (BF16 out) + kda_recurrent_step_bf16 + gated RMSNorm, replayed from one HIP graph"}
    if want("decode_chain_fused_bf16_b64_h32"):
        log("decode_chain_fused_bf16_b64_h32")
        us, nbytes = bench_decode_chain(torch, kda, ki, args.reps or 50, fused=True)
        workloads["decode_chain_fused_bf16_b64_h32"] = {
            "tokens_per_s": 64 / (us * 1e-6), "us_per_step": us, "GB_per_s": nbytes / (us * 1e-6) / 1e9,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "steps": "front end (BF16 out) + kda_recurrent_step_bf16_norm (norm fused), replayed from one HIP graph"}
    if want("decode_fused_b64_h32"):
        log("decode_fused_b64_h32")
        us, nbytes = bench_decode_chain(torch, kda, ki, args.reps or 50, whole=True)
        workloads["decode_fused_b64_h32"] = {
            "tokens_per_s": 64 / (us * 1e-6), "us_per_step": us, "GB_per_s": nbytes / (us * 1e-6) / 1e9,
            "hbm_frac": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "steps": "kda_decode_fused_step (front end, core and gated RMSNorm in one kernel), replayed from one "
                     "HIP graph"}
    if want("decode_fused_k4_b128_h32"):
        log("decode_fused_k4_b128_h32")
        r, tokens, nbytes, n_set = bench_decode_fused_k(torch, kda, ki, args.reps or args.steps, 0 if args.reps else
                                                        args.warmup, timer)
        gbs = nbytes / r["launch_avg_s"] / 1e9
        workloads["decode_fused_k4_b128_h32"] = {
            "tokens_per_s": tokens / r["s_per_step"], "us_per_call": r["s_per_step"] * 1e6,
            "kernel_us": r["launch_avg_s"] * 1e6, "GB_per_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "state_buffers_rotated": n_set,
            "steps": "kda_decode_fused_k: 4 rows, 4 snapshots of the state and of the conv state, y only"}
    if want("prefill_chain_t8192_h32"):
        log("prefill_chain_t8192_h32")
        r, tokens = bench_prefill_chain(torch, kda, ki, args.reps or 20, 0 if args.reps else 60, timer)
        workloads["prefill_chain_t8192_h32"] = {
            "tokens_per_s": tokens / r["s_per_step"], "ms_per_call": r["s_per_step"] * 1e3,
            "device_ms": r["launch_avg_s"] * 1e3,
            "steps": "kda_prefill_front_end + kda_chunk_prefill + gated RMSNorm"}
    for name in ki.VARLEN_WORKLOADS:
        fname = name.replace("prefill_varlen_", "prefill_varlen_fused_")
        if not want(fname):
            continue
        log(fname)
        r, lens = bench_varlen_fused(torch, kda, ki, name, args.reps or 20, 0 if args.reps else 20, timer)
        workloads[fname] = {"tokens_per_s": sum(lens) / r["s_per_step"], "ms_per_call": r["s_per_step"] * 1e3,
                            "call_ms": r["launch_avg_s"] * 1e3, "sequences": len(lens),
                            "steps": "kda_chunk_prefill_varlen_fused: the varlen front end inside the varlen prefill"}
    if want("prefill_chain_fused_t8192_h32"):
        log("prefill_chain_fused_t8192_h32")
        r, tokens = bench_prefill_chain(torch, kda, ki, args.reps or 20, 0 if args.reps else 60, timer, fused=True)
        workloads["prefill_chain_fused_t8192_h32"] = {
            "tokens_per_s": tokens / r["s_per_step"], "ms_per_call": r["s_per_step"] * 1e3,
            "device_ms": r["launch_avg_s"] * 1e3,
            "steps": "kda_chunk_prefill_fused (front end inside the prepare) + gated RMSNorm"}
    for name in ki.NORM_WORKLOADS:
        if not want(name):
            continue
        log(name)
        r, nbytes, n_set = bench_norm(torch, kda, ki, name, args.reps or args.steps, args.warmup, timer)
        rows, heads, _ = ki.NORM_WORKLOADS[name]
        gbs = nbytes / r["launch_avg_s"] / 1e9
        workloads[name] = {"tokens_per_s": rows / r["s_per_step"], "us_per_call": r["s_per_step"] * 1e6,
                           "kernel_us": r["launch_avg_s"] * 1e6, "GB_per_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                           "buffer_sets_rotated": n_set}
    copy_gbs = None
    if want("copy_ceiling"):
        # the practical HBM ceiling beside the vendor peak: a plain 1 GiB device copy (torch's elementwise
        # kernel, 1 GiB read + 1 GiB written per launch), timed like the workloads
        log("copy_ceiling")
        n = 1 << 28
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        r = timer.run(lambda i: torch.mul(src, 1.0, out=dst), args.reps or 20, 3)
        copy_gbs = 2 * n * 4 / r["launch_avg_s"] / 1e9
        workloads["copy_ceiling"] = {"GB_per_s": copy_gbs, "hbm_frac": copy_gbs / HBM_PEAK_GBS,
                                     "kernel_us": r["launch_avg_s"] * 1e6,
                                     "steps": "1 GiB read + 1 GiB written per launch by a plain copy kernel"}
        del src, dst
    if copy_gbs:
        for res in workloads.values():
            if "prepare_GB_per_s" in res:
                res["prepare_frac_of_copy"] = res["prepare_GB_per_s"] / copy_gbs
    for name, res in workloads.items():
        log(f"{name}: " + ", ".join(f"{k}={v:.4g}" if isinstance(v, float) else f"{k}={v}"
                                    for k, v in res.items()))

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic"}
    if headline is not None:
        w, r, nbytes, n_buf, gbs = headline
        traffic = committed_traffic("kda_gated_delta_core_amd/csrc/kda_recurrent.hip",
                                    "recurrent_decode_b64_h32_counters.txt")
        line.update({
            "value": w.batch / r["s_per_step"], "unit": "tokens/s", "ms_per_step": r["s_per_step"] * 1e3,
            "config": {"workload": w.name, "op": "kda_recurrent_step", "batch": w.batch, "heads": w.heads,
                       "head_dim": D, "tokens_per_step": w.batch, "state_dtype": "f32",
                       "state_buffers_rotated": n_buf},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                         "kernel": "recurrent_kernel", "algorithmic_bytes_per_launch": nbytes,
                         "kernel_avg_us": r["launch_avg_s"] * 1e6, "copy_GB_per_s": copy_gbs,
                         "frac_of_copy": gbs / copy_gbs if copy_gbs else None},
        })
    line["workloads"] = workloads
    if not args.no_cpu and headline is not None:
        log("cpu baselines (fp64 oracle beside every configuration)")
        base = cpu_baselines(ki)
        line["cpu_baseline"] = base["decode_b64_h32"]
        for name, b in base.items():
            log(f"oracle {name}: {b['value']:.4g} {b['unit']} ({b['sample']})")
            if name in workloads:
                workloads[name]["cpu_oracle"] = b
                rate = workloads[name].get("tokens_per_s")
                if rate:
                    workloads[name]["gpu_over_oracle"] = rate / b["value"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
