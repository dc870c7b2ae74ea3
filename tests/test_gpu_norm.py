"""GPU parity of kda_gated_rmsnorm (through the C ABI) with the fp64 oracle.

The result is BF16: every element must lie within one BF16 unit in the last place of the exact
(fp64) value, which is what FP32 arithmetic followed by round-to-nearest-even can guarantee."""
import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle
from kda_testlib import announce, assert_within_one_ulp

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _dev_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _host_f64(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _run(kda, core, gate_bits, w_bits, eps, out=None):
    c = torch.from_numpy(np.ascontiguousarray(core, dtype=np.float32)).cuda()
    got = kda.kda_gated_rmsnorm(c, _dev_bits(gate_bits), _dev_bits(w_bits), eps, out=out)
    torch.cuda.synchronize()
    return oracle.bf16_to_f64(_host_f64(got))


@pytest.mark.parametrize("rows,heads,scale", [(37, 3, 1.0), (1, 1, 1e-3), (5, 32, 1e3), (64, 32, 1.0)])
def test_gated_rmsnorm_matches_oracle(device, rows, heads, scale):
    import kda_gated_delta_core_amd as kda
    announce(f"kda_gated_rmsnorm rows={rows} heads={heads} scale={scale}")
    x = ki.norm_inputs(900 + rows, rows, heads)
    core = x["core"] * np.float32(scale)
    got = _run(kda, core, x["out_gate"], x["o_norm"], ki.NORM_EPS)
    assert_within_one_ulp("norm", got, oracle.gated_rmsnorm(core, x["out_gate"], x["o_norm"], ki.NORM_EPS))


def test_gated_rmsnorm_edges(device):
    """Zero vectors, magnitudes near the ends of the FP32 range, saturated gates, negative weights,
    a large eps."""
    import kda_gated_delta_core_amd as kda
    announce("kda_gated_rmsnorm edges")
    rows, heads = 6, 4
    x = ki.norm_inputs(950, rows, heads)
    core = x["core"].copy()
    core[0, 0] = 0.0
    core[1, 1] *= np.float32(1e30)
    core[2, 2] *= np.float32(1e-30)
    core[3, 3, :64] = 0.0
    core[4, 0] = np.float32(3.0e38)
    gate = x["out_gate"].copy()
    gate[5, :, :16] = 0x7F80    # +inf: sigmoid 1
    gate[5, :, 16:32] = 0xFF80  # -inf: sigmoid 0
    gate[5, :, 32:48] = ki.to_bf16_bits(np.float32(80.0))
    gate[5, :, 48:64] = ki.to_bf16_bits(np.float32(-80.0))
    w = x["o_norm"].copy()
    w[:8] = ki.to_bf16_bits(-np.abs(oracle.bf16_to_f64(w[:8])).astype(np.float32))
    for eps in (ki.NORM_EPS, 0.5):
        got = _run(kda, core, gate, w, eps)
        assert_within_one_ulp(f"edges eps={eps}", got, oracle.gated_rmsnorm(core, gate, w, eps))


def test_gated_rmsnorm_full_size_and_no_write_past_out(device):
    """The T=8192 H=32 workload in full, written into the head of a larger sentinel-filled buffer."""
    import kda_gated_delta_core_amd as kda
    rows, heads, seed = ki.NORM_WORKLOADS["gated_rmsnorm_t8192_h32"]
    announce(f"kda_gated_rmsnorm full size rows={rows} heads={heads}")
    x = ki.norm_inputs(seed, rows, heads)
    big = torch.full((rows + 3, heads, D), 7.0, dtype=torch.bfloat16, device="cuda")
    got = _run(kda, x["core"], x["out_gate"], x["o_norm"], ki.NORM_EPS, out=big[:rows])
    assert torch.all(big[rows:] == 7.0)
    assert_within_one_ulp("full size", got, oracle.gated_rmsnorm(x["core"], x["out_gate"], x["o_norm"], ki.NORM_EPS))


def test_prefill_then_gated_rmsnorm(device):
    """The block's order: chunked prefill, then the gated RMSNorm of its output rows < T.  Each
    stage is held to its own bar: the core to the core tolerance against the oracle's core, the
    norm to one BF16 ulp against the oracle's norm of the core the GPU produced (the norm
    magnifies the core's absolute FP32 error on small elements, so the oracle's norm of the
    oracle's core is not a one-ulp target)."""
    import kda_gated_delta_core_amd as kda
    from kda_testlib import assert_close
    B, H, T, C = 1, 4, 150, 64
    announce(f"kda_chunk_prefill + kda_gated_rmsnorm B={B} H={H} T={T}")
    t_pad = -(-T // C) * C
    x = ki.make_batch(960, B, H, T, -5.0, 0.02, alloc_rows=t_pad, pad_value=0.0)
    d = {n: torch.from_numpy(a).cuda() for n, a in x.items()}
    st = d["state"].clone()
    core = kda.kda_chunk_prefill(d["q"], d["k"], d["v"], d["gate"], d["beta"], st, T, C)
    nx = ki.norm_inputs(961, T, H)
    y = kda.kda_gated_rmsnorm(core[0, :T].contiguous(), _dev_bits(nx["out_gate"]), _dev_bits(nx["o_norm"]),
                              ki.NORM_EPS)
    torch.cuda.synchronize()
    core_gpu = core[0, :T].cpu().numpy()
    o_ref = oracle.serial(x["q"], x["k"], x["v"], x["gate"], x["beta"], x["state"], T=T)[0]
    assert_close("prefill core", core_gpu[None], o_ref[:, :T])
    got = oracle.bf16_to_f64(_host_f64(y))
    assert_within_one_ulp("prefill + norm", got,
                          oracle.gated_rmsnorm(core_gpu, nx["out_gate"], nx["o_norm"], ki.NORM_EPS))
