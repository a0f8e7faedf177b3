"""bf16 output of the product (nvfp4_gemm_ex / nvfp4_linear_ex): every element must be the
round-to-nearest-even bf16 of the FP32 element the same call writes with FP32 output (torch's
FP32 -> bf16 cast rounds the same way), and within the product's bound plus half a bf16 ulp of
the FP64 oracle."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_03_amd as nv
import workloads
from gpu_util import DEV, host, say, to_dev
from oracle import nvfp4_ref as ref

pytestmark = pytest.mark.gpu


def _case(M, N, K, seed):
    x = workloads.random_matrix(seed, M, K, 1.0, "bf16")
    w = [workloads.random_matrix(seed + 1, N // 2, K, 0.02, "bf16"),
         workloads.random_matrix(seed + 2, N - N // 2, K, 0.5, "bf16")]     # two modules, own g each
    return x, w


def _check_vs_oracle(y_bf16, x, w, what):
    y_ref, a_ref = ref.gemm(ref.quantize(x), [ref.quantize(m) for m in w])
    got = host(y_bf16.float()).astype(np.float64)
    bound = ref.GEMM_RTOL * a_ref + 2.0 ** -8 * np.abs(y_ref) + 1e-30
    worst = float(np.max(np.abs(got - y_ref) / bound))
    assert worst <= 1.0, f"{what}: worst |dy| / bound = {worst:.3f}"


@pytest.mark.parametrize("M", [1, 5, 16, 160, 1000])
def test_gemm_bf16(M):
    N, K = 640, 1024
    x, w = _case(M, N, K, 900 + M)
    say(f"bf16 out: gemm M={M} N={N} K={K}")
    xq = nv.quantize(to_dev(x, "bf16"))
    pw = nv.PackedWeight([nv.quantize(to_dev(m, "bf16")) for m in w], K)
    y32 = nv.gemm(*xq, pw)
    y16 = nv.gemm(*xq, pw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert y16.dtype == torch.bfloat16
    assert torch.equal(y16, y32.to(torch.bfloat16)), "bf16 Y is not the RNE of the FP32 Y"
    _check_vs_oracle(y16, x, w, f"gemm M={M}")


@pytest.mark.parametrize("M", [16, 300])
def test_linear_bf16_strided(M):
    """Quantize + product in one call, into a bf16 Y with a row stride of N + 3 elements (odd, so rows start
    on 2-byte boundaries only)."""
    N, K = 384, 512
    x, w = _case(M, N, K, 950 + M)
    say(f"bf16 out: linear M={M}, ld_y = N + 3")
    pw = nv.PackedWeight([nv.quantize(to_dev(m, "bf16")) for m in w], K)
    xd = to_dev(x, "bf16")
    y32, *_ = nv.linear(xd, pw)
    big = torch.full((M, N + 3), 7.0, dtype=torch.bfloat16, device=DEV)
    y16 = big[:, :N]
    ws = nv.linear_workspace(M, xd.dtype, pw, DEV)
    codes, scales, g = nv.empty_quantized(M, K, DEV)
    nv.nvfp4_linear(xd, codes, scales, g, pw.desc, y16, ws)
    torch.cuda.synchronize()
    assert torch.equal(y16, y32.to(torch.bfloat16))
    assert torch.all(big[:, N:] == 7.0), "wrote past the row"
    _check_vs_oracle(y16, x, w, f"linear M={M}")


@pytest.mark.parametrize("M", [16, 160])
def test_gated_bf16(M):
    """The GDN projection with gates and bf16 output: the RNE of the gated FP32 output."""
    wl = workloads.make_gdn(M=M)
    gp = workloads.gdn_gate_params()
    gates = nv.GdnGates(gp.a_col, gp.n_a, gp.b_col, gp.n_b, torch.from_numpy(gp.a_log).to(DEV),
                        torch.from_numpy(gp.dt_bias).to(DEV))
    say(f"bf16 out: gated gdn projection M={M}")
    pw = nv.PackedWeight([nv.quantize(to_dev(workloads.to_bf16_values(m), "bf16")) for m in wl.w], wl.K)
    x = to_dev(wl.x, "bf16")
    y32, *_ = nv.linear(x, pw, gates=gates)
    y16, *_ = nv.linear(x, pw, gates=gates, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y16, y32.to(torch.bfloat16))


def test_bf16_graph_replays():
    """The few-token bf16 linear call captured in a HIP graph: every replay equals the eager call."""
    N, K = 640, 1024
    x, w = _case(16, N, K, 990)
    pw = nv.PackedWeight([nv.quantize(to_dev(m, "bf16")) for m in w], K)
    xd = to_dev(x, "bf16")
    ws = nv.linear_workspace(16, xd.dtype, pw, DEV)
    codes, scales, g = nv.empty_quantized(16, K, DEV)
    y = torch.empty((16, N), dtype=torch.bfloat16, device=DEV)
    say("bf16 out: graph replays")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        nv.nvfp4_linear(xd, codes, scales, g, pw.desc, y, ws, stream=s)
    torch.cuda.synchronize()
    eager = y.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        nv.nvfp4_linear(xd, codes, scales, g, pw.desc, y, ws, stream=s)
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager)
