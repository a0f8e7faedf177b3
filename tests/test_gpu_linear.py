"""nvfp4_linear (quantize + GEMM in one call) against the oracle and against the two-call path.

For few tokens the call is an amax pass plus one kernel that quantizes each K-slice of the
activations and takes the split-K product; its codes, scales, g and Y must equal
nvfp4_quantize followed by nvfp4_gemm bit for bit (the same k-slices, summed in the same
slice order), and the oracle within the GEMM tolerance."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_03_amd as nv
import workloads
from gpu_util import DEV, assert_quant_equal, host, say, to_dev
from oracle import nvfp4_ref as ref

pytestmark = pytest.mark.gpu


def _two_call(xd, pw, g=None):
    c, s, gx = nv.quantize(xd, g=g)
    return nv.gemm(c, s, gx, pw), c, s, gx


def _check(x, x_dtype, ws, w_dtype, what, g=None, calls=3):
    say(f"linear: {what} M={x.shape[0]} K={x.shape[1]} N={sum(w.shape[0] for w in ws)} {x_dtype}")
    xd = to_dev(x, x_dtype)
    mods = [nv.quantize(to_dev(w, w_dtype)) for w in ws]
    pw = nv.PackedWeight(mods, x.shape[1])
    wsp = nv.linear_workspace(x.shape[0], xd.dtype, pw)
    outs = [nv.linear(xd, pw, wsp, g=g) for _ in range(calls)]      # workspace reused across calls
    y2, c2, s2, g2 = _two_call(xd, pw, g)
    torch.cuda.synchronize()
    for y, c, s, gx in outs:
        assert torch.equal(c, c2) and torch.equal(s, s2) and torch.equal(gx, g2)
        assert torch.equal(y, y2), f"{what}: fused Y differs from the two-call path"
    xq = ref.quantize(x) if g is None else ref.quantize(x, "given", g)
    wq = [ref.quantize(w) for w in ws]
    assert_quant_equal(outs[0][1], outs[0][2], outs[0][3], xq, what=f"{what} X")
    y_ref, a_ref = ref.gemm(xq, wq)
    ok, worst = ref.gemm_within_tolerance(host(outs[0][0]), y_ref, a_ref)
    assert ok, f"{what}: worst |dy|/sum|terms| = {worst:.3e}"


def test_decode_workload():
    wl = workloads.make_decode()
    _check(wl.x, "bf16", wl.w, "bf16", "decode")


@pytest.mark.parametrize("M,K,N", [(1, 512, 64), (7, 2048, 300), (16, 1024, 512), (3, 8192, 128), (16, 640, 96)])
def test_shapes(M, K, N):
    x = workloads.random_matrix(700 + M, M, K, dtype="bf16")
    w = workloads.random_matrix(800 + M, N, K, 0.05, dtype="bf16")
    _check(x, "bf16", [w], "bf16", f"shape {M}x{K}x{N}")


def test_fp32_input_and_fused_modules():
    wl = workloads.make_tiny()
    x = wl.x[:9]
    ws = [workloads.random_matrix(900 + i, r, 512, s) for i, (r, s) in enumerate([(100, 0.02), (37, 0.2), (48, 0.002)])]
    _check(x, "f32", ws, "f32", "f32 fused modules")


def test_given_scale():
    wl = workloads.make_ngpt(M=16)
    _check(wl.x, "bf16", [wl.w[0][:1024]], "bf16", "ngpt g=1", g=1.0)


def test_falls_back_beyond_skinny():
    x = workloads.random_matrix(1001, 40, 512, dtype="bf16")
    w = workloads.random_matrix(1002, 200, 512, 0.05, dtype="bf16")
    _check(x, "bf16", [w], "bf16", "M=40 (two launches)", calls=1)


def test_graph_replays():
    wl = workloads.make_decode()
    say("linear graph replays")
    xd = to_dev(wl.x, "bf16")
    pw = nv.PackedWeight([nv.quantize(to_dev(wl.w[0], "bf16"))], wl.K)
    wsp = nv.linear_workspace(wl.M, xd.dtype, pw)
    codes, scales, g = nv.empty_quantized(wl.M, wl.K)
    y = torch.empty((wl.M, wl.N), dtype=torch.float32, device=DEV)

    def step():
        nv.nvfp4_linear(xd, codes, scales, g, pw.desc, y, wsp)

    step()
    torch.cuda.synchronize()
    want = y.clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
        step()
    torch.cuda.synchronize()
    for i in range(5):
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want), f"replay {i}"
        step()                                   # eager call between replays shares the workspace
    torch.cuda.synchronize()
    assert torch.equal(y, want)


def test_alternating_inputs_see_fresh_codes():
    """Consecutive calls with different activations into the same code buffers: every call must use its
    own freshly encoded activations, and the split-K counters must be back at zero after each call."""
    wl = workloads.make_decode()
    say("linear alternating inputs")
    xs = [to_dev(wl.x, "bf16"), to_dev(workloads.random_matrix(1234, wl.M, wl.K, 3.0, dtype="bf16"), "bf16")]
    pw = nv.PackedWeight([nv.quantize(to_dev(wl.w[0], "bf16"))], wl.K)
    wsp = nv.linear_workspace(wl.M, torch.bfloat16, pw)
    want = [_two_call(x, pw)[0] for x in xs]
    codes, scales, g = nv.empty_quantized(wl.M, wl.K)
    y = torch.empty((wl.M, wl.N), dtype=torch.float32, device=DEV)
    outs = []
    for i in range(8):
        nv.nvfp4_linear(xs[i % 2], codes, scales, g, pw.desc, y, wsp)
        outs.append(y.clone())
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, want[i % 2]), f"call {i}"


@pytest.mark.parametrize("shape", ["decode", "3x2048x300"])
def test_amax_fallback_when_peers_do_not_publish(shape, monkeypatch):
    """The few-token kernel takes the global amax from the slice maxima its peer workgroups publish;
    with a poll bound of zero every workgroup reduces all slices itself. Same bits either way."""
    monkeypatch.setenv("NVFP4_AMAX_POLLS", "0")
    if shape == "decode":
        wl = workloads.make_decode()
        _check(wl.x, "bf16", wl.w, "bf16", "decode, amax fallback", calls=2)
    else:
        x = workloads.random_matrix(1301, 3, 2048, dtype="bf16")
        w = workloads.random_matrix(1302, 300, 2048, 0.05, dtype="bf16")
        _check(x, "bf16", [w], "bf16", "3x2048x300, amax fallback", calls=2)
