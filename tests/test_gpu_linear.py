"""nvfp4_linear (quantize + GEMM in one call) against the oracle and against the two-call path.

For few tokens the call is one kernel: its first workgroups encode the activations and the
others multiply them as soon as the encoding is published; its codes, scales, g and Y must
equal nvfp4_quantize followed by nvfp4_gemm bit for bit (the same product kernel and the
same order of sums), and the oracle within the GEMM tolerance."""
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


@pytest.mark.parametrize("M,K,N", [(1, 512, 64), (7, 2048, 300), (16, 1024, 512), (3, 8192, 128), (16, 640, 96),
                                   # k-steps that do not fill every wavefront (dead k-steps read zero): 23 over
                                   # 8 x 3, 39 over 8 x 5; one wavefront per k-step below 8
                                   (5, 2944, 200), (16, 4992, 5120), (2, 384, 33),
                                   # K above the one-workgroup-per-row-block limit: quantize + tiled product
                                   (9, 9216, 256),
                                   # degenerate layers: one output column, one token, one k-step; past 16
                                   # tokens the tiled product with a single (ragged) column tile
                                   (1, 128, 1), (16, 128, 1), (1, 128, 17), (17, 128, 1), (300, 256, 1),
                                   (33, 128, 5)])
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
    own freshly encoded activations, and the publication counters must be back at zero after each call."""
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
    """The few-token kernel's product workgroups wait for the encoder workgroups to publish the
    activations' encoding; with a poll bound of zero each of them encodes everything itself (the
    same bytes). Same bits either way, also with the workspace reused by a second call."""
    monkeypatch.setenv("NVFP4_AMAX_POLLS", "0")
    if shape == "decode":
        wl = workloads.make_decode()
        _check(wl.x, "bf16", wl.w, "bf16", "decode, amax fallback", calls=2)
    else:
        x = workloads.random_matrix(1301, 3, 2048, dtype="bf16")
        w = workloads.random_matrix(1302, 300, 2048, 0.05, dtype="bf16")
        _check(x, "bf16", [w], "bf16", "3x2048x300, amax fallback", calls=2)


@pytest.mark.parametrize("M", [4, 16, 64])
def test_side_stream(M):
    """The conveniences on a stream other than the current one: the workspace and g are allocated and
    filled on that stream, after the current stream's work, so the results equal the same calls on the
    current stream (few tokens: the one-kernel path with its zero-filled workspace)."""
    say(f"linear/gemm on a side stream: M={M} K=1024 N=320")
    x = workloads.random_matrix(1200 + M, M, 1024, dtype="bf16")
    w = workloads.random_matrix(1300 + M, 320, 1024, 0.05, dtype="bf16")
    xd = to_dev(x, "bf16")
    pw = nv.PackedWeight([nv.quantize(to_dev(w, "bf16"))], 1024)
    y0, c0, s0, g0 = nv.linear(xd, pw)
    y0g = nv.gemm(c0, s0, g0, pw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for _ in range(3):
        y1, c1, s1, g1 = nv.linear(xd, pw, stream=side)
        y1g = nv.gemm(c1, s1, g1, pw, stream=side)
        y1h, _, _, _ = nv.linear(xd, pw, g=1.0, stream=side.cuda_stream)   # raw handle, given g
        side.synchronize()
        assert torch.equal(c1, c0) and torch.equal(s1, s0) and torch.equal(g1, g0)
        assert torch.equal(y1, y0) and torch.equal(y1g, y0g)
    y2, _, _, _ = nv.linear(xd, pw, g=1.0)
    torch.cuda.synchronize()
    assert torch.equal(y1h, y2)


def test_workspace_shared_across_token_counts():
    """One workspace for calls with many tokens (two launches: amax partials in the workspace) and few
    tokens (one launch: counters in the workspace), interleaved: the partials never touch the counters,
    so every call equals the same call with a fresh workspace."""
    say("linear: one workspace for M = 300, 16, 40, 3, 16")
    K, N = 1024, 320
    w = workloads.random_matrix(1401, N, K, 0.05, dtype="bf16")
    pw = nv.PackedWeight([nv.quantize(to_dev(w, "bf16"))], K)
    shared = torch.zeros((nv.nvfp4_linear_workspace_bytes(300, nv.NVFP4_IN_BF16, pw.desc),), dtype=torch.uint8,
                         device=DEV)
    for i, M in enumerate([300, 16, 40, 3, 16]):
        xd = to_dev(workloads.random_matrix(1410 + i, M, K, dtype="bf16"), "bf16")
        assert nv.nvfp4_linear_workspace_bytes(M, nv.NVFP4_IN_BF16, pw.desc) <= shared.numel()
        y, c, s, g = nv.linear(xd, pw, shared)
        y2, c2, s2, g2 = nv.linear(xd, pw)          # fresh zeroed workspace
        torch.cuda.synchronize()
        assert torch.equal(c, c2) and torch.equal(s, s2) and torch.equal(g, g2), f"call {i} M={M}"
        assert torch.equal(y, y2), f"call {i} M={M}"


def test_graph_replays_with_changing_inputs():
    """The one-launch decode layer captured in a HIP graph and replayed on activations of very different
    magnitude copied into the captured input between replays: each replay equals the eager call on that
    input (codes, scales, g and Y), so no replay reads records an earlier launch published."""
    wl = workloads.make_decode()
    pw = nv.PackedWeight([nv.quantize(to_dev(wl.w[0], "bf16"))], wl.K)
    xs = [to_dev(workloads.random_matrix(2300 + i, wl.M, wl.K, sc, dtype="bf16"), "bf16")
          for i, sc in enumerate((1.0, 1e-3, 40.0))]
    wsp = nv.linear_workspace(wl.M, torch.bfloat16, pw)
    xd = torch.empty_like(xs[0])

    def outs():
        return (*nv.empty_quantized(wl.M, wl.K), torch.empty((wl.M, wl.N), dtype=torch.float32, device=DEV))

    def step(o, s=None):
        nv.nvfp4_linear(xd, o[0], o[1], o[2], pw.desc, o[3], wsp, stream=s)

    say("linear graph replays on changing inputs: eager outputs")
    want = []
    for x in xs:
        xd.copy_(x)
        o = outs()
        step(o)
        torch.cuda.synchronize()
        want.append(o)
    got = outs()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step(got, s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step(got, s)
    for rep in range(6):
        i = (rep * 2) % 3
        xd.copy_(xs[i])
        for t in got:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b, what in zip(got, want[i], ("codes", "scales", "g", "y")):
            assert torch.equal(a, b), f"replay {rep} (input {i}): {what} differs from the eager call"
        step(outs())                        # an eager call between replays shares the workspace
