"""nvfp4_linear_noalloc (the library's static scratch instead of a workspace) against nvfp4_linear:
the same codes, scales, g and Y bit for bit, on two calls in a row, the second with a smaller input,
for the one-launch few-token path (counters in the scratch) and the two-launch path (amax partials
in the scratch).  Runs last: the scratch persists for the process, as it would for a caller."""
import pytest
import torch

import nvfp4_block_scaled_03_amd as nv
import workloads
from gpu_util import DEV, say, to_dev

pytestmark = pytest.mark.gpu


def _pair(M, K, N, seed, g_mode):
    x = to_dev(workloads.random_matrix(seed, M, K, dtype="bf16"), "bf16")
    w = to_dev(workloads.random_matrix(seed + 1, N, K, 0.05, dtype="bf16"), "bf16")
    return x, nv.PackedWeight([nv.quantize(w)], K)


def _both(x, pw, g_mode):
    M, K = x.shape
    ref_out = nv.empty_quantized(M, K)
    got_out = nv.empty_quantized(M, K)
    for c, s, g in (ref_out, got_out):
        c.fill_(0x5A)
        s.fill_(0xA5)
        g.fill_(1.0 if g_mode == nv.NVFP4_G_GIVEN else -7.0)
    y_ref = torch.full((M, pw.n), float("nan"), dtype=torch.float32, device=DEV)
    y_got = torch.full((M, pw.n), float("nan"), dtype=torch.float32, device=DEV)
    ws = nv.linear_workspace(M, x.dtype, pw)
    nv.nvfp4_linear(x, *ref_out, pw.desc, y_ref, ws, g_mode)
    nv.nvfp4_linear_noalloc(x, *got_out, pw.desc, y_got, g_mode)
    torch.cuda.synchronize()
    for a, b in zip(ref_out, got_out):
        assert torch.equal(a, b)
    assert torch.equal(y_ref, y_got)


@pytest.mark.parametrize("g_mode", [nv.NVFP4_G_COMPUTE, nv.NVFP4_G_GIVEN])
@pytest.mark.parametrize("first,second", [((16, 5120, 5120), (3, 2048, 300)),     # few tokens, then fewer
                                          ((300, 1024, 512), (40, 512, 200))])      # two launches, then smaller
def test_noalloc_matches_linear(first, second, g_mode):
    for i, (M, K, N) in enumerate((first, second)):
        say(f"nvfp4_linear_noalloc call {i}: M={M} K={K} N={N} g_mode={g_mode}")
        x, pw = _pair(M, K, N, 4000 + 10 * i + M, g_mode)
        _both(x, pw, g_mode)


def test_noalloc_graph_capture():
    """Inside a captured graph (the caller that cannot allocate): replays equal eager calls."""
    say("nvfp4_linear_noalloc under graph capture: M=16 K=5120 N=5120")
    x, pw = _pair(16, 5120, 5120, 4100, nv.NVFP4_G_COMPUTE)
    c, s, g = nv.empty_quantized(16, 5120)
    y = torch.empty((16, 5120), dtype=torch.float32, device=DEV)
    nv.nvfp4_linear_noalloc(x, c, s, g, pw.desc, y)
    torch.cuda.synchronize()
    want = y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        nv.nvfp4_linear_noalloc(x, c, s, g, pw.desc, y)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        nv.nvfp4_linear_noalloc(x, c, s, g, pw.desc, y)
    torch.cuda.synchronize()
    for i in range(4):
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want), f"replay {i}"
        nv.nvfp4_linear_noalloc(x, c, s, g, pw.desc, y)   # an eager call between replays shares the scratch
        torch.cuda.synchronize()
        assert torch.equal(y, want)
