"""GDN gate epilogue on the GPU against the FP64 oracle (``oracle.gdn_gates``).

The fused GDN projection (q, k, v, z, a, b) is multiplied with and without the epilogue:
the columns outside the two gate modules must keep the plain product's bits, and the gate
columns must match the oracle's gates of the oracle's product within the bound derived in
``gdn_gates.gates_tolerance`` (the product's own bound carried through each gate's
derivative, plus the FP32 evaluation of the gate)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_03_amd as nv
import workloads
from gpu_util import DEV, host, say, to_dev
from oracle import gdn_gates as gates_ref
from oracle import nvfp4_ref as ref

pytestmark = pytest.mark.gpu


def _setup(M, dt_bias=None, a_scale=1.0):
    wl = workloads.make_gdn(M=M)
    ws = [w * np.float32(a_scale) if name == "a" else w for w, name in zip(wl.w, wl.module_names)]
    ws = [workloads.to_bf16_values(w) for w in ws]
    gp = workloads.gdn_gate_params()
    if dt_bias is not None:
        gp.dt_bias = np.asarray(dt_bias, np.float32)
    gates = nv.GdnGates(gp.a_col, gp.n_a, gp.b_col, gp.n_b, torch.from_numpy(gp.a_log).to(DEV),
                        torch.from_numpy(gp.dt_bias).to(DEV))
    mods = [nv.quantize(to_dev(w, "bf16")) for w in ws]
    pw = nv.PackedWeight(mods, wl.K)
    return wl, ws, gp, gates, pw


def _oracle_gate_columns(x, ws, gp, names):
    """Oracle product and gates on the gate columns only: the a and b modules, each quantized with its own
    global scale, against the activations' quantization."""
    xq = ref.quantize(x, "compute")
    wa = ref.dequantize(ref.quantize(ws[names.index("a")]))
    wb = ref.dequantize(ref.quantize(ws[names.index("b")]))
    y, a = ref.gemm_dequantized(ref.dequantize(xq), np.concatenate([wa, wb]))
    la, lb = 0, gp.b_col - gp.a_col          # the two modules are adjacent
    args = (la, gp.n_a, lb, gp.n_b, gp.a_log.astype(np.float64), gp.dt_bias.astype(np.float64))
    cols = np.arange(gp.a_col, gp.b_col + gp.n_b)
    return cols, gates_ref.apply_gates(y, *args), gates_ref.gates_tolerance(y, a, *args)


def _check(y_gated, y_plain, x, ws, gp, what, names=("q", "k", "v", "z", "a", "b")):
    yg, yp = host(y_gated), host(y_plain)
    keep = np.ones(yg.shape[1], bool)
    keep[gp.a_col:gp.a_col + gp.n_a] = False
    keep[gp.b_col:gp.b_col + gp.n_b] = False
    assert np.array_equal(yg[:, keep], yp[:, keep]), f"{what}: ungated columns changed"
    cols, out, tol = _oracle_gate_columns(x, ws, gp, list(names))
    ok, worst = gates_ref.within(yg[:, cols], out, tol)
    assert ok, f"{what}: worst |d gate| / bound = {worst:.3f}"
    a = yg[:, gp.a_col:gp.a_col + gp.n_a]
    b = yg[:, gp.b_col:gp.b_col + gp.n_b]
    assert np.all((a >= 0) & (a <= 1)), f"{what}: decay outside [0, 1]"
    assert np.all((b >= 0) & (b <= 1)), f"{what}: write strength outside [0, 1]"


@pytest.mark.parametrize("M", [160, 1000])
def test_gemm_gated_tiles(M):
    wl, ws, gp, gates, pw = _setup(M)
    say(f"gates: gemm, tiled, M={M}")
    xc, xs, gx = nv.quantize(to_dev(wl.x, "bf16"))
    y_plain = nv.gemm(xc, xs, gx, pw)
    y_gated = nv.gemm(xc, xs, gx, pw, gates=gates)
    torch.cuda.synchronize()
    _check(y_gated, y_plain, wl.x, ws, gp, f"tiled M={M}")


@pytest.mark.parametrize("M", [1, 5, 16])
def test_gemm_gated_few_tokens(M):
    wl, ws, gp, gates, pw = _setup(M)
    say(f"gates: gemm, few tokens, M={M}")
    xc, xs, gx = nv.quantize(to_dev(wl.x, "bf16"))
    y_plain = nv.gemm(xc, xs, gx, pw)
    y_gated = nv.gemm(xc, xs, gx, pw, gates=gates)
    torch.cuda.synchronize()
    _check(y_gated, y_plain, wl.x, ws, gp, f"few tokens M={M}")


@pytest.mark.parametrize("M", [16, 300])
def test_linear_gated(M):
    """Quantize + product + gates in one call (one kernel for 16 tokens)."""
    wl, ws, gp, gates, pw = _setup(M)
    say(f"gates: linear M={M}")
    x = to_dev(wl.x, "bf16")
    y_plain, c0, s0, g0 = nv.linear(x, pw)
    y_gated, c1, s1, g1 = nv.linear(x, pw, gates=gates)
    torch.cuda.synchronize()
    assert torch.equal(c0, c1) and torch.equal(s0, s1) and torch.equal(g0, g1)
    _check(y_gated, y_plain, wl.x, ws, gp, f"linear M={M}")


def test_gates_both_branches():
    """Biases of +-30 and a strongly scaled decay projection put the softplus argument and the sigmoid
    input far on both sides of zero (decay near 0 and near 1, write strength near 0 and near 1)."""
    dt = np.where(np.arange(48) % 2 == 0, -30.0, 30.0).astype(np.float32)
    wl, ws, gp, gates, pw = _setup(64, dt_bias=dt, a_scale=50.0)
    say("gates: saturated branches, M=64")
    xc, xs, gx = nv.quantize(to_dev(wl.x, "bf16"))
    y_plain = nv.gemm(xc, xs, gx, pw)
    y_gated = nv.gemm(xc, xs, gx, pw, gates=gates)
    torch.cuda.synchronize()
    _check(y_gated, y_plain, wl.x, ws, gp, "saturated")
    a = host(y_gated)[:, gp.a_col:gp.a_col + gp.n_a]
    assert a.min() < 1e-6 and a.max() > 0.999


def test_gated_graph_replays_match_eager():
    """The gated few-token linear call captured in a HIP graph: every replay equals the eager call."""
    wl, ws, gp, gates, pw = _setup(16)
    say("gates: graph replays, M=16")
    x = to_dev(wl.x, "bf16")
    ws_t = nv.linear_workspace(16, x.dtype, pw, DEV)
    codes, scales, g = nv.empty_quantized(16, wl.K, DEV)
    y = torch.empty((16, wl.N), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        nv.nvfp4_linear(x, codes, scales, g, pw.desc, y, ws_t, stream=s, gates=gates)
    torch.cuda.synchronize()
    eager = y.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        nv.nvfp4_linear(x, codes, scales, g, pw.desc, y, ws_t, stream=s, gates=gates)
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager)
