"""Block-scaled GEMM parity on the GPU against the FP64 oracle.

Each output must satisfy |y_gpu - y_ref| <= 1e-5 * sum_k |x^[m,k] w^[n,k]| (the FP32
accumulation-order error scale), where the oracle quantizes both operands itself
(its codes are checked bit-for-bit against the GPU's in the same test).  Small
shapes are compared element by element; the full-size workloads on sampled
row x column blocks that include every module boundary and the ragged tail."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_03_amd as nv
import workloads
from gpu_util import DEV, assert_quant_equal, host, oracle_quantize_rows, say, to_dev
from oracle import nvfp4_ref as ref

pytestmark = pytest.mark.gpu
F32 = np.float32


def gpu_linear(x, x_dtype, ws, w_dtype, g_x=None, g_w=None):
    xd = to_dev(x, x_dtype)
    xc, xs, gx = nv.quantize(xd, g=g_x)
    mods = [nv.quantize(to_dev(w, w_dtype), g=g_w) for w in ws]
    pw = nv.PackedWeight(mods, x.shape[1])
    y = nv.gemm(xc, xs, gx, pw)
    torch.cuda.synchronize()
    return y, (xc, xs, gx), mods, pw


def check_dense(x, x_dtype, ws, w_dtype, what, g_x=None, g_w=None):
    say(f"gemm parity (dense): {what} M={x.shape[0]} K={x.shape[1]} modules={[w.shape[0] for w in ws]}")
    y, (xc, xs, gx), mods, _ = gpu_linear(x, x_dtype, ws, w_dtype, g_x, g_w)
    mode = "compute" if g_x is None else "given"
    xq = ref.quantize(x, mode, g_x)
    wq = [ref.quantize(w, "compute" if g_w is None else "given", g_w) for w in ws]
    assert_quant_equal(xc, xs, gx, xq, what=f"{what} X")
    for i, (m, q) in enumerate(zip(mods, wq)):
        assert_quant_equal(*m, q, what=f"{what} W[{i}]")
    y_ref, a_ref = ref.gemm(xq, wq)
    ok, worst = ref.gemm_within_tolerance(host(y), y_ref, a_ref)
    assert ok, f"{what}: worst |dy|/sum|terms| = {worst:.3e}"
    return y


def test_tiny_workload():
    wl = workloads.make_tiny()
    check_dense(wl.x, "f32", wl.w, "f32", "tiny")


def test_decode_workload():
    wl = workloads.make_decode()
    check_dense(wl.x, "bf16", wl.w, "bf16", "decode")


@pytest.mark.parametrize("M", [1, 2, 5, 15, 16])
def test_skinny_shapes(M):
    x = workloads.random_matrix(100 + M, M, 384, dtype="bf16")
    ws = [workloads.random_matrix(200 + M, 300, 384, 0.05, dtype="bf16")]
    check_dense(x, "bf16", ws, "bf16", f"skinny M={M}")


@pytest.mark.parametrize("M", [17, 33, 128, 300])
def test_tiled_ragged_fused(M):
    x = workloads.random_matrix(300 + M, M, 640, dtype="bf16")
    ws = [workloads.random_matrix(400 + i, r, 640, s, dtype="bf16")
          for i, (r, s) in enumerate([(100, 0.02), (37, 0.2), (48, 0.002)])]
    check_dense(x, "bf16", ws, "bf16", f"tiled fused M={M}")


@pytest.mark.parametrize("M", [5, 40])
def test_most_modules(M):
    """The most sub-modules one packed weight holds (16), several of a single row, each with its own
    global scale (weight scales spread over five decades), on the few-token and the tiled product:
    every module boundary, including ones inside a 16-row block and inside a column tile."""
    rows = [1, 2, 3, 1, 16, 17, 1, 5, 31, 33, 1, 64, 1, 7, 2, 1]
    x = workloads.random_matrix(1600 + M, M, 512, dtype="bf16")
    ws = [workloads.random_matrix(1700 + i, r, 512, 10.0 ** (-4 + (i % 5)), dtype="bf16")
          for i, r in enumerate(rows)]
    check_dense(x, "bf16", ws, "bf16", f"16 modules M={M}")


@pytest.mark.parametrize("M,K", [(40, 128), (260, 128), (260, 256), (260, 384), (40, 896)])
def test_tiled_short_and_odd_k(M, K):
    """k-step counts of 1, 2, 3 and 7: the tile kernels' load ring runs past the last k-step."""
    x = workloads.random_matrix(700 + K + M, M, K, dtype="bf16")
    ws = [workloads.random_matrix(800 + K, 300, K, 0.05, dtype="bf16")]
    check_dense(x, "bf16", ws, "bf16", f"tiled M={M} K={K}")


@pytest.mark.parametrize("M,N,K", [(300, 700, 2048), (100, 700, 2048), (300, 700, 640), (160, 1000, 5120),
                                   (1000, 600, 1024)])
def test_medium_shapes(M, N, K):
    """Ragged shapes between the few-token kernel and the big-tile regime (small tiles, partial row and
    column tiles, several k-steps)."""
    x = workloads.random_matrix(900 + M + K, M, K, dtype="bf16")
    ws = [workloads.random_matrix(950 + N + K, N, K, 0.05, dtype="bf16")]
    check_dense(x, "bf16", ws, "bf16", f"medium M={M} N={N} K={K}")


def test_repeat_calls_deterministic():
    """Repeated calls agree bit for bit."""
    x = workloads.random_matrix(990, 160, 5120, dtype="bf16")
    ws = [workloads.random_matrix(991, 1000, 5120, 0.05, dtype="bf16")]
    say("gemm determinism M=160 N=1000 K=5120")
    xc, xs, gx = nv.quantize(to_dev(x, "bf16"))
    pw = nv.PackedWeight([nv.quantize(to_dev(w, "bf16")) for w in ws], 5120)
    ys = [nv.gemm(xc, xs, gx, pw) for _ in range(4)]
    torch.cuda.synchronize()
    for t in ys[1:]:
        assert torch.equal(t, ys[0])


def test_fused_module_mix_skinny():
    x = workloads.random_matrix(501, 7, 512, dtype="bf16")
    ws = [workloads.random_matrix(502 + i, r, 512, s, dtype="bf16")
          for i, (r, s) in enumerate([(64, 0.02), (48, 0.2), (48, 0.002), (16, 3.0)])]
    check_dense(x, "bf16", ws, "bf16", "skinny fused")


def test_gdn_small_m_dense():
    wl = workloads.make_gdn(M=160)
    check_dense(wl.x, "bf16", wl.w, "bf16", "gdn M=160")


def test_ngpt_without_per_tensor_scaling():
    wl = workloads.make_ngpt(M=256)
    check_dense(wl.x, "bf16", [wl.w[0][:512]], "bf16", "ngpt g=1", g_x=1.0, g_w=1.0)


def _boundary_cols(wl):
    cols = [0, wl.N - 1]
    off = 0
    for w in wl.w:
        cols += [off, off + 1, off + w.shape[0] - 2, off + w.shape[0] - 1]
        off += w.shape[0]
    return np.array(sorted(set(c for c in cols if 0 <= c < wl.N)))


@pytest.mark.parametrize("name", ["gdn", "ngpt", "large"])
def test_workload_sampled(name):
    """Full-size workload in the bench launch configuration; sampled rows x columns against the oracle."""
    wl = workloads.make(name)
    say(f"gemm parity (sampled): {name} M={wl.M} K={wl.K} N={wl.N}")
    y, (xc, xs, gx), mods, _ = gpu_linear(wl.x, wl.x_dtype, wl.w, wl.w_dtype)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, wl.M - 1], rng.choice(wl.M, 40, replace=False)]))
    cols = np.unique(np.concatenate([_boundary_cols(wl), rng.choice(wl.N, 200, replace=False)]))
    xq = oracle_quantize_rows(wl.x, rows)
    assert_quant_equal(xc, xs, gx, xq, rows=torch.from_numpy(rows).to(DEV), what=f"{name} X rows")
    # oracle weight rows for the sampled columns, each with its own module's global scale
    off, parts = 0, []
    for w in wl.w:
        r0, r1 = off, off + w.shape[0]
        sel = cols[(cols >= r0) & (cols < r1)] - r0
        if len(sel):
            parts.append(ref.dequantize(oracle_quantize_rows(w, sel)))
        off = r1
    wh = np.concatenate(parts, axis=0)
    xh = ref.dequantize(xq)
    y_ref, a_ref = ref.gemm_dequantized(xh, wh)
    yd = host(y[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)])
    ok, worst = ref.gemm_within_tolerance(yd, y_ref, a_ref)
    assert ok, f"{name}: worst |dy|/sum|terms| = {worst:.3e}"
    say(f"{name}: worst |dy|/sum|terms| = {worst:.3e} over {yd.size} sampled outputs")


def test_fused_equals_per_module():
    """One fused GEMM over stacked sub-modules = the per-module GEMMs side by side, bit for bit (every output
    sums its k-steps in the same order whatever the tile shape and count), and both within the oracle's bound."""
    wl = workloads.make_gdn(M=96)
    say("gemm fused == per-module concat")
    y, (xc, xs, gx), mods, _ = gpu_linear(wl.x, "bf16", wl.w, "bf16")
    parts = [nv.gemm(xc, xs, gx, nv.PackedWeight([m], wl.K)) for m in mods]
    torch.cuda.synchronize()
    assert torch.equal(y, torch.cat(parts, dim=1))
    xq = ref.quantize(wl.x, "compute")
    wq = [ref.quantize(w, "compute") for w in wl.w]
    y_ref, a_ref = ref.gemm(xq, wq)
    ok, worst = ref.gemm_within_tolerance(host(y), y_ref, a_ref)
    assert ok, f"worst |dy|/sum|terms| = {worst:.3e}"


def test_tile_shape_does_not_change_results():
    """8192 rows run on 256 x 256 tiles; their first 256 rows alone run on 128 x 128 tiles.  The rows agree
    bit for bit."""
    x = workloads.random_matrix(1201, 8192, 1024, dtype="bf16")
    ws = [workloads.random_matrix(1202, 4096, 1024, 0.05, dtype="bf16")]
    say("gemm tile shapes: M=8192 vs its first 256 rows, N=4096 K=1024")
    xc, xs, gx = nv.quantize(to_dev(x, "bf16"))
    pw = nv.PackedWeight([nv.quantize(to_dev(w, "bf16")) for w in ws], 1024)
    y_all = nv.gemm(xc, xs, gx, pw)
    y_top = nv.gemm(xc[:256].contiguous(), xs[:256].contiguous(), gx, pw)
    torch.cuda.synchronize()
    assert torch.equal(y_all[:256], y_top)


@pytest.mark.parametrize("M", [1024, 1000])
def test_mixed_tile_split(M):
    """A ragged column edge (16384 + 96 columns, as the fused GDN projection's gate modules leave) at about
    a thousand tokens runs its first 16384 columns on 256 x 256 tiles and the last 96 in a second launch on
    64 x 64 tiles (128 x 128 tiles would occupy only 8 units); 1000 rows also leave ragged row tiles in
    both launches: every output within the oracle's bound, and bit for bit what 128 x 128 tiles alone give."""
    x = workloads.random_matrix(1301, M, 512, dtype="bf16")
    ws = [workloads.random_matrix(1302, 16384, 512, 0.05, dtype="bf16"),
          workloads.random_matrix(1303, 96, 512, 2.0, dtype="bf16")]
    y = check_dense(x, "bf16", ws, "bf16", "mixed tiles")
    xc, xs, gx = nv.quantize(to_dev(x, "bf16"))
    pw = nv.PackedWeight([nv.quantize(to_dev(w, "bf16")) for w in ws], 512)
    y_top = nv.gemm(xc[:128].contiguous(), xs[:128].contiguous(), gx, pw)     # 128 rows: small tiles only
    torch.cuda.synchronize()
    assert torch.equal(y[:128], y_top)


def test_small_tile_shapes_agree():
    """1024 tokens x 4096 columns run on 128 x 128 tiles (256 of them, one round at two per unit); the
    first 128 rows alone make only 32 such tiles and run on 64 x 64 tiles instead: the same sums, bit for
    bit, and every output within the oracle's bound."""
    x = workloads.random_matrix(1311, 1024, 512, dtype="bf16")
    ws = [workloads.random_matrix(1312, 4096, 512, 0.05, dtype="bf16")]
    y = check_dense(x, "bf16", ws, "bf16", "128x128 tiles")
    xc, xs, gx = nv.quantize(to_dev(x, "bf16"))
    pw = nv.PackedWeight([nv.quantize(to_dev(w, "bf16")) for w in ws], 512)
    y_top = nv.gemm(xc[:128].contiguous(), xs[:128].contiguous(), gx, pw)
    torch.cuda.synchronize()
    assert torch.equal(y[:128], y_top)


def test_shared_scale_pitfall_is_detected():
    """Negative control: packing module a's codes with module q's global scale (one scale for a
    fused kernel) corrupts exactly the a columns, and the parity check catches it."""
    wl = workloads.make_gdn(M=64)
    say("gemm pitfall negative control")
    xd = to_dev(wl.x, "bf16")
    xc, xs, gx = nv.quantize(xd)
    q = nv.quantize(to_dev(wl.w[0][:256], "bf16"))
    a = nv.quantize(to_dev(wl.w[4], "bf16"))
    y_bad = nv.gemm(xc, xs, gx, nv.PackedWeight([q, (a[0], a[1], q[2])], wl.K))
    torch.cuda.synchronize()
    xq = ref.quantize(wl.x)
    y_ref, a_ref = ref.gemm(xq, [ref.quantize(wl.w[0][:256]), ref.quantize(wl.w[4])])
    ok_q, _ = ref.gemm_within_tolerance(host(y_bad)[:, :256], y_ref[:, :256], a_ref[:, :256])
    ok_a, worst_a = ref.gemm_within_tolerance(host(y_bad)[:, 256:], y_ref[:, 256:], a_ref[:, 256:])
    assert ok_q and not ok_a and worst_a > 1e-2


def test_unpack_round_trip():
    wl = workloads.make_gdn(M=16)
    say("pack/unpack round trip")
    mods = [nv.quantize(to_dev(w[:200], "bf16")) for w in wl.w]
    pw = nv.PackedWeight(mods, wl.K)
    c, s, cs = pw.unpack()
    torch.cuda.synchronize()
    assert torch.equal(c, torch.cat([m[0] for m in mods]))
    assert torch.equal(s, torch.cat([m[1] for m in mods]))
    want = torch.cat([m[2].expand(m[0].shape[0]) for m in mods])
    assert torch.equal(cs, want)


def test_clone_and_determinism():
    wl = workloads.make_decode()
    say("gemm clone + determinism")
    y, (xc, xs, gx), mods, pw = gpu_linear(wl.x, "bf16", wl.w, "bf16")
    pw2 = pw.clone()
    ys = [nv.gemm(xc, xs, gx, p) for p in (pw, pw2, pw)]
    torch.cuda.synchronize()
    for t in ys:
        assert torch.equal(t, y)


def test_empty_m():
    wl = workloads.make_tiny()
    _, (xc, xs, gx), _, pw = gpu_linear(wl.x, "f32", wl.w, "f32")
    y = torch.full((0, pw.n), 7.0, device=DEV)
    nv.nvfp4_gemm(0, xc, xs, gx, pw.desc, y, pw.n)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,M", [("decode", None), ("gdn", 96)])
def test_graph_replays_match_eager(name, M):
    """Quantize + GEMM captured in a HIP graph: every replay (with eager work in between) equals the eager result."""
    wl = workloads.make(name) if M is None else workloads.make(name, M=M)
    say(f"graph replay vs eager: {name}")
    xd = to_dev(wl.x, "bf16")
    mods = [nv.quantize(to_dev(w, "bf16")) for w in wl.w]
    pw = nv.PackedWeight(mods, wl.K)
    codes, scales, g = nv.empty_quantized(wl.M, wl.K)
    ws = torch.empty((max(nv.nvfp4_quantize_workspace_bytes(wl.M, wl.K), 256),), dtype=torch.uint8, device=DEV)
    gws = torch.zeros((max(nv.nvfp4_gemm_workspace_bytes(wl.M, pw.desc), 256),), dtype=torch.uint8, device=DEV)
    y = torch.empty((wl.M, wl.N), dtype=torch.float32, device=DEV)

    def step():
        nv.nvfp4_quantize(xd, codes, scales, g, nv.NVFP4_G_COMPUTE, ws)
        nv.nvfp4_gemm(wl.M, codes, scales, g, pw.desc, y, wl.N, gws)

    step()
    torch.cuda.synchronize()
    want = (y.clone(), codes.clone(), scales.clone(), g.clone())
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        y.zero_()
        codes.zero_()
        g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want[0]) and torch.equal(codes, want[1]) and torch.equal(scales, want[2]) \
            and torch.equal(g, want[3]), f"replay {i} differs from eager"
        _ = (xd.float() * 2).sum().item()      # unrelated eager work between replays


def test_odd_kstep_count_many_tokens():
    """K = 9 k-steps of 128 with two thousand tokens: the 256 x 256 tiles read their activation scales by
    aligned pairs of k-steps and need an even count, so this product runs on the smaller tiles (a ragged last
    row tile too): every output within the oracle's bound."""
    x = workloads.random_matrix(1401, 2000, 1152, dtype="bf16")
    ws = [workloads.random_matrix(1402, 1024, 1152, 0.05, dtype="bf16")]
    check_dense(x, "bf16", ws, "bf16", "odd k-step count, M=2000 K=1152 N=1024")
