"""Parity of the x^T encoding (nvfp4_quantize_t) on the GPU against the CPU oracle, bit for bit,
and of the two backward products built from it against the FP64 oracle product.

The oracle's x^T encoding is its row quantizer applied to the transpose; the GPU kernel reads x
in its own layout and never forms the transpose in memory."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_03_amd as nv
import workloads
from gpu_util import DEV, assert_quant_equal, host, say, to_dev
from oracle import nvfp4_ref as ref
from test_gpu_quantize import EDGE_CASES

pytestmark = pytest.mark.gpu
F32 = np.float32


def gpu_quantize_t(x_np, dtype, g=None, ld_pad=0):
    rows, cols = x_np.shape
    if ld_pad:
        big = np.zeros((rows, cols + ld_pad), F32)
        big[:, :cols] = x_np
        xd = to_dev(big, dtype)[:, :cols]
    else:
        xd = to_dev(x_np, dtype)
    out = nv.quantize_t(xd, g=g)
    torch.cuda.synchronize()
    return out


# (rows, cols): one tile, several tiles with ragged row and column tails, odd widths, 64-row
# multiples (word-wide scale stores) and not (byte scale stores)
SHAPES = [(16, 1), (16, 64), (48, 7), (256, 64), (272, 130), (320, 200), (784, 333), (1024, 1030)]


@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shapes(rows, cols, dtype):
    x = workloads.random_matrix(100 + rows + cols, rows, cols, dtype=dtype)
    x[rows // 2, cols // 2] = F32(-37.5)
    say(f"quantize_t parity {dtype} rows={rows} cols={cols}")
    c, s, g = gpu_quantize_t(x, dtype)
    assert_quant_equal(c, s, g, ref.quantize_t(x), what=f"x^T {dtype} {rows}x{cols}")
    c, s, g = gpu_quantize_t(x, dtype, g=0.0625)
    assert_quant_equal(c, s, g, ref.quantize_t(x, "given", 0.0625), what=f"x^T given {dtype} {rows}x{cols}")


@pytest.mark.parametrize("case", sorted(EDGE_CASES))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_cases(case, dtype):
    """The row quantizer's edge cases, fed transposed: the x^T encoding of x^T is the row encoding of x."""
    x = EDGE_CASES[case]()
    if dtype == "bf16":
        x = workloads.to_bf16_values(x)
    xt = np.ascontiguousarray(x.T)
    say(f"quantize_t edge case {case} {dtype} {xt.shape}")
    c, s, g = gpu_quantize_t(xt, dtype)
    assert_quant_equal(c, s, g, ref.quantize(x), what=f"{case}/{dtype}")
    c, s, g = gpu_quantize_t(xt, dtype, g=0.125)
    assert_quant_equal(c, s, g, ref.quantize(x, g_mode="given", g=0.125), what=f"{case}/{dtype} given")


def test_strided_rows():
    x = workloads.random_matrix(13, 96, 150)
    say("quantize_t strided rows (ld_x = cols + 10 / + 26)")
    c, s, g = gpu_quantize_t(x, "f32", ld_pad=10)
    assert_quant_equal(c, s, g, ref.quantize_t(x), what="strided f32")
    xb = workloads.to_bf16_values(x)
    c, s, g = gpu_quantize_t(xb, "bf16", ld_pad=26)
    assert_quant_equal(c, s, g, ref.quantize_t(xb), what="strided bf16")


def test_empty():
    say("quantize_t empty tensors")
    for shape in [(0, 64), (64, 0)]:
        xd = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        c, s, g = nv.quantize_t(xd)
        torch.cuda.synchronize()
        assert c.shape == (shape[1], shape[0] // 2) and float(host(g)[0]) == 1.0


def _sampled(n, seed, k):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(k, n), replace=False)]))


@pytest.mark.parametrize("name", ["ngpt", "gdn"])
def test_workload_operands(name):
    """Full-size activations and weights of a workload, encoded transposed; the oracle checks g and a
    sample of output rows (= columns of the input) that includes the first and the last."""
    wl = workloads.make(name)
    for what, x, dtype in [("X", wl.x, wl.x_dtype), ("W[0]", wl.w[0], wl.w_dtype)]:
        say(f"quantize_t parity: {name} {what} {x.shape}")
        c, s, g = gpu_quantize_t(x, dtype)
        cols = _sampled(x.shape[1], 7, 24)
        g_ref = ref.global_scale(F32(np.max(np.abs(x))))
        oq = ref.quantize_t(x[:, cols], "given", g_ref)
        sel = torch.from_numpy(cols).to(DEV)
        assert_quant_equal(c, s, g, oq, rows=sel, what=f"{name} {what}^T")
        del c, s


def _backward_case(M, N, K, seed, dtype="bf16"):
    dy = workloads.random_matrix(seed, M, N, 0.01, dtype)
    w = workloads.random_matrix(seed + 1, N, K, 0.02, dtype)
    x = workloads.random_matrix(seed + 2, M, K, 1.0, dtype)
    return dy, w, x


@pytest.mark.parametrize("M,N,K", [(256, 384, 192), (384, 128, 80)])
def test_backward_products(M, N, K):
    """dX = dY . W and dW = dY^T . X with every operand encoded along its contraction axis:
    X^ of dX is quantize(dY), its weight quantize_t(W); X^ of dW is quantize_t(dY), its weight
    quantize_t(X).  Codes and scales bit-exact, products within 1e-5 * sum|terms|."""
    dy, w, x = _backward_case(M, N, K, 40 + M)
    dyd, wd, xd = to_dev(dy, "bf16"), to_dev(w, "bf16"), to_dev(x, "bf16")
    say(f"backward products M={M} N={N} K={K}: dX")
    a = nv.quantize(dyd)
    wt = nv.quantize_t(wd)
    dx = nv.gemm(*a, nv.PackedWeight([wt], N))
    torch.cuda.synchronize()
    aq, wtq = ref.quantize(dy), ref.quantize_t(w)
    assert_quant_equal(*a, aq, what="dY")
    assert_quant_equal(*wt, wtq, what="W^T")
    y_ref, a_ref = ref.gemm(aq, [wtq])
    ok, worst = ref.gemm_within_tolerance(host(dx), y_ref, a_ref)
    assert ok, f"dX: worst |dy|/sum|terms| = {worst:.3e}"
    # the quantized product approximates the exact one (a loose sanity bound, not the parity check)
    exact = dy.astype(np.float64) @ w.astype(np.float64)
    assert np.linalg.norm(host(dx) - exact) < 0.25 * np.linalg.norm(exact)

    say(f"backward products M={M} N={N} K={K}: dW")
    at = nv.quantize_t(dyd)
    xt = nv.quantize_t(xd)
    dw = nv.gemm(*at, nv.PackedWeight([xt], M))
    torch.cuda.synchronize()
    atq, xtq = ref.quantize_t(dy), ref.quantize_t(x)
    assert_quant_equal(*at, atq, what="dY^T")
    assert_quant_equal(*xt, xtq, what="X^T")
    y_ref, a_ref = ref.gemm(atq, [xtq])
    ok, worst = ref.gemm_within_tolerance(host(dw), y_ref, a_ref)
    assert ok, f"dW: worst |dy|/sum|terms| = {worst:.3e}"
    exact = dy.T.astype(np.float64) @ x.astype(np.float64)
    assert np.linalg.norm(host(dw) - exact) < 0.25 * np.linalg.norm(exact)


def test_repeat_deterministic():
    x = workloads.random_matrix(77, 512, 384, dtype="bf16")
    xd = to_dev(x, "bf16")
    say("quantize_t repeated calls")
    first = nv.quantize_t(xd)
    for _ in range(3):
        again = nv.quantize_t(xd)
        torch.cuda.synchronize()
        assert all(torch.equal(p, q) for p, q in zip(first, again))


@pytest.mark.parametrize("rows,cols", [(16, 16), (48, 80), (272, 144), (1024, 1040)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_both_orientations(rows, cols, dtype):
    """nvfp4_quantize_both: the row and the column encodings from one read, each bit for bit the oracle's
    (and the GPU's separate calls')."""
    x = workloads.random_matrix(1400 + rows + cols, rows, cols, dtype=dtype)
    x[rows // 3, cols // 5] = F32(29.0)
    xd = to_dev(x, dtype)
    say(f"quantize both orientations {dtype} {rows}x{cols}")
    (c, s, g), (ct, st, gt) = nv.quantize_both(xd)
    torch.cuda.synchronize()
    assert_quant_equal(c, s, g, ref.quantize(x), what=f"rows {dtype} {rows}x{cols}")
    assert_quant_equal(ct, st, gt, ref.quantize_t(x), what=f"cols {dtype} {rows}x{cols}")
    sep_t = nv.quantize_t(xd)
    torch.cuda.synchronize()
    assert torch.equal(ct, sep_t[0]) and torch.equal(st, sep_t[1])
    (c, s, g), (ct, st, _) = nv.quantize_both(xd, g=0.25)
    torch.cuda.synchronize()
    assert_quant_equal(c, s, g, ref.quantize(x, "given", 0.25), what=f"rows given {dtype}")
    assert_quant_equal(ct, st, g, ref.quantize_t(x, "given", 0.25), what=f"cols given {dtype}")


def test_both_orientations_strided_workload():
    """The nGPT gradient-shaped tensor [8192 x 4096] bf16 viewed with a padded row stride: sampled rows of
    both encodings against the oracle."""
    x = workloads.random_matrix(1450, 8192, 4096, 1e-3, "bf16")
    big = torch.zeros((8192, 4096 + 64), dtype=torch.bfloat16, device=DEV)
    big[:, :4096] = to_dev(x, "bf16")
    say("quantize both orientations 8192x4096 bf16, ld = 4160")
    (c, s, g), (ct, st, _) = nv.quantize_both(big[:, :4096])
    torch.cuda.synchronize()
    g_ref = ref.global_scale(F32(np.max(np.abs(x))))
    rows = _sampled(8192, 11, 24)
    assert_quant_equal(c, s, g, ref.quantize(x[rows], "given", g_ref), rows=torch.from_numpy(rows).to(DEV),
                       what="rows")
    cols = _sampled(4096, 12, 24)
    assert_quant_equal(ct, st, g, ref.quantize_t(x[:, cols], "given", g_ref), rows=torch.from_numpy(cols).to(DEV),
                       what="cols")


def test_graph_replays_of_the_training_quantizers():
    """quantize_t, quantize_both, the RHT variants and the FP8 KV quantizer (g or the scale computed, so
    the amax pass runs too) captured in one HIP graph: every replay equals the eager calls."""
    x = workloads.random_matrix(1500, 512, 384, 0.5, "bf16")
    xd = to_dev(x, "bf16")
    rows, cols = x.shape
    ws = torch.empty((max(nv.nvfp4_quantize_workspace_bytes(rows, cols), 256),), dtype=torch.uint8, device=DEV)
    outs_t = nv.empty_quantized(cols, rows, DEV)
    outs_b = nv.empty_quantized(rows, cols, DEV) + nv.empty_quantized(cols, rows, DEV)[:2]
    outs_r = nv.empty_quantized(rows, cols, DEV)
    outs_rt = nv.empty_quantized(cols, rows, DEV)
    kv_c = torch.empty((rows, cols), dtype=torch.uint8, device=DEV)
    kv_s = torch.empty((1,), dtype=torch.float32, device=DEV)
    ws2, ws3, ws4, ws5 = (torch.empty_like(ws) for _ in range(4))

    def run(s):
        nv.nvfp4_quantize_t(xd, *outs_t, nv.NVFP4_G_COMPUTE, ws, stream=s)
        c, sc, g, ct, st = outs_b
        nv.nvfp4_quantize_both(xd, c, sc, ct, st, g, nv.NVFP4_G_COMPUTE, ws2, stream=s)
        nv.nvfp4_quantize_rht(xd, 0x5A5A, *outs_r, nv.NVFP4_G_COMPUTE, ws3, stream=s)
        nv.nvfp4_quantize_t_rht(xd, 0x0F0F, *outs_rt, nv.NVFP4_G_COMPUTE, ws4, stream=s)
        nv.nvfp4_kv_quantize_fp8(xd, kv_c, kv_s, nv.NVFP4_G_COMPUTE, ws5, stream=s)

    tensors = list(outs_t) + list(outs_b) + list(outs_r) + list(outs_rt) + [kv_c, kv_s]
    say("training quantizers: graph replays")
    strm = torch.cuda.Stream()
    with torch.cuda.stream(strm):
        run(strm)
    torch.cuda.synchronize()
    eager = [t.clone() for t in tensors]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=strm):
        run(strm)
    for _ in range(3):
        for t in tensors:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(tensors, eager))


def _blob_regions(pw: "nv.PackedWeight"):
    """The written parts of a packed blob: header fields, codes, scales and column scales (the bytes between
    them are alignment padding that no one writes)."""
    d, b = pw.desc, host(pw.blob)
    n_pad, k = d.n_padded, d.k
    return (b[:40], b[d.codes_offset:d.codes_offset + n_pad * k // 2],
            b[d.scales_offset:d.scales_offset + n_pad * k // 16], b[d.colscale_offset:d.colscale_offset + 4 * n_pad])


@pytest.mark.parametrize("n,k,dtype,ld_pad", [(128, 128, "bf16", 0), (384, 256, "bf16", 0), (640, 384, "f32", 0),
                                              (256, 640, "bf16", 24), (4096, 4096, "bf16", 0)])
def test_pack_weights_train(n, k, dtype, ld_pad):
    """Both packed operands from one read equal, byte for byte, quantize + pack and quantize_t + pack (whose
    codes the oracle checks), padding rows, column scales and header fields included; so do their products."""
    wt = workloads.random_matrix(1600 + n + k, n, k, 0.05, dtype)
    wt[n // 3, k // 7] = F32(3.5)
    if ld_pad:
        big = np.zeros((n, k + ld_pad), F32)
        big[:, :k] = wt
        wd = to_dev(big, dtype)[:, :k]
    else:
        wd = to_dev(wt, dtype)
    say(f"pack_weights_train {dtype} n={n} k={k} ld_pad={ld_pad}")
    fwd, bwd, g = nv.pack_weights_train(wd)
    ref_fwd = nv.PackedWeight([nv.quantize(wd)], k)
    ref_bwd = nv.PackedWeight([nv.quantize_t(wd)], n)
    torch.cuda.synchronize()
    for got, want, what in [(fwd, ref_fwd, "forward"), (bwd, ref_bwd, "backward")]:
        for part, (a, b) in zip(["header", "codes", "scales", "colscale"], zip(_blob_regions(got), _blob_regions(want))):
            assert np.array_equal(a, b), f"{what} {part} differs"
    assert np.float32(host(g)[0]) == ref.global_scale(F32(np.max(np.abs(wt))))
    x = to_dev(workloads.random_matrix(1700 + n, 64, k, 1.0, "bf16"), "bf16")
    xq = nv.quantize(x)
    assert torch.equal(nv.gemm(*xq, fwd), nv.gemm(*xq, ref_fwd))
    dy = to_dev(workloads.random_matrix(1800 + k, 64, n, 0.01, "bf16"), "bf16")
    dq = nv.quantize(dy)
    torch.cuda.synchronize()
    assert torch.equal(nv.gemm(*dq, bwd), nv.gemm(*dq, ref_bwd))
    fwd_g, bwd_g, _ = nv.pack_weights_train(wd, g=0.125)
    ref_fwd_g = nv.PackedWeight([nv.quantize(wd, g=0.125)], k)
    ref_bwd_g = nv.PackedWeight([nv.quantize_t(wd, g=0.125)], n)
    torch.cuda.synchronize()
    for got, want in [(fwd_g, ref_fwd_g), (bwd_g, ref_bwd_g)]:
        assert all(np.array_equal(a, b) for a, b in zip(_blob_regions(got), _blob_regions(want)))
