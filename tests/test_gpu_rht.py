"""NVFP4 behind the randomized Hadamard transform on the GPU against the CPU oracle (``oracle.rht``):
codes, scales and g bit for bit in both orientations, and products of transformed operands within
1e-5 * sum|terms| of the oracle's FP64 product."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_03_amd as nv
import workloads
from gpu_util import DEV, assert_quant_equal, host, say, to_dev
from oracle import nvfp4_ref as ref
from oracle import rht
from test_gpu_quantize import EDGE_CASES

pytestmark = pytest.mark.gpu
F32 = np.float32
SIGNS = workloads.rht_signs()


@pytest.mark.parametrize("rows,K", [(1, 16), (16, 64), (37, 160), (300, 1024), (1000, 5120)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rows(rows, K, dtype):
    x = workloads.random_matrix(200 + rows, rows, K, dtype=dtype)
    x[rows // 2, K // 3] = F32(55.0)
    say(f"rht quantize {dtype} {rows}x{K} signs=0x{SIGNS:04x}")
    xd = to_dev(x, dtype)
    out = nv.quantize_rht(xd, SIGNS)
    torch.cuda.synchronize()
    assert_quant_equal(*out, rht.quantize_rht(x, SIGNS), what=f"rht {dtype} {rows}x{K}")
    out = nv.quantize_rht(xd, 0xFFFF, g=0.03125)
    torch.cuda.synchronize()
    assert_quant_equal(*out, rht.quantize_rht(x, 0xFFFF, "given", 0.03125), what=f"rht given {dtype} {rows}x{K}")


@pytest.mark.parametrize("rows,cols", [(16, 1), (48, 7), (272, 130), (1024, 1030)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_transposed(rows, cols, dtype):
    x = workloads.random_matrix(300 + rows + cols, rows, cols, dtype=dtype)
    say(f"rht quantize_t {dtype} {rows}x{cols}")
    xd = to_dev(x, dtype)
    out = nv.quantize_t_rht(xd, SIGNS)
    torch.cuda.synchronize()
    assert_quant_equal(*out, rht.quantize_t_rht(x, SIGNS), what=f"rht^T {dtype} {rows}x{cols}")
    out = nv.quantize_t_rht(xd, 0x0001, g=0.5)
    torch.cuda.synchronize()
    assert_quant_equal(*out, rht.quantize_t_rht(x, 0x0001, "given", 0.5), what=f"rht^T given {dtype}")


@pytest.mark.parametrize("case", sorted(EDGE_CASES))
def test_edge_cases(case):
    """The quantizer's edge cases (zeros, signed zeros, subnormals, huge values, ...) through the transform,
    in both orientations (FP32 input)."""
    x = EDGE_CASES[case]()
    say(f"rht edge case {case} {x.shape}")
    out = nv.quantize_rht(to_dev(x, "f32"), SIGNS)
    torch.cuda.synchronize()
    assert_quant_equal(*out, rht.quantize_rht(x, SIGNS), what=f"{case} rows")
    xt = np.ascontiguousarray(x.T)
    out = nv.quantize_t_rht(to_dev(xt, "f32"), SIGNS)
    torch.cuda.synchronize()
    assert_quant_equal(*out, rht.quantize_rht(x, SIGNS), what=f"{case} transposed")


def test_one_hot_closed_form():
    """A one-hot block of 2688 becomes 16 entries of +-672: g = 1/4, scale 448, code magnitude 6."""
    x = np.zeros((2, 32), F32)
    x[0, 5] = 2688.0
    say("rht one-hot block")
    c, s, g = nv.quantize_rht(to_dev(x, "f32"), 0)
    torch.cuda.synchronize()
    assert float(host(g)[0]) == 0.25 and host(s)[0, 0] == 0x7E
    assert np.all(ref.unpack_codes(host(c))[0, :16] & 7 == 7)


@pytest.mark.parametrize("M,N,K", [(64, 96, 256), (300, 272, 640)])
def test_products(M, N, K):
    """Both operands transformed with the same signs: the unchanged product of their codes matches the
    oracle's product of the transformed operands, and approximates X . W^T."""
    x = workloads.random_matrix(500 + M, M, K, 1.0, "bf16")
    w = workloads.random_matrix(600 + N, N, K, 0.05, "bf16")
    say(f"rht products M={M} N={N} K={K}")
    xq = nv.quantize_rht(to_dev(x, "bf16"), SIGNS)
    wq = nv.quantize_rht(to_dev(w, "bf16"), SIGNS)
    y = nv.gemm(*xq, nv.PackedWeight([wq], K))
    torch.cuda.synchronize()
    oxq, owq = rht.quantize_rht(x, SIGNS), rht.quantize_rht(w, SIGNS)
    assert_quant_equal(*xq, oxq, what="X")
    assert_quant_equal(*wq, owq, what="W")
    y_ref, a_ref = ref.gemm(oxq, [owq])
    ok, worst = ref.gemm_within_tolerance(host(y), y_ref, a_ref)
    assert ok, f"worst |dy|/sum|terms| = {worst:.3e}"
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.linalg.norm(host(y) - exact) < 0.2 * np.linalg.norm(exact)


def test_workload_gdn_activations():
    """The heavy-tailed GDN activations (4096 x 5120 bf16) through the transform: g from the whole
    transformed tensor, sampled rows bit-exact."""
    wl = workloads.make("gdn")
    say(f"rht quantize gdn X {wl.x.shape}")
    c, s, g = nv.quantize_rht(to_dev(wl.x, "bf16"), SIGNS)
    torch.cuda.synchronize()
    t = rht.rht_blocks(wl.x, SIGNS)
    g_ref = ref.global_scale(F32(np.max(np.abs(t))))
    rows = np.unique(np.concatenate([[0, wl.M - 1], np.random.default_rng(3).choice(wl.M, 30, replace=False)]))
    oq = ref.quantize(t[rows], "given", g_ref)
    assert_quant_equal(c, s, g, oq, rows=torch.from_numpy(rows).to(DEV), what="gdn X rht")
