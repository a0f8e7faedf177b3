"""The FP8 KV-cache quantizer on the GPU against the CPU oracle (``oracle.fp8_kv``): bytes and the
calibrated scale bit for bit, in both scale modes, on KV-cache-shaped tensors and edge cases."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_03_amd as nv
import workloads
from gpu_util import DEV, host, say, to_dev
from oracle import fp8_kv

pytestmark = pytest.mark.gpu
F32 = np.float32


def _check(x_np, dtype, what, scale=None, ld_pad=0):
    rows, cols = x_np.shape
    if ld_pad:
        big = np.zeros((rows, cols + ld_pad), F32)
        big[:, :cols] = x_np
        xd = to_dev(big, dtype)[:, :cols]
    else:
        xd = to_dev(x_np, dtype)
    c, s = nv.kv_quantize_fp8(xd, scale)
    torch.cuda.synchronize()
    oc, os_ = fp8_kv.quantize_kv(x_np, "compute" if scale is None else "given", scale)
    assert np.float32(host(s)[0]).tobytes() == np.float32(os_).tobytes(), f"{what}: scale {host(s)[0]!r} != {os_!r}"
    got = host(c)
    if not np.array_equal(got, oc):
        bad = np.argwhere(got != oc)
        r, k = bad[0]
        raise AssertionError(f"{what}: {len(bad)} bytes differ, first at [{r}, {k}] x={x_np[r, k]!r}: "
                             f"gpu 0x{got[r, k]:02x} oracle 0x{oc[r, k]:02x}")


@pytest.mark.parametrize("rows,cols", [(1, 1), (3, 7), (16, 64), (37, 1000), (4096, 1024)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shapes(rows, cols, dtype):
    x = workloads.random_matrix(700 + rows + cols, rows, cols, 2.0, dtype)
    say(f"kv fp8 {dtype} {rows}x{cols}")
    _check(x, dtype, f"{dtype} {rows}x{cols}")
    _check(x, dtype, f"{dtype} {rows}x{cols} given", scale=0.0078125)


def test_strided_and_unaligned_rows():
    x = workloads.random_matrix(801, 50, 200, 1.0, "bf16")
    say("kv fp8 strided rows (ld = cols + 3, rows start on 2-byte boundaries)")
    _check(x, "bf16", "strided bf16", ld_pad=3)
    _check(workloads.random_matrix(802, 50, 200), "f32", "strided f32", ld_pad=16)


EDGE = {
    "zeros": lambda: np.zeros((4, 24), F32),
    "signed_zeros": lambda: np.tile(np.array([0.0, -0.0], F32), (3, 8)),
    "subnormal_fp32": lambda: workloads.random_matrix(803, 8, 64) * F32(1e-40),
    "saturating": lambda: np.concatenate([workloads.random_matrix(804, 4, 32), np.full((4, 32), 1e30, F32)], 1),
    "heavy_tail": lambda: (np.random.default_rng(805).standard_t(1.5, size=(64, 256)) * 10).astype(F32),
    "e4m3_midpoints": lambda: np.array([[(a + b) / 2 for a, b in zip(fp8_kv.ref.E4M3_VALS[:-1],
                                                                     fp8_kv.ref.E4M3_VALS[1:])]], F32),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_cases(case):
    x = EDGE[case]()
    say(f"kv fp8 edge case {case} {x.shape}")
    _check(x, "f32", case)
    _check(x, "f32", case + " given", scale=1.0)


def test_nan_keeps_sign():
    x = np.array([[np.nan, -np.nan, 1.0, -2.0, 500.0, -0.0, 3.0, 4.0]], F32)
    say("kv fp8 NaN and signs (given scale)")
    c, _ = nv.kv_quantize_fp8(to_dev(x, "f32"), 1.0)
    torch.cuda.synchronize()
    oc, _ = fp8_kv.quantize_kv(x, "given", 1.0)
    assert np.array_equal(host(c), oc) and host(c)[0, 0] == 0x7F and host(c)[0, 1] == 0xFF


def test_round_trip_error():
    """Dequantized K/V values within half an E4M3 step of the input (or the subnormal spacing)."""
    x = workloads.random_matrix(806, 512, 1024, 3.0, "bf16")
    c, s = nv.kv_quantize_fp8(to_dev(x, "bf16"))
    torch.cuda.synchronize()
    back = fp8_kv.dequantize_kv(host(c), host(s)[0])
    err = np.abs(back - x.astype(np.float64))
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * float(host(s)[0])) * (1 + 1e-6))
