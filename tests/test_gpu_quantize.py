"""Quantizer parity on the GPU: codes, scales and g from nvfp4_quantize must equal the
CPU oracle's bit for bit, on every workload's activations and weights and on edge cases."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_03_amd as nv
import workloads
from gpu_util import DEV, assert_quant_equal, host, oracle_quantize_rows, say, to_dev
from oracle import nvfp4_ref as ref

pytestmark = pytest.mark.gpu
F32 = np.float32


def gpu_quantize(x_np, dtype, g=None, ld_pad=0):
    rows, K = x_np.shape
    if ld_pad:
        big = np.zeros((rows, K + ld_pad), F32)
        big[:, :K] = x_np
        xd = to_dev(big, dtype)[:, :K]
    else:
        xd = to_dev(x_np, dtype)
    out = nv.quantize(xd, g=g)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_workload_full(name):
    wl = workloads.make(name)
    say(f"quantize parity: {name} X {wl.x.shape} {wl.x_dtype}, W {[w.shape for w in wl.w]}")
    c, s, g = gpu_quantize(wl.x, wl.x_dtype)
    assert_quant_equal(c, s, g, ref.quantize(wl.x), what=f"{name} X")
    for i, w in enumerate(wl.w):
        c, s, g = gpu_quantize(w, wl.w_dtype)
        assert_quant_equal(c, s, g, ref.quantize(w), what=f"{name} W[{i}]")


def _sampled_rows(n, seed, k=48):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=min(k, n), replace=False)]))
    return rows


@pytest.mark.parametrize("name", ["gdn", "ngpt", "large"])
def test_workload_sampled_rows(name):
    wl = workloads.make(name)
    say(f"quantize parity (g exact, sampled rows): {name} X {wl.x.shape}")
    c, s, g = gpu_quantize(wl.x, wl.x_dtype)
    rows = _sampled_rows(wl.M, 1)
    assert_quant_equal(c, s, g, oracle_quantize_rows(wl.x, rows), rows=torch.from_numpy(rows).to(DEV),
                       what=f"{name} X")
    del c, s
    for i, w in enumerate(wl.w):
        say(f"quantize parity: {name} W[{i}] {w.shape}")
        c, s, g = gpu_quantize(w, wl.w_dtype)
        rows = _sampled_rows(w.shape[0], 2 + i, k=16)
        assert_quant_equal(c, s, g, oracle_quantize_rows(w, rows), rows=torch.from_numpy(rows).to(DEV),
                           what=f"{name} W[{i}]")


def test_ngpt_without_per_tensor_scaling():
    """g = 1 (no per-tensor scaling): block scales of unit-norm rows fall in the E4M3 subnormal range."""
    wl = workloads.make_ngpt(M=512)
    say("quantize parity: ngpt X[512] with g = 1")
    c, s, g = gpu_quantize(wl.x, "bf16", g=1.0)
    oq = ref.quantize(wl.x, g_mode="given", g=1.0)
    assert (oq.scales < 8).mean() > 0.5     # mostly subnormal scales
    assert_quant_equal(c, s, g, oq, what="ngpt g=1")


def test_golden_fixtures_on_gpu():
    import oracle_pins
    for fname, mode in [("worked_given_g.txt", "given"), ("worked_computed_g.txt", "compute"),
                        ("worked_op_order.txt", "given")]:
        d = oracle_pins.load_golden(fname)
        x = np.array(d["x"], F32)[None, :]
        say(f"quantize golden fixture {fname}")
        c, s, g = gpu_quantize(x, "f32", g=d["g"] if mode == "given" else None)
        assert list(host(s)[0]) == d["scales"]
        assert list(ref.unpack_codes(host(c))[0]) == d["nibbles"]
        if mode == "compute":
            assert np.float32(host(g)[0]) == np.float32(d["g"])


EDGE_CASES = {
    "zeros": lambda: np.zeros((3, 64), F32),
    "one_block": lambda: workloads.random_matrix(5, 1, 16),
    "ragged_rows": lambda: workloads.random_matrix(6, 37, 48),
    "tiny_blocks_to_zero_scale": lambda: np.concatenate(
        [workloads.random_matrix(7, 4, 32) * F32(1e-7), workloads.random_matrix(8, 4, 32) * F32(40)], axis=1),
    "fp32_subnormals": lambda: workloads.random_matrix(9, 8, 64) * F32(1e-40),
    "huge": lambda: workloads.random_matrix(10, 8, 64) * F32(1e30),
    "subnormal_blocks_in_normal_tensor": lambda: np.concatenate(
        [workloads.random_matrix(16, 8, 32) * F32(1e-44), workloads.random_matrix(17, 8, 32) * F32(3e-39),
         workloads.random_matrix(18, 8, 32)], axis=1),
    "g_floor": lambda: workloads.random_matrix(11, 8, 64) * F32(1e-36),
    "signed_zeros": lambda: np.tile(np.array([0.0, -0.0] * 8, F32), (2, 2)),
    "heavy_tail": lambda: (np.random.default_rng(12).standard_t(1.5, size=(64, 256)) * 10).astype(F32),
}


@pytest.mark.parametrize("case", sorted(EDGE_CASES))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_edge_cases(case, dtype):
    x = EDGE_CASES[case]()
    if dtype == "bf16":
        x = workloads.to_bf16_values(x)
    say(f"quantize edge case {case} {dtype} {x.shape}")
    c, s, g = gpu_quantize(x, dtype)
    assert_quant_equal(c, s, g, ref.quantize(x), what=f"{case}/{dtype}")
    c, s, g = gpu_quantize(x, dtype, g=0.125)
    assert_quant_equal(c, s, g, ref.quantize(x, g_mode="given", g=0.125), what=f"{case}/{dtype} given")


def test_strided_rows():
    x = workloads.random_matrix(13, 33, 160)
    say("quantize strided rows (ld_x = K + 32)")
    c, s, g = gpu_quantize(x, "f32", ld_pad=32)
    assert_quant_equal(c, s, g, ref.quantize(x), what="strided f32")
    xb = workloads.to_bf16_values(x)
    c, s, g = gpu_quantize(xb, "bf16", ld_pad=64)
    assert_quant_equal(c, s, g, ref.quantize(xb), what="strided bf16")


def test_empty_tensor():
    say("quantize empty tensor")
    xd = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    c, s, g = nv.quantize(xd)
    torch.cuda.synchronize()
    assert c.numel() == 0 and float(g.item()) == 1.0


def test_e2m1_rounding_sweep():
    """Blocks whose largest element is 6 get S = 1 and r = 1 under g = 1, so codes are the E2M1
    rounding of the raw inputs: sweep FP32 values over [-6, 6] including every tie and its neighbours."""
    rng = np.random.default_rng(14)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1, 1.5, 2, 3, 4, 6], F32)
    near = np.concatenate([mids, np.nextafter(mids, F32(0)), np.nextafter(mids, F32(7))])
    sweep = np.linspace(0, 6, 600_000, dtype=F32)
    vals = np.concatenate([near, sweep, rng.uniform(0, 6, 100_000).astype(F32)])
    vals = np.concatenate([vals, -vals])
    vals = vals[np.abs(vals) <= 6]
    n15 = (len(vals) + 119) // 120 * 120           # whole rows of 8 blocks
    vals = np.resize(vals, n15).reshape(-1, 15)
    x = np.concatenate([np.full((vals.shape[0], 1), 6.0, F32), vals], axis=1).reshape(-1, 16 * 8)
    say(f"quantize e2m1 sweep {x.shape}")
    c, s, g = gpu_quantize(x, "f32", g=1.0)
    oq = ref.quantize(x, g_mode="given", g=1.0)
    assert np.all(oq.scales == 0x38)
    assert_quant_equal(c, s, g, oq, what="e2m1 sweep")


def test_e4m3_rounding_sweep():
    """Under g = 1 a block's scale is E4M3(fl32(bamax/6)): drive bamax = 6u over every E4M3 midpoint
    and its FP32 neighbours, and a log-uniform sweep, so every scale rounding case is exercised."""
    vals = np.array(ref.E4M3_VALS, np.float64)
    mids = ((vals[1:] + vals[:-1]) / 2).astype(F32)
    u = np.concatenate([mids, np.nextafter(mids, F32(0)), np.nextafter(mids, F32(1e9)), vals.astype(F32),
                        (F32(2.0) ** np.random.default_rng(15).uniform(-12, 9.5, 20000)).astype(F32),
                        np.array([448, 460, 500, 1e4], F32)])
    bamax = (u.astype(np.float64) * 6).astype(F32)
    x = np.zeros((len(bamax), 16), F32)
    x[:, 0] = bamax
    x[:, 1] = -bamax * F32(0.5)
    x[:, 2] = bamax * F32(0.3)
    x = x.reshape(-1, 16 * 4) if len(bamax) % 4 == 0 else x
    say(f"quantize e4m3 sweep {x.shape}")
    c, s, g = gpu_quantize(x, "f32", g=1.0)
    assert_quant_equal(c, s, g, ref.quantize(x, g_mode="given", g=1.0), what="e4m3 sweep")


def test_deterministic():
    wl = workloads.make_gdn(M=256)
    xd = to_dev(wl.x, "bf16")
    say("quantize determinism (3 runs)")
    outs = [nv.quantize(xd) for _ in range(3)]
    torch.cuda.synchronize()
    for c, s, g in outs[1:]:
        assert torch.equal(c, outs[0][0]) and torch.equal(s, outs[0][1]) and torch.equal(g, outs[0][2])
