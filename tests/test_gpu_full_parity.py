"""Full-size parity: every code and scale byte of the GDN, nGPT and large-layer operands against the
oracle, one dense slab of the large layer's product over all of K = 16384, and the hardware E2M1
conversion against the encoding rule over the whole finite FP32 range.

The oracle encodes row chunks with the whole tensor's g (its g is checked on its own first), in a
pool of threads: numpy's array operations release the interpreter lock, so the chunks run in
parallel on the host cores.

Pages: "Why Gated DeltaNet Survives 4-Bit Quantization", section "Why the 'Fragile' Recurrence is
Actually Robust" (16-element blocks, each with an E4M3 scale, and an FP32 tensor scale)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_03_amd as nv
import workloads
from gpu_util import DEV, assert_every_byte, host, oracle_quantize_whole, oracle_threads, say, to_dev
from oracle import nvfp4_ref as ref

pytestmark = pytest.mark.gpu
F32 = np.float32


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["gdn", "ngpt", "large"])
def test_workload_every_byte(name):
    """All operands of the workload, quantized whole on the device, against the oracle byte for byte."""
    wl = workloads.make(name)
    say(f"every-byte parity: {name} X {wl.x.shape} {wl.x_dtype} ({oracle_threads()} oracle threads)")
    c, s, g = nv.quantize(to_dev(wl.x, wl.x_dtype))
    torch.cuda.synchronize()
    assert_every_byte(c, s, g, wl.x, f"{name} X")
    del c, s, g
    for i, w in enumerate(wl.w):
        say(f"every-byte parity: {name} W[{i}] {w.shape}")
        c, s, g = nv.quantize(to_dev(w, wl.w_dtype))
        torch.cuda.synchronize()
        assert_every_byte(c, s, g, w, f"{name} W[{i}]")
        del c, s, g


@pytest.mark.timeout(300)
def test_large_dense_slab():
    """The large layer (32768 x 16384 by 16384 x 16384) in the timed launch configuration (one workspace,
    the layer call); 256 whole output rows, every column, against the FP64 oracle product of the oracle's
    own quantization: the first and last rows, rows straddling the tile boundary at 16384, and 64 drawn
    rows."""
    wl = workloads.make_large()
    say(f"large dense slab: M={wl.M} K={wl.K} N={wl.N}")
    xd = to_dev(wl.x, "bf16")
    pw = nv.PackedWeight([nv.quantize(to_dev(wl.w[0], "bf16"))], wl.K)
    ws = nv.linear_workspace(wl.M, xd.dtype, pw)
    y, xc, xs, gx = nv.linear(xd, pw, ws)
    torch.cuda.synchronize()
    del xd
    rng = np.random.default_rng(16384)
    fixed = np.concatenate([np.arange(64), np.arange(16384 - 32, 16384 + 32), np.arange(wl.M - 64, wl.M)])
    drawn = rng.choice(np.setdiff1d(np.arange(wl.M), fixed), 64, replace=False)
    rows = np.sort(np.concatenate([fixed, drawn]))
    assert rows.size == 256
    y_rows = host(y[torch.from_numpy(rows).to(DEV)])
    del y
    say("large dense slab: oracle quantization of W and the X rows")
    wq = oracle_quantize_whole(wl.w[0])
    g_x = ref.global_scale(F32(np.max(np.abs(wl.x))))
    xq = ref.quantize(wl.x[rows], "given", g_x)
    assert np.array_equal(host(xc[torch.from_numpy(rows).to(DEV)]), xq.codes)
    assert F32(host(gx)[0]).tobytes() == F32(g_x).tobytes()
    say("large dense slab: FP64 product")
    y_ref, a_ref = ref.gemm(xq, [wq])
    ok, worst = ref.gemm_within_tolerance(y_rows, y_ref, a_ref)
    assert ok, f"large dense slab: worst |dy|/sum|terms| = {worst:.3e}"


def _float_sweep(rng, n):
    """FP32 magnitudes over every binade (subnormal to the largest finite), random mantissas, plus the
    extremes and their neighbours."""
    bits = (rng.integers(1, 255, n, dtype=np.uint32) << 23) | rng.integers(0, 1 << 23, n, dtype=np.uint32)
    sub = rng.integers(1, 1 << 23, n // 16, dtype=np.uint32)            # subnormals
    edge = np.array([1, 2, 0x007FFFFF, 0x00800000, 0x00800001, 0x7F7FFFFE, 0x7F7FFFFF, 0x3F800000,
                     0x000001C0, 0x000001C1], np.uint32)            # 448 * 2^-149: q = 2^-149 under r = 1/448
    return np.concatenate([bits, sub, edge]).view(F32)


def _q_of(x, g):
    """The FP32 value each element is converted from, by the encoding steps (scale, reciprocal, product)."""
    blocks = x.reshape(x.shape[0], -1, 16)
    s_enc = F32(1.0) / F32(g)
    S = ref.encode_block_scale(np.max(np.abs(blocks), axis=2), s_enc)
    r = ref.block_reciprocal(S, s_enc)
    return (blocks * r[:, :, None]).astype(F32), S


def test_hardware_e2m1_whole_range():
    """Element codes over the whole FP32 range of q = fl32(v * r), both signs, against e2m1_encode:
    (a) blocks whose scale is 1 under g = 1 (r = 1, q = v exactly), v over [-6.375, 6.375] with every
    rounding tie and its neighbours; (b) blocks whose scale saturates at 448 under g = 1 and under
    g = 2^-60, where q spans every binade from the subnormals to the largest finite FP32 value and past
    it (products that overflow to infinity saturate like any value above 6)."""
    rng = np.random.default_rng(2688)

    def rows_of_blocks(v, first):
        """15 test values per block after a first element that sets the block's scale; 8 blocks a row."""
        v = np.resize(v, (v.size + 119) // 120 * 120).reshape(-1, 15)
        return np.concatenate([np.full((v.shape[0], 1), first, F32), v], axis=1).reshape(-1, 16 * 8)

    # (a) r = 1: a first element of 6 gives the scale byte 0x38 for a block amax up to 6.375
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 6.375], F32)
    near = np.concatenate([ties, np.nextafter(ties, F32(0)), np.nextafter(ties, F32(7))])
    va = np.concatenate([near, _float_sweep(rng, 200_000), rng.uniform(0, 6.375, 200_000).astype(F32), [F32(0)]])
    va = va[va <= F32(6.375)]
    xa = rows_of_blocks(np.concatenate([va, -va]), 6.0)
    # (b) S saturated: a first element of 3e38 makes t = bamax * s_enc exceed 6 * 448 under either g;
    # the rest sweep the whole range, so q runs from 0 (g = 1) to past the largest float (g = 2^-60)
    vb = _float_sweep(rng, 400_000)
    xb = rows_of_blocks(np.concatenate([vb, -vb]), 3.0e38)
    cases = [("r = 1", xa, 1.0), ("S = 448, g = 1", xb, 1.0), ("S = 448, g = 2^-60", xb, 2.0 ** -60)]
    exps = set()
    for what, x, g in cases:
        q, S = _q_of(x, g)
        if what == "r = 1":
            assert np.all(S == 0x38) and np.array_equal(q.reshape(x.shape), x)
        else:
            assert np.all(S == 0x7E)
            qa = np.abs(q[np.isfinite(q) & (q != 0)])
            exps |= set(np.unique(np.frexp(qa)[1]).tolist())
        if g < 1:
            assert np.isinf(q).any(), "overflowing products are part of the sweep"
        say(f"hardware e2m1 sweep: {what}, {x.shape[0]} x {x.shape[1]}")
        c, s, gd = nv.quantize(to_dev(x, "f32"), g=g)
        torch.cuda.synchronize()
        want = ref.quantize(x, "given", g)
        assert np.array_equal(host(s), want.scales), what
        nib = ref.unpack_codes(host(c))
        assert np.array_equal(nib, ref.e2m1_encode(q.reshape(x.shape))), f"{what}: codes differ from e2m1_encode"
        assert np.array_equal(host(c), want.codes), what
    assert exps >= set(range(-148, 129)), "q covers every FP32 binade"


@pytest.mark.timeout(300)
def test_largest_activation_operand():
    """Activation codes of exactly 2 GiB, the most the products address with their 32-bit byte offsets
    (262144 x 16384 bf16, 8 GiB), through the layer call. X is zero except its last 300 rows (two
    256-row tiles, the last operand offsets within a few MB of 2^31), so the tensor's amax is theirs:
    g, those rows' codes and scales and their output rows against the oracle; every other code, scale
    and output exactly zero."""
    K, N, tail = 16384, 256, 300
    M = (1 << 31) // (K // 2)
    rng = np.random.default_rng(1 << 31)
    xt = torch.from_numpy(rng.standard_normal((tail, K)).astype(F32)).to(torch.bfloat16).float().numpy()
    w = torch.from_numpy((0.01 * rng.standard_normal((N, K))).astype(F32)).to(torch.bfloat16).float().numpy()
    say(f"largest activation operand: M={M} K={K} N={N}, X {M * K * 2 >> 30} GiB bf16, codes {M * K // 2 >> 30} GiB")
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
    x[M - tail:] = to_dev(xt, "bf16")
    pw = nv.PackedWeight([nv.quantize(to_dev(w, "bf16"))], K)
    y, xc, xs, gx = nv.linear(x, pw, nv.linear_workspace(M, x.dtype, pw))
    torch.cuda.synchronize()
    del x
    g_x = ref.global_scale(F32(np.max(np.abs(xt))))
    xq = ref.quantize(xt, "given", g_x)
    assert F32(host(gx)[0]).tobytes() == F32(g_x).tobytes()
    assert np.array_equal(host(xs[M - tail:]), xq.scales)
    assert np.array_equal(host(xc[M - tail:]), xq.codes)
    assert int(torch.count_nonzero(xc[:M - tail])) == 0 and int(torch.count_nonzero(xs[:M - tail])) == 0
    assert int(torch.count_nonzero(y[:M - tail])) == 0
    y_ref, a_ref = ref.gemm(xq, [ref.quantize(w)])
    ok, worst = ref.gemm_within_tolerance(host(y[M - tail:]), y_ref, a_ref)
    assert ok, f"largest activation operand: worst |dy|/sum|terms| = {worst:.3e}"


@pytest.mark.timeout(300)
def test_largest_weight_operand():
    """A packed weight of exactly 2 GiB of codes (262144 x 16384 bf16, 8 GiB, its last column tiles'
    byte offsets within a few MB of 2^31), zero but for its last 300 rows, against 300 activation rows
    through the layer call: those 300 output columns against the oracle, every other column zero."""
    K, tail, M = 16384, 300, 300
    N = (1 << 31) // (K // 2)
    rng = np.random.default_rng((1 << 31) + 1)
    wt = torch.from_numpy((0.01 * rng.standard_normal((tail, K))).astype(F32)).to(torch.bfloat16).float().numpy()
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(F32)).to(torch.bfloat16).float().numpy()
    say(f"largest weight operand: M={M} K={K} N={N}, W {N * K * 2 >> 30} GiB bf16, codes {N * K // 2 >> 30} GiB")
    w = torch.zeros((N, K), dtype=torch.bfloat16, device=DEV)
    w[N - tail:] = to_dev(wt, "bf16")
    pw = nv.PackedWeight([nv.quantize(w)], K)
    del w
    y, _, _, _ = nv.linear(to_dev(x, "bf16"), pw, nv.linear_workspace(M, torch.bfloat16, pw))
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(y[:, :N - tail])) == 0
    wq = ref.quantize(wt, "given", ref.global_scale(F32(np.max(np.abs(wt)))))
    y_ref, a_ref = ref.gemm(ref.quantize(x), [wq])
    ok, worst = ref.gemm_within_tolerance(host(y[:, N - tail:]), y_ref, a_ref)
    assert ok, f"largest weight operand: worst |dy|/sum|terms| = {worst:.3e}"
