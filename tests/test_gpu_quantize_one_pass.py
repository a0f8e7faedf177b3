"""The one-pass quantizer: tensors of about 8.4M to 32M elements (16 to 64 MB of bf16) are quantized by
one workgroup per compute unit, each holding its share of the blocks in registers while the
workgroups exchange their maxima, so x is read once.  Codes, scales and g must equal the oracle's
bit for bit, every byte: bf16 and FP32, dense and strided rows, the tensor maximum in the first or
the last workgroup's share, sizes at both ends of the range, and the local path a workgroup takes
when the exchange does not complete (forced with a poll bound of zero: every workgroup then reduces
max|x| over the whole tensor itself); the same for the transposed encoder (and the encoding both
ways), for the encoding behind the randomized Hadamard transform and for the training-weight packer
(both packed operands of a weight).

Pages: "Why Gated DeltaNet Survives 4-Bit Quantization", section "Why the 'Fragile' Recurrence is
Actually Robust" (16-element blocks with E4M3 scales and one FP32 tensor scale)."""
import numpy as np
import pytest
import torch

import nvfp4_block_scaled_03_amd as nv
from gpu_util import assert_every_byte, say, to_dev
from oracle import rht

pytestmark = pytest.mark.gpu
F32 = np.float32


def _tensor(seed, rows, K, where):
    """Student-t(3) values with one outlier of 60 in the first or last row (the tensor maximum then
    sits in the first or the last workgroup's share)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(rows, K)).astype(F32)
    np.clip(x, -40.0, 40.0, out=x)
    r = 0 if where == "first" else rows - 1
    x[r, int(rng.integers(K))] = F32(-60.0 if where == "first" else 60.0)
    return x


def _dev(x, dtype, ld_pad=0):
    if not ld_pad:
        return to_dev(x, dtype)
    big = np.zeros((x.shape[0], x.shape[1] + ld_pad), F32)
    big[:, :x.shape[1]] = x
    return to_dev(big, dtype)[:, :x.shape[1]]


def _quantize(x, dtype, ld_pad=0):
    out = nv.quantize(_dev(x, dtype, ld_pad))
    torch.cuda.synchronize()
    return out


def _as_dtype(x, dtype):
    """Host values of the device dtype (bf16: rounded to nearest even, as the device holds them)."""
    return x if dtype == "f32" else torch.from_numpy(x).to(torch.bfloat16).float().numpy()


# (dtype, rows, K, row padding, where the maximum is): the smallest size that takes the path
# (1024 amax partials' worth of elements), a ragged share per workgroup, the bf16 capacity
# (32M elements, nGPT's activations), the FP32 capacity (16M elements), strided rows
CASES = [("bf16", 2048, 4112, 0, "last"), ("bf16", 3000, 8192, 0, "first"), ("bf16", 8192, 4096, 0, "last"),
         ("f32", 2048, 8192, 0, "first"), ("bf16", 2100, 4096, 64, "last"), ("f32", 1100, 8192, 4, "first")]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,rows,K,ld_pad,where", CASES)
def test_one_pass_every_byte(dtype, rows, K, ld_pad, where):
    say(f"one-pass quantizer: {dtype} {rows}x{K} ld pad {ld_pad}, maximum in the {where} share")
    x = _as_dtype(_tensor(rows * 7 + K, rows, K, where), dtype)
    c, s, g = _quantize(x, dtype, ld_pad)
    assert_every_byte(c, s, g, x, f"{dtype} {rows}x{K}")


@pytest.mark.timeout(300)
def test_one_pass_local_path(monkeypatch):
    """A poll bound of zero: no workgroup waits for the others' maxima; each reads the whole tensor."""
    monkeypatch.setenv("NVFP4_AMAX_POLLS", "0")
    say("one-pass quantizer, local path: bf16 2048x4112")
    x = _as_dtype(_tensor(11, 2048, 4112, "last"), "bf16")
    c, s, g = _quantize(x, "bf16")
    assert_every_byte(c, s, g, x, "local path")


def test_one_pass_repeated_calls():
    """Records of an earlier call stay in the workspace; the next call's tags tell them apart: three calls
    on different tensors through one workspace, each against the oracle."""
    rows, K = 2048, 4112
    ws = torch.empty(nv.nvfp4_quantize_workspace_bytes(rows, K), dtype=torch.uint8, device="cuda")
    for i, scale in enumerate((1.0, 1e-3, 30.0)):
        say(f"one-pass quantizer, call {i} (scale {scale}) on one workspace")
        x = _as_dtype((_tensor(100 + i, rows, K, "first" if i % 2 else "last") * F32(scale)).astype(F32), "bf16")
        xd = to_dev(x, "bf16")
        c, s, g = nv.empty_quantized(rows, K)
        nv.nvfp4_quantize(xd, c, s, g, nv.NVFP4_G_COMPUTE, ws)
        torch.cuda.synchronize()
        assert_every_byte(c, s, g, x, f"call {i}")


def test_one_pass_zero_tensor():
    """An all-zero tensor in the one-pass range: every workgroup publishes 0, g = 1, codes and scales 0."""
    say("one-pass quantizer: zeros bf16 2048x4112")
    x = np.zeros((2048, 4112), F32)
    c, s, g = _quantize(x, "bf16")
    assert_every_byte(c, s, g, x, "zeros")
    assert float(g.cpu()[0]) == 1.0


def _quantize_t(x, dtype, ld_pad=0, both=False):
    rows, cols = x.shape
    xd = _dev(x, dtype, ld_pad)
    ws = torch.empty(nv.nvfp4_quantize_workspace_bytes(rows, cols), dtype=torch.uint8, device="cuda")
    ct, st, g = nv.empty_quantized(cols, rows)
    if both:
        cr, sr, _ = nv.empty_quantized(rows, cols)
        nv.nvfp4_quantize_both(xd, cr, sr, ct, st, g, nv.NVFP4_G_COMPUTE, ws)
        torch.cuda.synchronize()
        return (cr, sr), (ct, st), g
    nv.nvfp4_quantize_t(xd, ct, st, g, nv.NVFP4_G_COMPUTE, ws)
    torch.cuda.synchronize()
    return None, (ct, st), g


# (dtype, rows, cols, row padding): nGPT's activations and weight (the backward products' operands), FP32,
# strided rows, a width that leaves the last workgroups' column tiles partly past the tensor, and heights
# that leave the last row tile (four quarters of 512 rows) with one live 16-row patch per column lane
# (4112 rows) or with quarters 2 and 3 almost or wholly past the tensor (FP32, 1040 rows)
T_CASES = [("bf16", 8192, 4096, 0), ("bf16", 4096, 4096, 0), ("f32", 2048, 8192, 0), ("bf16", 4096, 2560, 64),
           ("bf16", 6144, 2000, 0), ("bf16", 4112, 4096, 0), ("f32", 1040, 8192, 0)]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,rows,cols,ld_pad", T_CASES)
@pytest.mark.parametrize("both", [False, True])
def test_one_pass_transposed_every_byte(dtype, rows, cols, ld_pad, both):
    """x^T's encoding (and with both=True x's too, from the same registers) against the oracle, every byte."""
    if both and cols % 16:
        pytest.skip("the encoding both ways needs whole 16-column blocks")
    say(f"one-pass transposed encoder: {dtype} {rows}x{cols} ld pad {ld_pad} both={both}")
    x = _as_dtype(_tensor(rows + 3 * cols, rows, cols, "last"), dtype)
    rowq, (ct, st), g = _quantize_t(x, dtype, ld_pad, both)
    assert_every_byte(ct, st, g, np.ascontiguousarray(x.T), f"x^T {dtype} {rows}x{cols}")
    if both:
        assert_every_byte(rowq[0], rowq[1], g, x, f"x {dtype} {rows}x{cols}")


@pytest.mark.timeout(300)
def test_one_pass_transposed_local_path(monkeypatch):
    monkeypatch.setenv("NVFP4_AMAX_POLLS", "0")
    say("one-pass transposed encoder, local path: bf16 4096x4096 both ways")
    x = _as_dtype(_tensor(77, 4096, 4096, "first"), "bf16")
    rowq, (ct, st), g = _quantize_t(x, "bf16", both=True)
    assert_every_byte(ct, st, g, np.ascontiguousarray(x.T), "x^T local path")
    assert_every_byte(rowq[0], rowq[1], g, x, "x local path")


SIGNS = 0xB5C3
# (dtype, rows, K, row padding, where the maximum is): the transform's one-pass form (taken from 4 blocks
# per thread, 16.8M elements, up to the capacity) on nGPT's and GDN's activations, the FP32 capacity, strided
# bf16 and FP32 rows; and a tensor below that size (two passes)
RHT_CASES = [("bf16", 8192, 4096, 0, "last"), ("bf16", 4096, 5120, 0, "first"), ("f32", 2048, 8192, 0, "first"),
             ("bf16", 4200, 4096, 64, "first"), ("f32", 2048, 8192, 4, "last"), ("bf16", 2048, 4112, 0, "last")]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,rows,K,ld_pad,where", RHT_CASES)
def test_one_pass_rht_every_byte(dtype, rows, K, ld_pad, where):
    """The randomized Hadamard transform before the encoding: g from the maximum of the transformed tensor,
    every code and scale byte against the oracle's encoding of its transformed blocks."""
    say(f"one-pass quantizer with RHT: {dtype} {rows}x{K} ld pad {ld_pad}, maximum in the {where} share")
    x = _as_dtype(_tensor(rows * 5 + K, rows, K, where), dtype)
    c, s, g = nv.quantize_rht(_dev(x, dtype, ld_pad), SIGNS)
    torch.cuda.synchronize()
    assert_every_byte(c, s, g, rht.rht_blocks(x, SIGNS), f"rht {dtype} {rows}x{K}")


@pytest.mark.timeout(300)
def test_one_pass_rht_local_path(monkeypatch):
    """A poll bound of zero with the transform: each workgroup reduces the transformed blocks of the whole
    tensor itself."""
    monkeypatch.setenv("NVFP4_AMAX_POLLS", "0")
    say("one-pass quantizer with RHT, local path: bf16 4096x4112")
    x = _as_dtype(_tensor(13, 4096, 4112, "first"), "bf16")
    c, s, g = nv.quantize_rht(to_dev(x, "bf16"), SIGNS)
    torch.cuda.synchronize()
    assert_every_byte(c, s, g, rht.rht_blocks(x, SIGNS), "rht local path")


# (dtype, n, k, row padding): nGPT's W [4096 x 4096] (two quarters per workgroup), the bf16 and FP32
# capacities (four quarters), strided rows, and n = 1152 (padding rows up to 1280 in the forward blob)
PACK_CASES = [("bf16", 4096, 4096, 0), ("bf16", 8192, 4096, 0), ("f32", 2048, 8192, 0), ("bf16", 4096, 2560, 64),
              ("f32", 1152, 8192, 0)]


def _check_packed(fwd, bwd, g, w, what):
    """Both blobs unpacked against the oracle's encodings of w and w^T, every byte, and every real row's
    column scale equal to g; the padding rows, column scales and headers against the separate calls."""
    for pw, x, side in ((fwd, w, "forward"), (bwd, np.ascontiguousarray(w.T), "backward")):
        c, s, cs = pw.unpack()
        torch.cuda.synchronize()
        assert_every_byte(c, s, g, x, f"{what} {side}")
        assert torch.equal(cs, g.expand_as(cs)), f"{what} {side}: column scales differ from g"


@pytest.mark.timeout(300)
@pytest.mark.parametrize("dtype,n,k,ld_pad", PACK_CASES)
def test_one_pass_pack_weights_train(dtype, n, k, ld_pad):
    """A training weight's two packed operands from registers: every code and scale against the oracle,
    every blob byte (padding included) against quantize + pack and quantize_t + pack."""
    from test_gpu_quantize_t import _blob_regions
    say(f"one-pass training-weight packer: {dtype} {n}x{k} ld pad {ld_pad}")
    w = _as_dtype(_tensor(n + 11 * k, n, k, "last"), dtype)
    wd = _dev(w, dtype, ld_pad)
    fwd, bwd, g = nv.pack_weights_train(wd)
    torch.cuda.synchronize()
    _check_packed(fwd, bwd, g, w, f"{dtype} {n}x{k}")
    ref_fwd = nv.PackedWeight([nv.quantize(wd)], k)
    ref_bwd = nv.PackedWeight([nv.quantize_t(wd)], n)
    torch.cuda.synchronize()
    for got, want, side in ((fwd, ref_fwd, "forward"), (bwd, ref_bwd, "backward")):
        for part, (a, b) in zip(["header", "codes", "scales", "colscale"], zip(_blob_regions(got), _blob_regions(want))):
            assert np.array_equal(a, b), f"{side} {part} differs from the separate calls"


@pytest.mark.timeout(300)
def test_one_pass_pack_weights_train_local_path(monkeypatch):
    monkeypatch.setenv("NVFP4_AMAX_POLLS", "0")
    say("one-pass training-weight packer, local path: bf16 4096x4096")
    w = _as_dtype(_tensor(91, 4096, 4096, "first"), "bf16")
    fwd, bwd, g = nv.pack_weights_train(to_dev(w, "bf16"))
    torch.cuda.synchronize()
    _check_packed(fwd, bwd, g, w, "local path")


def test_one_pass_graph_replays_with_changing_inputs():
    """The one-pass kernels captured in one HIP graph (row, transposed, both ways, RHT, the training-weight
    packer), replayed on three tensors of very different magnitude copied into the captured input between
    replays: every replay equals the eager calls on that tensor, so no replay takes a maximum that an
    earlier one published (the launch tags differ between replays)."""
    rows, cols = 4096, 4096
    xs = [_as_dtype((_tensor(300 + i, rows, cols, "first" if i % 2 else "last") * F32(sc)).astype(F32), "bf16")
          for i, sc in enumerate((1.0, 1e-3, 50.0))]
    xd = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    ws = [torch.empty(nv.nvfp4_quantize_workspace_bytes(rows, cols), dtype=torch.uint8, device="cuda")
          for _ in range(5)]
    blob_f = torch.zeros((nv.nvfp4_packed_weight_bytes([rows], cols),), dtype=torch.uint8, device="cuda")
    blob_b = torch.zeros((nv.nvfp4_packed_weight_bytes([cols], rows),), dtype=torch.uint8, device="cuda")

    def buffers():
        return {"q": nv.empty_quantized(rows, cols), "t": nv.empty_quantized(cols, rows),
                "b": nv.empty_quantized(rows, cols) + nv.empty_quantized(cols, rows)[:2],
                "r": nv.empty_quantized(rows, cols),      # (blobs zeroed: the alignment gaps are never written)
                "p": (torch.zeros_like(blob_f), torch.zeros_like(blob_b),
                      torch.empty((1,), dtype=torch.float32, device="cuda"))}

    def run(o, s=None):
        nv.nvfp4_quantize(xd, *o["q"], nv.NVFP4_G_COMPUTE, ws[0], stream=s)
        nv.nvfp4_quantize_t(xd, *o["t"], nv.NVFP4_G_COMPUTE, ws[1], stream=s)
        c, sc, g, ct, st = o["b"]
        nv.nvfp4_quantize_both(xd, c, sc, ct, st, g, nv.NVFP4_G_COMPUTE, ws[2], stream=s)
        nv.nvfp4_quantize_rht(xd, SIGNS, *o["r"], nv.NVFP4_G_COMPUTE, ws[3], stream=s)
        bf, bb, gp = o["p"]
        nv.nvfp4_pack_weights_train(xd, gp, bf, bb, nv.NVFP4_G_COMPUTE, ws[4], stream=s)

    def flat(o):
        return [t for v in o.values() for t in v]

    say("one-pass kernels: eager outputs of three tensors")
    want = []
    for x in xs:
        xd.copy_(torch.from_numpy(x).to(torch.bfloat16))
        o = buffers()
        run(o)
        torch.cuda.synchronize()
        want.append(o)
    assert len({float(o["q"][2].cpu()[0]) for o in want}) == 3      # three different g
    got = buffers()
    strm = torch.cuda.Stream()
    with torch.cuda.stream(strm):
        run(got, strm)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=strm):
        run(got, strm)
    for rep in range(6):
        i = (rep * 2) % 3
        say(f"one-pass kernels: replay {rep} on tensor {i}")
        xd.copy_(torch.from_numpy(xs[i]).to(torch.bfloat16))
        for t in flat(got):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in got:
            for a, b in zip(got[name], want[i][name]):
                assert torch.equal(a, b), f"replay {rep} (tensor {i}): {name} differs from the eager call"
        run(buffers())                      # eager calls between replays share the workspaces
