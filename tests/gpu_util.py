"""Helpers for the GPU parity tests: host <-> device marshalling and oracle comparisons."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import nvfp4_ref as ref

DEV = torch.device("cuda:0")


def say(msg):
    """Print and flush what names the case before a GPU step."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """FP32 host values (bf16-exact when dtype == 'bf16') -> device tensor of that dtype."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
        assert torch.equal(t.float(), torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))), \
            "input is not bf16-representable"
    return t.to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_quant_equal(codes, scales, g, oq, rows=None, what=""):
    """Bit-exact comparison of device codes/scales/g with an oracle Quantized (optionally on a row subset)."""
    c = host(codes) if rows is None else host(codes[rows])
    s = host(scales) if rows is None else host(scales[rows])
    gv = np.float32(host(g)[0])
    assert gv.tobytes() == np.float32(oq.g).tobytes(), f"{what}: g {gv!r} != oracle {oq.g!r}"
    if not np.array_equal(s, oq.scales):
        bad = np.argwhere(s != oq.scales)
        r, b = bad[0]
        raise AssertionError(f"{what}: {len(bad)} scale bytes differ, first at row {r} block {b}: "
                             f"gpu 0x{s[r, b]:02x} oracle 0x{oq.scales[r, b]:02x}")
    if not np.array_equal(c, oq.codes):
        bad = np.argwhere(c != oq.codes)
        r, j = bad[0]
        raise AssertionError(f"{what}: {len(bad)} code bytes differ, first at row {r} byte {j}: "
                             f"gpu 0x{c[r, j]:02x} oracle 0x{oq.codes[r, j]:02x}")


def oracle_quantize_rows(x: np.ndarray, rows, g_mode="compute", g=None):
    """Oracle quantization of a row subset with the global scale of the whole tensor."""
    if g_mode == "compute":
        g = ref.global_scale(np.float32(np.max(np.abs(x))) if x.size else np.float32(0))
    return ref.quantize(x[rows], g_mode="given", g=g)


CHUNK_ROWS = 256


def oracle_threads():
    """Host threads for chunked oracle runs (numpy releases the interpreter lock in its array operations)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _oracle_chunks(x, g, chunk=CHUNK_ROWS):
    """Oracle quantization of row chunks of x with the tensor scale g, yielded as (r0, Quantized) in order."""
    starts = range(0, x.shape[0], chunk)
    with ThreadPoolExecutor(oracle_threads()) as ex:
        yield from zip(starts, ex.map(lambda r0: ref.quantize(x[r0:r0 + chunk], "given", g), starts))


def oracle_quantize_whole(x):
    """Oracle quantization of the whole tensor (g from its amax), assembled from row chunks."""
    g = ref.global_scale(np.float32(np.max(np.abs(x))) if x.size else np.float32(0))
    codes = np.empty((x.shape[0], x.shape[1] // 2), np.uint8)
    scales = np.empty((x.shape[0], x.shape[1] // 16), np.uint8)
    for r0, q in _oracle_chunks(x, g):
        codes[r0:r0 + q.codes.shape[0]] = q.codes
        scales[r0:r0 + q.scales.shape[0]] = q.scales
    return ref.Quantized(codes, scales, g)


def assert_every_byte(codes, scales, g, x, what):
    """Device codes/scales/g of x against the oracle, every byte, chunk by chunk."""
    c, s, gv = host(codes), host(scales), np.float32(host(g)[0])
    g_ref = ref.global_scale(np.float32(np.max(np.abs(x))) if x.size else np.float32(0))
    assert gv.tobytes() == np.float32(g_ref).tobytes(), f"{what}: g {gv!r} != oracle {g_ref!r}"
    for r0, q in _oracle_chunks(x, g_ref):
        r1 = r0 + q.codes.shape[0]
        if not np.array_equal(s[r0:r1], q.scales):
            r, b = np.argwhere(s[r0:r1] != q.scales)[0]
            raise AssertionError(f"{what}: scale byte differs at row {r0 + r} block {b}: "
                                 f"gpu 0x{s[r0 + r, b]:02x} oracle 0x{q.scales[r, b]:02x}")
        if not np.array_equal(c[r0:r1], q.codes):
            r, j = np.argwhere(c[r0:r1] != q.codes)[0]
            raise AssertionError(f"{what}: code byte differs at row {r0 + r} byte {j}: "
                                 f"gpu 0x{c[r0 + r, j]:02x} oracle 0x{q.codes[r, j]:02x}")
