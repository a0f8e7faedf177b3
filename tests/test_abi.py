"""The C-ABI library on the host: it loads, exports every function include/nvfp4.h
declares, and validates arguments before touching a device.  No GPU needed:
pointers here are fake but never dereferenced, because every call either fails
validation or (with no GPU present) stops at the device check."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")
LIB = os.environ.get("NVFP4_LIBRARY") or os.path.join(ROOT, "nvfp4_block_scaled_03_amd", "libnvfp4.so")


def _ensure_built():
    if not os.path.exists(LIB):   # build.py by path: the package refuses to import before the library exists
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_nvfp4_build", os.path.join(ROOT, "nvfp4_block_scaled_03_amd", "build.py"))
        b = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(b)
        b.build()


_ensure_built()
import nvfp4_block_scaled_03_amd as nv  # noqa: E402

FAKE = 1 << 20  # 256-byte aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = "\n".join(l for l in text.splitlines() if not l.lstrip().startswith("#"))
    names = set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["nvfp4_quantize", "nvfp4_pack_weights", "nvfp4_gemm", "nvfp4_last_error",
                     "nvfp4_quantize_workspace_bytes", "nvfp4_packed_weight_bytes", "nvfp4_unpack_weights",
                     "nvfp4_gemm_workspace_bytes", "nvfp4_abi_version", "nvfp4_device_check", "nvfp4_quantize_t", "nvfp4_quantize_rht", "nvfp4_quantize_t_rht",
                     "nvfp4_gemm_ex", "nvfp4_linear_ex", "nvfp4_kv_quantize_fp8", "nvfp4_quantize_both",
                     "nvfp4_pack_weights_train"]:
        assert required in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(LIB)
    for n in declared_functions():
        getattr(lib, n)


def test_abi_version():
    assert nv.lib.nvfp4_abi_version() == 1


def _no_gpu():
    return nv.device_check() == nv.NVFP4_ERR_NO_DEVICE


def q(**kw):
    args = dict(x=FAKE, in_dtype=nv.NVFP4_IN_BF16, rows=4, K=64, ld_x=64, codes=FAKE, scales=FAKE, g=FAKE,
                g_mode=nv.NVFP4_G_COMPUTE, ws=FAKE, ws_bytes=1 << 16)
    args.update(kw)
    return nv.lib.nvfp4_quantize(args["x"], args["in_dtype"], args["rows"], args["K"], args["ld_x"], args["codes"],
                                 args["scales"], args["g"], args["g_mode"], args["ws"], args["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(in_dtype=7), nv.NVFP4_ERR_INVALID_ARG),
    (dict(g_mode=3), nv.NVFP4_ERR_INVALID_ARG),
    (dict(g=None), nv.NVFP4_ERR_INVALID_ARG),
    (dict(x=None), nv.NVFP4_ERR_INVALID_ARG),
    (dict(codes=None), nv.NVFP4_ERR_INVALID_ARG),
    (dict(K=0), nv.NVFP4_ERR_SHAPE),
    (dict(K=24, ld_x=24), nv.NVFP4_ERR_SHAPE),
    (dict(rows=-1), nv.NVFP4_ERR_SHAPE),
    (dict(ld_x=32), nv.NVFP4_ERR_SHAPE),
    (dict(x=FAKE + 2), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(ld_x=68), nv.NVFP4_ERR_UNSUPPORTED),            # bf16 row stride not a multiple of 16 bytes
    (dict(codes=FAKE + 4), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(ws=None), nv.NVFP4_ERR_WORKSPACE),
    (dict(ws_bytes=0), nv.NVFP4_ERR_WORKSPACE),
])
def test_quantize_validation(kw, status):
    assert q(**kw) == status
    assert nv.last_error() != ""


def test_quantize_given_mode_needs_no_workspace():
    if not _no_gpu():
        pytest.skip("a GPU is visible; this host-only check would launch on fake pointers")
    assert q(ws=None, ws_bytes=0, g_mode=nv.NVFP4_G_GIVEN) == nv.NVFP4_ERR_NO_DEVICE


def test_valid_calls_stop_at_device_check_without_gpu():
    if not _no_gpu():
        pytest.skip("a GPU is visible; this host-only check would launch on fake pointers")
    assert q() == nv.NVFP4_ERR_NO_DEVICE
    assert "device" in nv.last_error()


def qt(**kw):
    args = dict(x=FAKE, in_dtype=nv.NVFP4_IN_BF16, rows=32, cols=40, ld_x=40, codes=FAKE, scales=FAKE, g=FAKE,
                g_mode=nv.NVFP4_G_COMPUTE, ws=FAKE, ws_bytes=1 << 16)
    args.update(kw)
    return nv.lib.nvfp4_quantize_t(args["x"], args["in_dtype"], args["rows"], args["cols"], args["ld_x"],
                                   args["codes"], args["scales"], args["g"], args["g_mode"], args["ws"],
                                   args["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(in_dtype=7), nv.NVFP4_ERR_INVALID_ARG),
    (dict(g_mode=3), nv.NVFP4_ERR_INVALID_ARG),
    (dict(g=None), nv.NVFP4_ERR_INVALID_ARG),
    (dict(x=None), nv.NVFP4_ERR_INVALID_ARG),
    (dict(scales=None), nv.NVFP4_ERR_INVALID_ARG),
    (dict(rows=24), nv.NVFP4_ERR_SHAPE),                  # the blocked axis is rows
    (dict(rows=-16), nv.NVFP4_ERR_SHAPE),
    (dict(cols=-1), nv.NVFP4_ERR_SHAPE),
    (dict(ld_x=32), nv.NVFP4_ERR_SHAPE),
    (dict(x=FAKE + 1), nv.NVFP4_ERR_UNSUPPORTED),          # bf16 elements not 2-byte aligned
    (dict(x=FAKE + 2, in_dtype=nv.NVFP4_IN_F32), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(codes=FAKE + 4), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(ws=None), nv.NVFP4_ERR_WORKSPACE),
    (dict(ws_bytes=0), nv.NVFP4_ERR_WORKSPACE),
])
def test_quantize_t_validation(kw, status):
    assert qt(**kw) == status
    assert nv.last_error() != ""


def test_quantize_t_valid_calls_stop_at_device_check_without_gpu():
    if not _no_gpu():
        pytest.skip("a GPU is visible; this host-only check would launch on fake pointers")
    assert qt() == nv.NVFP4_ERR_NO_DEVICE
    assert qt(rows=0, cols=0, x=None, codes=None, scales=None) == nv.NVFP4_ERR_NO_DEVICE   # empty is valid
    assert qt(ws=None, ws_bytes=0, g_mode=nv.NVFP4_G_GIVEN, cols=13, ld_x=16) == nv.NVFP4_ERR_NO_DEVICE
    assert qt(ld_x=43, x=FAKE + 2) == nv.NVFP4_ERR_NO_DEVICE      # any element-aligned layout is accepted


def test_rht_validation():
    args = (FAKE, nv.NVFP4_IN_BF16, 32, 64, 64)
    tail = (FAKE, FAKE, FAKE, nv.NVFP4_G_COMPUTE, FAKE, 1 << 16, None)
    assert nv.lib.nvfp4_quantize_rht(*args, 1 << 16, *tail) == nv.NVFP4_ERR_INVALID_ARG
    assert "16-bit" in nv.last_error()
    assert nv.lib.nvfp4_quantize_t_rht(*args, 0x12345, *tail) == nv.NVFP4_ERR_INVALID_ARG
    assert nv.lib.nvfp4_quantize_rht(FAKE, nv.NVFP4_IN_BF16, 32, 40, 40, 7, *tail) == nv.NVFP4_ERR_SHAPE
    assert nv.lib.nvfp4_quantize_t_rht(FAKE, nv.NVFP4_IN_BF16, 40, 64, 64, 7, *tail) == nv.NVFP4_ERR_SHAPE
    if _no_gpu():
        assert nv.lib.nvfp4_quantize_rht(*args, 0xFFFF, *tail) == nv.NVFP4_ERR_NO_DEVICE
        assert nv.lib.nvfp4_quantize_t_rht(*args, 0, *tail) == nv.NVFP4_ERR_NO_DEVICE


def test_workspace_query():
    assert nv.nvfp4_quantize_workspace_bytes(16, 5120) >= 4
    assert nv.nvfp4_quantize_workspace_bytes(32768, 16384) % 256 == 0
    assert nv.nvfp4_quantize_workspace_bytes(32768, 16384) <= 1024 * 4
    assert nv.nvfp4_quantize_workspace_bytes(-1, 16) == 0


def expected_blob_bytes(rows, K):
    n = sum(rows)
    n_pad = (n + 255) // 256 * 256
    scales_off = 256 + n_pad * K // 2
    colscale_off = (scales_off + n_pad * K // 16 + 255) // 256 * 256
    return colscale_off + n_pad * 4


@pytest.mark.parametrize("rows,K", [([5120], 5120), ([4096, 4096, 4096, 4096, 48, 48], 5120), ([256], 512),
                                    ([16384], 16384), ([1], 128), ([100, 37, 48], 640)])
def test_packed_weight_bytes(rows, K):
    got = nv.nvfp4_packed_weight_bytes(rows, K)
    assert got == expected_blob_bytes(rows, K)
    # 4.5 bits per weight element, plus the header, padding rows and one FP32 per row
    n_pad = (sum(rows) + 255) // 256 * 256
    assert got >= n_pad * K * 9 // 16


@pytest.mark.parametrize("rows,K", [([], 512), ([0], 512), ([16], 100), ([16], 144), ([1] * 17, 128)])
def test_packed_weight_bytes_invalid(rows, K):
    assert nv.nvfp4_packed_weight_bytes(rows, K) == 0


def _pack(n_modules=1, rows=(64,), K=256, blob=FAKE, blob_bytes=1 << 30, codes=FAKE, scales=FAKE, g=FAKE):
    n = len(rows)
    r = (ctypes.c_int64 * max(n, 1))(*rows)
    cp = (ctypes.c_void_p * max(n, 1))(*([codes] * max(n, 1)))
    sp = (ctypes.c_void_p * max(n, 1))(*([scales] * max(n, 1)))
    gp = (ctypes.c_void_p * max(n, 1))(*([g] * max(n, 1)))
    d = nv.WeightDesc()
    return nv.lib.nvfp4_pack_weights(n_modules, r, K, cp, sp, gp, blob, blob_bytes, ctypes.byref(d), None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_modules=0, rows=()), nv.NVFP4_ERR_INVALID_ARG),
    (dict(n_modules=17, rows=(1,) * 17), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(rows=(0,)), nv.NVFP4_ERR_SHAPE),
    (dict(K=100), nv.NVFP4_ERR_SHAPE),
    (dict(K=144), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(codes=None), nv.NVFP4_ERR_INVALID_ARG),
    (dict(codes=FAKE + 8), nv.NVFP4_ERR_UNSUPPORTED),
    (dict(blob=None), nv.NVFP4_ERR_INVALID_ARG),
    (dict(blob=FAKE + 16), nv.NVFP4_ERR_INVALID_ARG),
    (dict(blob_bytes=1000), nv.NVFP4_ERR_WORKSPACE),
])
def test_pack_validation(kw, status):
    assert _pack(**kw) == status


def make_desc(rows=(100, 37, 48), K=640, blob=FAKE):
    d = nv.WeightDesc()
    n = sum(rows)
    d.magic, d.version = nv.NVFP4_WEIGHT_MAGIC, nv.NVFP4_WEIGHT_VERSION
    d.n, d.k, d.n_padded, d.n_modules = n, K, (n + 255) // 256 * 256, len(rows)
    off = 0
    for i, r in enumerate(rows):
        d.module_rows[i], d.module_row_offset[i] = r, off
        off += r
    d.blob = blob
    d.codes_offset = 256
    d.scales_offset = 256 + d.n_padded * K // 2
    d.colscale_offset = (d.scales_offset + d.n_padded * K // 16 + 255) // 256 * 256
    d.blob_bytes = d.colscale_offset + d.n_padded * 4
    return d


def g_(M=32, d=None, a=FAKE, s=FAKE, gx=FAKE, y=FAKE, ld_y=None, ws=None, ws_bytes=0):
    d = make_desc() if d is None else d
    return nv.lib.nvfp4_gemm(M, a, s, gx, ctypes.byref(d) if d is not False else None, y,
                             d.n if ld_y is None else ld_y, ws, ws_bytes, None)


def test_gemm_validation():
    assert g_(M=-1) == nv.NVFP4_ERR_SHAPE
    assert g_(M=0) == nv.NVFP4_OK                     # empty: nothing to do
    assert g_(y=None) == nv.NVFP4_ERR_INVALID_ARG
    assert g_(a=None) == nv.NVFP4_ERR_INVALID_ARG
    assert g_(ld_y=100) == nv.NVFP4_ERR_SHAPE
    assert g_(a=FAKE + 4) == nv.NVFP4_ERR_UNSUPPORTED
    assert nv.lib.nvfp4_gemm(4, FAKE, FAKE, FAKE, None, FAKE, 1000, None, 0, None) == nv.NVFP4_ERR_INVALID_ARG
    d = make_desc()
    d.magic = 0
    assert g_(d=d) == nv.NVFP4_ERR_DESCRIPTOR
    d = make_desc()
    d.version = 9
    assert g_(d=d) == nv.NVFP4_ERR_DESCRIPTOR
    d = make_desc()
    d.n = 999
    assert g_(d=d) == nv.NVFP4_ERR_DESCRIPTOR
    d = make_desc()
    d.module_row_offset[1] = 5
    assert g_(d=d) == nv.NVFP4_ERR_DESCRIPTOR
    d = make_desc(blob=FAKE + 64)
    assert g_(d=d) == nv.NVFP4_ERR_DESCRIPTOR
    assert nv.lib.nvfp4_unpack_weights(None, FAKE, FAKE, FAKE, None) == nv.NVFP4_ERR_INVALID_ARG


def test_operand_size_limit():
    """The products address codes with 32-bit byte offsets: activation codes of exactly 2 GiB pass the
    checks, one row more is refused before any launch; a weight whose padded codes pass 2 GiB has no
    packed size."""
    d = make_desc(K=640)                      # 320 code bytes per row
    m_max = (1 << 31) // 320
    assert g_(M=m_max + 1, d=d) == nv.NVFP4_ERR_UNSUPPORTED
    if _no_gpu():
        assert g_(M=m_max, d=d) == nv.NVFP4_ERR_NO_DEVICE
    assert nv.nvfp4_packed_weight_bytes([1 << 18], 16384) > 0       # 262144 x 16384: exactly 2 GiB of codes
    assert nv.nvfp4_packed_weight_bytes([(1 << 18) + 1], 16384) == 0


def test_gemm_valid_stops_at_device_check_without_gpu():
    if not _no_gpu():
        pytest.skip("a GPU is visible; this host-only check would launch on fake pointers")
    assert g_() == nv.NVFP4_ERR_NO_DEVICE


def test_linear_validation():
    d = make_desc(rows=(5120,), K=5120)
    need = nv.lib.nvfp4_linear_workspace_bytes(16, nv.NVFP4_IN_BF16, ctypes.byref(d))
    # the one-launch path's per-XCD flags (8 x 256 bytes) and its product-order copy of the activation
    # encoding (40 k-steps x 1152 bytes, rounded to 256), then the two-launch path's amax partials
    assert need == 2048 + 46080 + nv.nvfp4_quantize_workspace_bytes(16, 5120)
    assert nv.lib.nvfp4_gemm_workspace_bytes(16, ctypes.byref(d)) == 0      # the product alone needs none

    def call(**kw):
        a = dict(x=FAKE, dt=nv.NVFP4_IN_BF16, M=16, ld_x=5120, c=FAKE, s=FAKE, g=FAKE, mode=0, d=d, y=FAKE,
                 ld_y=5120, ws=FAKE, wsb=need)
        a.update(kw)
        return nv.lib.nvfp4_linear(a["x"], a["dt"], a["M"], a["ld_x"], a["c"], a["s"], a["g"], a["mode"],
                                   ctypes.byref(a["d"]) if a["d"] is not None else None, a["y"], a["ld_y"],
                                   a["ws"], a["wsb"], None)
    assert call(dt=5) == nv.NVFP4_ERR_INVALID_ARG
    assert call(mode=9) == nv.NVFP4_ERR_INVALID_ARG
    assert call(M=-1) == nv.NVFP4_ERR_SHAPE
    assert call(ld_x=100) == nv.NVFP4_ERR_SHAPE
    assert call(ld_y=100) == nv.NVFP4_ERR_SHAPE
    assert call(y=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(x=FAKE + 8) == nv.NVFP4_ERR_UNSUPPORTED
    assert call(ws=None) == nv.NVFP4_ERR_WORKSPACE
    assert call(wsb=need - 1) == nv.NVFP4_ERR_WORKSPACE
    assert call(d=None) == nv.NVFP4_ERR_INVALID_ARG
    if _no_gpu():
        assert call() == nv.NVFP4_ERR_NO_DEVICE


def test_gated_validation():
    """The gate epilogue's arguments are checked on the host before anything is launched."""
    d = make_desc()          # n = sum of the module rows

    def gg(a_col=0, n_a=4, b_col=8, n_b=4, a_log=FAKE, dt_bias=FAKE, gates=True):
        g = nv.GdnGatesDesc(a_col, n_a, b_col, n_b, a_log, dt_bias)
        return nv.lib.nvfp4_gemm_gated(32, FAKE, FAKE, FAKE, ctypes.byref(d), ctypes.byref(g) if gates else None,
                                       FAKE, d.n, None, 0, None)
    assert gg(gates=False) == nv.NVFP4_ERR_INVALID_ARG
    assert gg(a_log=None) == nv.NVFP4_ERR_INVALID_ARG
    assert gg(dt_bias=None) == nv.NVFP4_ERR_INVALID_ARG
    assert gg(n_a=-1) == nv.NVFP4_ERR_SHAPE
    assert gg(a_col=d.n - 2) == nv.NVFP4_ERR_SHAPE             # runs past the last column
    assert gg(b_col=d.n) == nv.NVFP4_ERR_SHAPE
    assert gg(b_col=2) == nv.NVFP4_ERR_SHAPE                   # overlaps the decay columns
    assert gg(a_log=FAKE + 2) == nv.NVFP4_ERR_UNSUPPORTED
    assert gg(n_a=0, a_log=None, dt_bias=None) != nv.NVFP4_ERR_INVALID_ARG   # no decay columns: no parameters
    g = nv.GdnGatesDesc(0, 4, 8, 4, FAKE, FAKE)
    assert nv.lib.nvfp4_linear_gated(FAKE, nv.NVFP4_IN_BF16, 16, d.k, FAKE, FAKE, FAKE, 0, ctypes.byref(d), None,
                                     FAKE, d.n, FAKE, 1 << 30, None) == nv.NVFP4_ERR_INVALID_ARG
    if _no_gpu():
        assert gg() == nv.NVFP4_ERR_NO_DEVICE
        assert nv.lib.nvfp4_linear_gated(FAKE, nv.NVFP4_IN_BF16, 16, d.k, FAKE, FAKE, FAKE, 0, ctypes.byref(d),
                                         ctypes.byref(g), FAKE, d.n, FAKE, 1 << 30, None) == nv.NVFP4_ERR_NO_DEVICE


def test_epilogue_validation():
    """The output epilogue (y type, reserved field, gates) is checked on the host before any launch."""
    d = make_desc()
    g = nv.GdnGatesDesc(0, 4, 8, 4, FAKE, FAKE)

    def ge(y_dtype=nv.NVFP4_OUT_BF16, reserved=0, gates=None, y=FAKE, ep=True):
        e = nv.EpilogueDesc(y_dtype, reserved, ctypes.addressof(gates) if gates is not None else None)
        return nv.lib.nvfp4_gemm_ex(32, FAKE, FAKE, FAKE, ctypes.byref(d), ctypes.byref(e) if ep else None, y, d.n,
                                    None, 0, None)
    assert ge(ep=False) == nv.NVFP4_ERR_INVALID_ARG
    assert ge(y_dtype=2) == nv.NVFP4_ERR_INVALID_ARG
    assert ge(reserved=1) == nv.NVFP4_ERR_INVALID_ARG
    assert ge(gates=nv.GdnGatesDesc(0, 4, 2, 4, FAKE, FAKE)) == nv.NVFP4_ERR_SHAPE   # overlapping gate columns
    assert ge(y=FAKE + 1) == nv.NVFP4_ERR_UNSUPPORTED                                 # bf16 y needs 2-byte alignment
    assert ge(y_dtype=nv.NVFP4_OUT_F32, y=FAKE + 2) == nv.NVFP4_ERR_UNSUPPORTED       # FP32 y needs 4
    e = nv.EpilogueDesc(nv.NVFP4_OUT_BF16, 0, None)
    assert nv.lib.nvfp4_linear_ex(FAKE, nv.NVFP4_IN_BF16, 16, d.k, FAKE, FAKE, FAKE, 0, ctypes.byref(d), None,
                                  FAKE, d.n, FAKE, 1 << 30, None) == nv.NVFP4_ERR_INVALID_ARG
    if _no_gpu():
        assert ge(y=FAKE + 2) == nv.NVFP4_ERR_NO_DEVICE
        assert ge(gates=g) == nv.NVFP4_ERR_NO_DEVICE
        assert nv.lib.nvfp4_linear_ex(FAKE, nv.NVFP4_IN_BF16, 16, d.k, FAKE, FAKE, FAKE, 0, ctypes.byref(d),
                                      ctypes.byref(e), FAKE + 2, d.n, FAKE, 1 << 30, None) == nv.NVFP4_ERR_NO_DEVICE


def test_kv_fp8_validation():
    def kv(**kw):
        a = dict(x=FAKE, in_dtype=nv.NVFP4_IN_BF16, rows=16, cols=40, ld_x=40, codes=FAKE, scale=FAKE,
                 s_mode=nv.NVFP4_G_COMPUTE, ws=FAKE, ws_bytes=1 << 16)
        a.update(kw)
        return nv.lib.nvfp4_kv_quantize_fp8(a["x"], a["in_dtype"], a["rows"], a["cols"], a["ld_x"], a["codes"],
                                            a["scale"], a["s_mode"], a["ws"], a["ws_bytes"], None)
    assert kv(in_dtype=9) == nv.NVFP4_ERR_INVALID_ARG
    assert kv(s_mode=5) == nv.NVFP4_ERR_INVALID_ARG
    assert kv(scale=None) == nv.NVFP4_ERR_INVALID_ARG
    assert kv(codes=None) == nv.NVFP4_ERR_INVALID_ARG
    assert kv(rows=-1) == nv.NVFP4_ERR_SHAPE
    assert kv(ld_x=39) == nv.NVFP4_ERR_SHAPE
    assert kv(x=FAKE + 1) == nv.NVFP4_ERR_UNSUPPORTED
    assert kv(ws=None) == nv.NVFP4_ERR_WORKSPACE
    if _no_gpu():
        assert kv() == nv.NVFP4_ERR_NO_DEVICE
        assert kv(ws=None, ws_bytes=0, s_mode=nv.NVFP4_G_GIVEN, cols=7, ld_x=9, x=FAKE + 2) == nv.NVFP4_ERR_NO_DEVICE
        assert kv(rows=0, x=None, codes=None) == nv.NVFP4_ERR_NO_DEVICE


def test_quantize_both_validation():
    def qb(**kw):
        a = dict(x=FAKE, in_dtype=nv.NVFP4_IN_BF16, rows=32, cols=48, ld_x=48, c=FAKE, s=FAKE, ct=FAKE, st=FAKE,
                 g=FAKE, g_mode=nv.NVFP4_G_COMPUTE, ws=FAKE, ws_bytes=1 << 16)
        a.update(kw)
        return nv.lib.nvfp4_quantize_both(a["x"], a["in_dtype"], a["rows"], a["cols"], a["ld_x"], a["c"], a["s"],
                                          a["ct"], a["st"], a["g"], a["g_mode"], a["ws"], a["ws_bytes"], None)
    assert qb(in_dtype=3) == nv.NVFP4_ERR_INVALID_ARG
    assert qb(g=None) == nv.NVFP4_ERR_INVALID_ARG
    assert qb(ct=None) == nv.NVFP4_ERR_INVALID_ARG
    assert qb(rows=24) == nv.NVFP4_ERR_SHAPE
    assert qb(cols=40, ld_x=40) == nv.NVFP4_ERR_SHAPE
    assert qb(ld_x=32) == nv.NVFP4_ERR_SHAPE
    assert qb(c=FAKE + 2) == nv.NVFP4_ERR_UNSUPPORTED
    assert qb(ct=FAKE + 4) == nv.NVFP4_ERR_UNSUPPORTED
    assert qb(ws_bytes=0) == nv.NVFP4_ERR_WORKSPACE
    if _no_gpu():
        assert qb() == nv.NVFP4_ERR_NO_DEVICE
        assert qb(ld_x=50, x=FAKE + 2, ws=None, ws_bytes=0, g_mode=nv.NVFP4_G_GIVEN) == nv.NVFP4_ERR_NO_DEVICE


def test_pack_weights_train_validation():
    df, db = nv.WeightDesc(), nv.WeightDesc()

    def pt(**kw):
        a = dict(w=FAKE, in_dtype=nv.NVFP4_IN_BF16, n=256, k=384, ld=384, g=FAKE, g_mode=nv.NVFP4_G_COMPUTE,
                 bf=FAKE, bfb=1 << 30, df=ctypes.byref(df), bb=FAKE, bbb=1 << 30, db=ctypes.byref(db), ws=FAKE,
                 wsb=1 << 16)
        a.update(kw)
        return nv.lib.nvfp4_pack_weights_train(a["w"], a["in_dtype"], a["n"], a["k"], a["ld"], a["g"], a["g_mode"],
                                               a["bf"], a["bfb"], a["df"], a["bb"], a["bbb"], a["db"], a["ws"],
                                               a["wsb"], None)
    assert pt(in_dtype=5) == nv.NVFP4_ERR_INVALID_ARG
    assert pt(g=None) == nv.NVFP4_ERR_INVALID_ARG
    assert pt(df=None) == nv.NVFP4_ERR_INVALID_ARG
    assert pt(n=200) == nv.NVFP4_ERR_SHAPE                  # the backward blob's K must be a multiple of 128
    assert pt(k=400, ld=400) == nv.NVFP4_ERR_SHAPE
    assert pt(ld=300) == nv.NVFP4_ERR_SHAPE
    assert pt(w=FAKE + 1) == nv.NVFP4_ERR_UNSUPPORTED
    assert pt(bf=FAKE + 16) == nv.NVFP4_ERR_INVALID_ARG     # blobs 256-byte aligned
    assert pt(bfb=1024) == nv.NVFP4_ERR_WORKSPACE
    assert pt(bbb=1024) == nv.NVFP4_ERR_WORKSPACE
    assert pt(ws=None) == nv.NVFP4_ERR_WORKSPACE
    if _no_gpu():
        assert pt() == nv.NVFP4_ERR_NO_DEVICE
        assert pt(ws=None, wsb=0, g_mode=nv.NVFP4_G_GIVEN, ld=390, w=FAKE + 2) == nv.NVFP4_ERR_NO_DEVICE


def test_linear_noalloc_validation():
    """The allocation-free layer call validates like nvfp4_linear (no workspace argument to check) and, with
    no GPU, stops at the device check before it looks up or touches its static scratch."""
    d = make_desc(rows=(5120,), K=5120)

    def call(**kw):
        a = dict(x=FAKE, dt=nv.NVFP4_IN_BF16, M=16, ld_x=5120, c=FAKE, s=FAKE, g=FAKE, mode=0, d=d, y=FAKE,
                 ld_y=5120)
        a.update(kw)
        return nv.lib.nvfp4_linear_noalloc(a["x"], a["dt"], a["M"], a["ld_x"], a["c"], a["s"], a["g"], a["mode"],
                                           ctypes.byref(a["d"]) if a["d"] is not None else None, a["y"],
                                           a["ld_y"], None)
    assert call(d=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(dt=5) == nv.NVFP4_ERR_INVALID_ARG
    assert call(mode=9) == nv.NVFP4_ERR_INVALID_ARG
    assert call(M=-1) == nv.NVFP4_ERR_SHAPE
    assert call(ld_x=100) == nv.NVFP4_ERR_SHAPE
    assert call(ld_y=100) == nv.NVFP4_ERR_SHAPE
    assert call(y=None) == nv.NVFP4_ERR_INVALID_ARG
    assert call(x=FAKE + 8) == nv.NVFP4_ERR_UNSUPPORTED
    # every shape's workspace fits the static scratch (80 KiB), the few-token part first for every M
    assert nv.lib.nvfp4_linear_workspace_bytes(300, nv.NVFP4_IN_BF16, ctypes.byref(d)) == \
        2048 + 46080 + nv.nvfp4_quantize_workspace_bytes(300, 5120)
    for M, K in [(16, 5120), (1, 128), (32768, 16384), (300, 8192), (4096, 5120), (16, 8192), (16, 8320)]:
        dd = make_desc(rows=(256,), K=K)
        assert nv.lib.nvfp4_linear_workspace_bytes(M, nv.NVFP4_IN_F32, ctypes.byref(dd)) <= 81920
    if _no_gpu():
        assert call() == nv.NVFP4_ERR_NO_DEVICE
