"""Python binding of libnvfp4 (include/nvfp4.h): argument marshalling only.

Every computation runs in the HIP kernels of the shared library; this module
turns torch tensors into device pointers and the current HIP stream, checks
the returned status and raises ``NVFP4Error`` on failure.  It never computes
anything itself and has no fallback: if the library is missing, importing
this package raises.

The functions mirror the C entry points (``nvfp4_quantize``,
``nvfp4_pack_weights``, ``nvfp4_gemm`` ...) and take the output tensors as
arguments.  ``quantize``, ``PackedWeight`` and ``gemm`` are conveniences that
allocate outputs with torch before calling the same entry points.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# The library next to this file; NVFP4_LIBRARY names another build of the same sources (an instrumented
# build of the host code, say).
LIB_PATH = os.environ.get("NVFP4_LIBRARY") or os.path.join(_HERE, "libnvfp4.so")

NVFP4_OK = 0
NVFP4_ERR_INVALID_ARG = 1
NVFP4_ERR_SHAPE = 2
NVFP4_ERR_WORKSPACE = 3
NVFP4_ERR_UNSUPPORTED = 4
NVFP4_ERR_NO_DEVICE = 5
NVFP4_ERR_HIP = 6
NVFP4_ERR_DESCRIPTOR = 7

NVFP4_IN_F32 = 0
NVFP4_IN_BF16 = 1
NVFP4_G_COMPUTE = 0
NVFP4_G_GIVEN = 1
NVFP4_MAX_MODULES = 16
NVFP4_WEIGHT_MAGIC = 0x34504656
NVFP4_WEIGHT_VERSION = 1


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"nvfp4 status {status}: {message}")
        self.status = status


class WeightDesc(ctypes.Structure):
    """Mirror of ``nvfp4_weight_desc``."""
    _fields_ = [
        ("magic", ctypes.c_uint32),
        ("version", ctypes.c_uint32),
        ("n", ctypes.c_int64),
        ("k", ctypes.c_int64),
        ("n_padded", ctypes.c_int64),
        ("n_modules", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("module_rows", ctypes.c_int64 * NVFP4_MAX_MODULES),
        ("module_row_offset", ctypes.c_int64 * NVFP4_MAX_MODULES),
        ("blob", ctypes.c_void_p),
        ("blob_bytes", ctypes.c_size_t),
        ("codes_offset", ctypes.c_size_t),
        ("scales_offset", ctypes.c_size_t),
        ("colscale_offset", ctypes.c_size_t),
    ]


class GdnGatesDesc(ctypes.Structure):
    """Mirror of ``nvfp4_gdn_gates``."""
    _fields_ = [
        ("a_col", ctypes.c_int64),
        ("n_a", ctypes.c_int64),
        ("b_col", ctypes.c_int64),
        ("n_b", ctypes.c_int64),
        ("a_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
    ]


class GdnGates:
    """Gate epilogue of a fused Gated DeltaNet projection: decay columns [a_col, a_col + n_a) become
    exp(-exp(a_log[h]) * softplus(y + dt_bias[h])), write-strength columns [b_col, b_col + n_b) become
    sigmoid(y).  a_log and dt_bias are FP32 device tensors of n_a values (kept alive by this object)."""

    def __init__(self, a_col: int, n_a: int, b_col: int, n_b: int, a_log: torch.Tensor, dt_bias: torch.Tensor):
        self.a_log = a_log.contiguous().float()
        self.dt_bias = dt_bias.contiguous().float()
        self.desc = GdnGatesDesc(a_col, n_a, b_col, n_b, self.a_log.data_ptr(), self.dt_bias.data_ptr())


NVFP4_OUT_F32 = 0
NVFP4_OUT_BF16 = 1


class EpilogueDesc(ctypes.Structure):
    """Mirror of ``nvfp4_epilogue``."""
    _fields_ = [("y_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32), ("gates", ctypes.c_void_p)]


def _epilogue(y, gates):
    """The nvfp4_epilogue for y's dtype and the optional gates (whose descriptor the caller keeps alive)."""
    if y.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("y must be float32 or bfloat16")
    ep = EpilogueDesc(NVFP4_OUT_BF16 if y.dtype == torch.bfloat16 else NVFP4_OUT_F32, 0,
                      ctypes.addressof(gates.desc) if gates is not None else None)
    return ep


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python nvfp4_block_scaled_03_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    c_i64, c_sz, c_vp, c_int = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int
    sig = {
        "nvfp4_abi_version": (c_int, []),
        "nvfp4_last_error": (ctypes.c_char_p, []),
        "nvfp4_device_check": (c_int, []),
        "nvfp4_quantize_workspace_bytes": (c_sz, [c_i64, c_i64]),
        "nvfp4_quantize": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_int, c_vp, c_sz, c_vp]),
        "nvfp4_quantize_t": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_int, c_vp, c_sz, c_vp]),
        "nvfp4_pack_weights_train": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_int, c_vp, c_sz,
                                             ctypes.POINTER(WeightDesc), c_vp, c_sz, ctypes.POINTER(WeightDesc), c_vp,
                                             c_sz, c_vp]),
        "nvfp4_quantize_both": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_vp,
                                        c_sz, c_vp]),
        "nvfp4_kv_quantize_fp8": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_vp, c_int, c_vp, c_sz, c_vp]),
        "nvfp4_quantize_rht": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, ctypes.c_uint32, c_vp, c_vp, c_vp, c_int,
                                       c_vp, c_sz, c_vp]),
        "nvfp4_quantize_t_rht": (c_int, [c_vp, c_int, c_i64, c_i64, c_i64, ctypes.c_uint32, c_vp, c_vp, c_vp, c_int,
                                         c_vp, c_sz, c_vp]),
        "nvfp4_packed_weight_bytes": (c_sz, [c_int, ctypes.POINTER(c_i64), c_i64]),
        "nvfp4_pack_weights": (c_int, [c_int, ctypes.POINTER(c_i64), c_i64, ctypes.POINTER(c_vp),
                                       ctypes.POINTER(c_vp), ctypes.POINTER(c_vp), c_vp, c_sz,
                                       ctypes.POINTER(WeightDesc), c_vp]),
        "nvfp4_unpack_weights": (c_int, [ctypes.POINTER(WeightDesc), c_vp, c_vp, c_vp, c_vp]),
        "nvfp4_gemm_workspace_bytes": (c_sz, [c_i64, ctypes.POINTER(WeightDesc)]),
        "nvfp4_gemm": (c_int, [c_i64, c_vp, c_vp, c_vp, ctypes.POINTER(WeightDesc), c_vp, c_i64, c_vp, c_sz, c_vp]),
        "nvfp4_linear_workspace_bytes": (c_sz, [c_i64, c_int, ctypes.POINTER(WeightDesc)]),
        "nvfp4_linear_noalloc": (c_int, [c_vp, c_int, c_i64, c_i64, c_vp, c_vp, c_vp, c_int,
                                         ctypes.POINTER(WeightDesc), c_vp, c_i64, c_vp]),
        "nvfp4_linear": (c_int, [c_vp, c_int, c_i64, c_i64, c_vp, c_vp, c_vp, c_int, ctypes.POINTER(WeightDesc), c_vp,
                                 c_i64, c_vp, c_sz, c_vp]),
        "nvfp4_gemm_gated": (c_int, [c_i64, c_vp, c_vp, c_vp, ctypes.POINTER(WeightDesc),
                                     ctypes.POINTER(GdnGatesDesc), c_vp, c_i64, c_vp, c_sz, c_vp]),
        "nvfp4_gemm_ex": (c_int, [c_i64, c_vp, c_vp, c_vp, ctypes.POINTER(WeightDesc), ctypes.POINTER(EpilogueDesc),
                                  c_vp, c_i64, c_vp, c_sz, c_vp]),
        "nvfp4_linear_ex": (c_int, [c_vp, c_int, c_i64, c_i64, c_vp, c_vp, c_vp, c_int, ctypes.POINTER(WeightDesc),
                                    ctypes.POINTER(EpilogueDesc), c_vp, c_i64, c_vp, c_sz, c_vp]),
        "nvfp4_linear_gated": (c_int, [c_vp, c_int, c_i64, c_i64, c_vp, c_vp, c_vp, c_int, ctypes.POINTER(WeightDesc),
                                       ctypes.POINTER(GdnGatesDesc), c_vp, c_i64, c_vp, c_sz, c_vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if lib.nvfp4_abi_version() != 1:
        raise ImportError("libnvfp4 ABI version mismatch")
    return lib


_lib = _load()
lib = _lib


def _check(status: int):
    if status != NVFP4_OK:
        raise NVFP4Error(status, _lib.nvfp4_last_error().decode(errors="replace"))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _on_stream(stream):
    """Context for the conveniences below when the caller names a stream: the stream first waits for the
    current stream (whose work produced the inputs), and every allocation and fill inside runs on it, so
    temporaries (workspaces, g) are ordered with the launches that use them and are only reused by the
    caching allocator after that stream's work.  No stream: the current one, nothing to do."""
    import contextlib
    if stream is None:
        return contextlib.nullcontext()
    s = torch.cuda.ExternalStream(stream) if isinstance(stream, int) else stream
    s.wait_stream(torch.cuda.current_stream())
    return torch.cuda.stream(s)


def _stream_ordered(fn):
    """Runs a convenience under _on_stream of its ``stream`` argument."""
    import functools
    import inspect
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        with _on_stream(sig.bind(*args, **kwargs).arguments.get("stream")):
            return fn(*args, **kwargs)
    return wrapper


def last_error() -> str:
    return _lib.nvfp4_last_error().decode(errors="replace")


def device_check() -> int:
    return _lib.nvfp4_device_check()


# ---------------------------------------------------------------------------
# Direct entry points
# ---------------------------------------------------------------------------


def nvfp4_quantize_workspace_bytes(rows: int, K: int) -> int:
    return _lib.nvfp4_quantize_workspace_bytes(rows, K)


def nvfp4_quantize(x, codes, scales, g, g_mode=NVFP4_G_COMPUTE, workspace=None, stream=None, *,
                   rows=None, K=None, ld_x=None, in_dtype=None):
    """Quantize a 2-D device tensor x [rows, K] (float32 or bfloat16) into codes/scales/g."""
    if rows is None:
        rows, K = x.shape
        ld_x = x.stride(0) if rows > 1 else K   # a single row's stride is arbitrary
        if K > 1 and x.stride(-1) != 1:
            raise ValueError("x must have unit stride along K")
        in_dtype = NVFP4_IN_BF16 if x.dtype == torch.bfloat16 else NVFP4_IN_F32
        if x.dtype not in (torch.bfloat16, torch.float32):
            raise TypeError("x must be float32 or bfloat16")
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    _check(_lib.nvfp4_quantize(_ptr(x), in_dtype, rows, K, ld_x, _ptr(codes), _ptr(scales), _ptr(g), g_mode,
                               _ptr(workspace), ws_bytes, _stream(stream)))


def nvfp4_quantize_t(x, codes, scales, g, g_mode=NVFP4_G_COMPUTE, workspace=None, stream=None):
    """Encode x^T: x [rows, cols] (float32 or bfloat16, rows a multiple of 16) into codes [cols, rows/2],
    scales [cols, rows/16] and g."""
    rows, cols = x.shape
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("x must be float32 or bfloat16")
    if cols > 1 and x.stride(-1) != 1:
        raise ValueError("x must have unit stride along its columns")
    ld_x = x.stride(0) if rows > 1 else cols
    in_dtype = NVFP4_IN_BF16 if x.dtype == torch.bfloat16 else NVFP4_IN_F32
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    _check(_lib.nvfp4_quantize_t(_ptr(x), in_dtype, rows, cols, ld_x, _ptr(codes), _ptr(scales), _ptr(g), g_mode,
                                 _ptr(workspace), ws_bytes, _stream(stream)))


def _layout(x, unit_stride_msg):
    rows, cols = x.shape
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("x must be float32 or bfloat16")
    if cols > 1 and x.stride(-1) != 1:
        raise ValueError(unit_stride_msg)
    ld_x = x.stride(0) if rows > 1 else cols
    return rows, cols, ld_x, NVFP4_IN_BF16 if x.dtype == torch.bfloat16 else NVFP4_IN_F32


def nvfp4_quantize_rht(x, signs: int, codes, scales, g, g_mode=NVFP4_G_COMPUTE, workspace=None, stream=None):
    """nvfp4_quantize of the randomized Hadamard transform of x [rows, K] (16-bit sign mask)."""
    rows, K, ld_x, in_dtype = _layout(x, "x must have unit stride along K")
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    _check(_lib.nvfp4_quantize_rht(_ptr(x), in_dtype, rows, K, ld_x, int(signs), _ptr(codes), _ptr(scales), _ptr(g),
                                   g_mode, _ptr(workspace), ws_bytes, _stream(stream)))


def nvfp4_quantize_t_rht(x, signs: int, codes, scales, g, g_mode=NVFP4_G_COMPUTE, workspace=None, stream=None):
    """nvfp4_quantize_t of the randomized Hadamard transform of x^T (blocks of 16 rows of x)."""
    rows, cols, ld_x, in_dtype = _layout(x, "x must have unit stride along its columns")
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    _check(_lib.nvfp4_quantize_t_rht(_ptr(x), in_dtype, rows, cols, ld_x, int(signs), _ptr(codes), _ptr(scales),
                                     _ptr(g), g_mode, _ptr(workspace), ws_bytes, _stream(stream)))


def nvfp4_quantize_both(x, codes, scales, codes_t, scales_t, g, g_mode=NVFP4_G_COMPUTE, workspace=None,
                        stream=None):
    """Row and column encodings of x [rows, cols] (both multiples of 16) from one read, one g."""
    rows, cols, ld_x, in_dtype = _layout(x, "x must have unit stride along its columns")
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    _check(_lib.nvfp4_quantize_both(_ptr(x), in_dtype, rows, cols, ld_x, _ptr(codes), _ptr(scales), _ptr(codes_t),
                                    _ptr(scales_t), _ptr(g), g_mode, _ptr(workspace), ws_bytes, _stream(stream)))


def nvfp4_pack_weights_train(w, g, blob_fwd, blob_bwd, g_mode=NVFP4_G_COMPUTE, workspace=None, stream=None):
    """Both packed operands of a training weight w [n, k] from one read; returns (desc_fwd, desc_bwd)."""
    n, k, ld_w, in_dtype = _layout(w, "w must have unit stride along k")
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    df, db = WeightDesc(), WeightDesc()
    _check(_lib.nvfp4_pack_weights_train(_ptr(w), in_dtype, n, k, ld_w, _ptr(g), g_mode, _ptr(blob_fwd),
                                         blob_fwd.numel(), ctypes.byref(df), _ptr(blob_bwd), blob_bwd.numel(),
                                         ctypes.byref(db), _ptr(workspace), ws_bytes, _stream(stream)))
    return df, db


def nvfp4_kv_quantize_fp8(x, codes, scale, s_mode=NVFP4_G_COMPUTE, workspace=None, stream=None):
    """FP8 (E4M3) bytes of x [rows, cols] with one per-tensor scale (calibrated here, or given in scale)."""
    rows, cols, ld_x, in_dtype = _layout(x, "x must have unit stride along its columns")
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    _check(_lib.nvfp4_kv_quantize_fp8(_ptr(x), in_dtype, rows, cols, ld_x, _ptr(codes), _ptr(scale), s_mode,
                                      _ptr(workspace), ws_bytes, _stream(stream)))


def nvfp4_packed_weight_bytes(module_rows: Sequence[int], K: int) -> int:
    arr = (ctypes.c_int64 * len(module_rows))(*module_rows)
    return _lib.nvfp4_packed_weight_bytes(len(module_rows), arr, K)


def nvfp4_pack_weights(modules, K: int, blob, stream=None) -> WeightDesc:
    """modules: sequence of (codes [rows, K/2] uint8, scales [rows, K/16] uint8, g [1] float32) device tensors."""
    n = len(modules)
    rows = (ctypes.c_int64 * n)(*[int(m[0].shape[0]) for m in modules])
    cp = (ctypes.c_void_p * n)(*[_ptr(m[0]) for m in modules])
    sp = (ctypes.c_void_p * n)(*[_ptr(m[1]) for m in modules])
    gp = (ctypes.c_void_p * n)(*[_ptr(m[2]) for m in modules])
    desc = WeightDesc()
    nbytes = blob.numel() * blob.element_size()
    _check(_lib.nvfp4_pack_weights(n, rows, K, cp, sp, gp, _ptr(blob), nbytes, ctypes.byref(desc),
                                   _stream(stream)))
    return desc


def nvfp4_unpack_weights(desc: WeightDesc, codes, scales, colscale, stream=None):
    _check(_lib.nvfp4_unpack_weights(ctypes.byref(desc), _ptr(codes), _ptr(scales), _ptr(colscale),
                                     _stream(stream)))


def nvfp4_gemm_workspace_bytes(M: int, desc: WeightDesc) -> int:
    return _lib.nvfp4_gemm_workspace_bytes(M, ctypes.byref(desc))


def nvfp4_gemm(M: int, a_codes, a_scales, g_x, desc: WeightDesc, y, ld_y=None, workspace=None, stream=None,
               gates: "GdnGates | None" = None):
    """nvfp4_gemm; nvfp4_gemm_gated when gates are given; nvfp4_gemm_ex when y is bfloat16."""
    if ld_y is None:
        ld_y = y.stride(0) if y.dim() == 2 and y.shape[0] > 1 else desc.n
    ws_bytes = workspace.numel() * workspace.element_size() if isinstance(workspace, torch.Tensor) else 0
    if y.dtype == torch.bfloat16:   # output epilogue entry point (bf16 Y, with or without gates)
        ep = _epilogue(y, gates)
        _check(_lib.nvfp4_gemm_ex(M, _ptr(a_codes), _ptr(a_scales), _ptr(g_x), ctypes.byref(desc), ctypes.byref(ep),
                                  _ptr(y), ld_y, _ptr(workspace), ws_bytes, _stream(stream)))
    elif gates is None:
        _check(_lib.nvfp4_gemm(M, _ptr(a_codes), _ptr(a_scales), _ptr(g_x), ctypes.byref(desc), _ptr(y), ld_y,
                               _ptr(workspace), ws_bytes, _stream(stream)))
    else:
        _check(_lib.nvfp4_gemm_gated(M, _ptr(a_codes), _ptr(a_scales), _ptr(g_x), ctypes.byref(desc),
                                     ctypes.byref(gates.desc), _ptr(y), ld_y, _ptr(workspace), ws_bytes,
                                     _stream(stream)))


def nvfp4_linear_workspace_bytes(M: int, in_dtype: int, desc: WeightDesc) -> int:
    return _lib.nvfp4_linear_workspace_bytes(M, in_dtype, ctypes.byref(desc))


def nvfp4_linear(x, x_codes, x_scales, g_x, desc: WeightDesc, y, workspace, g_mode=NVFP4_G_COMPUTE, stream=None, *,
                 M=None, ld_x=None, in_dtype=None, ld_y=None, gates: "GdnGates | None" = None):
    """Quantize x [M, K] and multiply by a packed weight in one call (workspace zero-filled before first use);
    nvfp4_linear_gated when gates are given; nvfp4_linear_ex when y is bfloat16."""
    if M is None:
        M = x.shape[0]
        ld_x = x.stride(0) if M > 1 else x.shape[1]
        in_dtype = NVFP4_IN_BF16 if x.dtype == torch.bfloat16 else NVFP4_IN_F32
    if ld_y is None:
        ld_y = y.stride(0) if y.dim() == 2 and y.shape[0] > 1 else desc.n
    ws_bytes = workspace.numel() * workspace.element_size()
    if y.dtype == torch.bfloat16:   # output epilogue entry point (bf16 Y, with or without gates)
        ep = _epilogue(y, gates)
        _check(_lib.nvfp4_linear_ex(_ptr(x), in_dtype, M, ld_x, _ptr(x_codes), _ptr(x_scales), _ptr(g_x), g_mode,
                                    ctypes.byref(desc), ctypes.byref(ep), _ptr(y), ld_y, _ptr(workspace), ws_bytes,
                                    _stream(stream)))
    elif gates is None:
        _check(_lib.nvfp4_linear(_ptr(x), in_dtype, M, ld_x, _ptr(x_codes), _ptr(x_scales), _ptr(g_x), g_mode,
                                 ctypes.byref(desc), _ptr(y), ld_y, _ptr(workspace), ws_bytes, _stream(stream)))
    else:
        _check(_lib.nvfp4_linear_gated(_ptr(x), in_dtype, M, ld_x, _ptr(x_codes), _ptr(x_scales), _ptr(g_x), g_mode,
                                       ctypes.byref(desc), ctypes.byref(gates.desc), _ptr(y), ld_y, _ptr(workspace),
                                       ws_bytes, _stream(stream)))


def nvfp4_linear_noalloc(x, x_codes, x_scales, g_x, desc: WeightDesc, y, g_mode=NVFP4_G_COMPUTE, stream=None, *,
                         M=None, ld_x=None, in_dtype=None, ld_y=None):
    """nvfp4_linear with the library's static scratch instead of a workspace (FP32 y, no gates)."""
    if M is None:
        M = x.shape[0]
        ld_x = x.stride(0) if M > 1 else x.shape[1]
        in_dtype = NVFP4_IN_BF16 if x.dtype == torch.bfloat16 else NVFP4_IN_F32
    if ld_y is None:
        ld_y = y.stride(0) if y.dim() == 2 and y.shape[0] > 1 else desc.n
    _check(_lib.nvfp4_linear_noalloc(_ptr(x), in_dtype, M, ld_x, _ptr(x_codes), _ptr(x_scales), _ptr(g_x), g_mode,
                                     ctypes.byref(desc), _ptr(y), ld_y, _stream(stream)))


# ---------------------------------------------------------------------------
# Conveniences (outputs allocated with torch, then the entry points above)
# ---------------------------------------------------------------------------


def empty_quantized(rows: int, K: int, device="cuda"):
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=device)
    scales = torch.empty((rows, K // 16), dtype=torch.uint8, device=device)
    g = torch.empty((1,), dtype=torch.float32, device=device)
    return codes, scales, g


@_stream_ordered
def quantize(x: torch.Tensor, g=None, stream=None):
    """NVFP4-quantize x [rows, K]; g=None computes the global scale, otherwise uses the given value."""
    rows, K = x.shape
    codes, scales, gt = empty_quantized(rows, K, x.device)
    if g is None:
        ws = torch.empty((max(nvfp4_quantize_workspace_bytes(rows, K), 1),), dtype=torch.uint8, device=x.device)
        nvfp4_quantize(x, codes, scales, gt, NVFP4_G_COMPUTE, ws, stream)
    else:
        if isinstance(g, torch.Tensor):
            gt.copy_(g.reshape(1))
        else:
            gt.fill_(float(g))
        nvfp4_quantize(x, codes, scales, gt, NVFP4_G_GIVEN, None, stream)
    return codes, scales, gt


@_stream_ordered
def quantize_t(x: torch.Tensor, g=None, stream=None):
    """NVFP4 encoding of x^T for x [rows, cols]: codes [cols, rows/2], scales [cols, rows/16] and g
    (computed from x's amax when g is None, otherwise the given value)."""
    rows, cols = x.shape
    codes, scales, gt = empty_quantized(cols, rows, x.device)
    if g is None:
        ws = torch.empty((max(nvfp4_quantize_workspace_bytes(rows, cols), 1),), dtype=torch.uint8, device=x.device)
        nvfp4_quantize_t(x, codes, scales, gt, NVFP4_G_COMPUTE, ws, stream)
    else:
        if isinstance(g, torch.Tensor):
            gt.copy_(g.reshape(1))
        else:
            gt.fill_(float(g))
        nvfp4_quantize_t(x, codes, scales, gt, NVFP4_G_GIVEN, None, stream)
    return codes, scales, gt


def _quantize_with(fn, x, signs, out_rows, out_k, g, stream):
    codes, scales, gt = empty_quantized(out_rows, out_k, x.device)
    if g is None:
        ws = torch.empty((max(nvfp4_quantize_workspace_bytes(*x.shape), 1),), dtype=torch.uint8, device=x.device)
        fn(x, signs, codes, scales, gt, NVFP4_G_COMPUTE, ws, stream)
    else:
        if isinstance(g, torch.Tensor):
            gt.copy_(g.reshape(1))
        else:
            gt.fill_(float(g))
        fn(x, signs, codes, scales, gt, NVFP4_G_GIVEN, None, stream)
    return codes, scales, gt


@_stream_ordered
def quantize_rht(x: torch.Tensor, signs: int, g=None, stream=None):
    """NVFP4 codes, scales and g of the randomized Hadamard transform of x [rows, K]."""
    return _quantize_with(nvfp4_quantize_rht, x, signs, x.shape[0], x.shape[1], g, stream)


@_stream_ordered
def quantize_t_rht(x: torch.Tensor, signs: int, g=None, stream=None):
    """The same for x^T: codes [cols, rows/2], scales [cols, rows/16]."""
    return _quantize_with(nvfp4_quantize_t_rht, x, signs, x.shape[1], x.shape[0], g, stream)


@_stream_ordered
def quantize_both(x: torch.Tensor, g=None, stream=None):
    """((codes, scales, g), (codes_t, scales_t, g)) of x [rows, cols]: the encodings of x and of x^T, sharing
    one g tensor."""
    rows, cols = x.shape
    codes, scales, gt = empty_quantized(rows, cols, x.device)
    codes_t, scales_t, _ = empty_quantized(cols, rows, x.device)
    if g is None:
        ws = torch.empty((max(nvfp4_quantize_workspace_bytes(rows, cols), 1),), dtype=torch.uint8, device=x.device)
        nvfp4_quantize_both(x, codes, scales, codes_t, scales_t, gt, NVFP4_G_COMPUTE, ws, stream)
    else:
        if isinstance(g, torch.Tensor):
            gt.copy_(g.reshape(1))
        else:
            gt.fill_(float(g))
        nvfp4_quantize_both(x, codes, scales, codes_t, scales_t, gt, NVFP4_G_GIVEN, None, stream)
    return (codes, scales, gt), (codes_t, scales_t, gt)


@_stream_ordered
def kv_quantize_fp8(x: torch.Tensor, scale=None, stream=None):
    """(codes uint8 [rows, cols], scale [1]) of x in FP8 E4M3; scale=None calibrates on x."""
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    st = torch.empty((1,), dtype=torch.float32, device=x.device)
    if scale is None:
        ws = torch.empty((max(nvfp4_quantize_workspace_bytes(rows, cols), 1),), dtype=torch.uint8, device=x.device)
        nvfp4_kv_quantize_fp8(x, codes, st, NVFP4_G_COMPUTE, ws, stream)
    else:
        if isinstance(scale, torch.Tensor):
            st.copy_(scale.reshape(1))
        else:
            st.fill_(float(scale))
        nvfp4_kv_quantize_fp8(x, codes, st, NVFP4_G_GIVEN, None, stream)
    return codes, st


class PackedWeight:
    """A packed (possibly fused multi-module) weight: the device blob plus its descriptor."""

    @_stream_ordered
    def __init__(self, modules, K: int, stream=None):
        rows = [int(m[0].shape[0]) for m in modules]
        nbytes = nvfp4_packed_weight_bytes(rows, K)
        if nbytes == 0:
            raise NVFP4Error(NVFP4_ERR_SHAPE, f"invalid packed weight shape rows={rows} K={K}")
        dev = modules[0][0].device
        self.blob = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
        self.desc = nvfp4_pack_weights(modules, K, self.blob, stream)
        self.module_rows = rows
        self.K = K

    @property
    def n(self) -> int:
        return int(self.desc.n)

    def clone(self) -> "PackedWeight":
        """A copy of the blob at another device address (the descriptor points at the copy)."""
        other = PackedWeight.__new__(PackedWeight)
        other.blob = self.blob.clone()
        other.desc = WeightDesc.from_buffer_copy(self.desc)
        other.desc.blob = other.blob.data_ptr()
        other.module_rows, other.K = self.module_rows, self.K
        return other

    @_stream_ordered
    def unpack(self, stream=None):
        n, K = self.n, self.K
        codes = torch.empty((n, K // 2), dtype=torch.uint8, device=self.blob.device)
        scales = torch.empty((n, K // 16), dtype=torch.uint8, device=self.blob.device)
        colscale = torch.empty((n,), dtype=torch.float32, device=self.blob.device)
        nvfp4_unpack_weights(self.desc, codes, scales, colscale, stream)
        return codes, scales, colscale


@_stream_ordered
def pack_weights_train(w: torch.Tensor, g=None, stream=None):
    """(forward PackedWeight of w along k, backward PackedWeight of w^T along n, g) for a training weight
    w [n, k], from one read of w (g computed when None)."""
    n, k = w.shape
    fwd, bwd = PackedWeight.__new__(PackedWeight), PackedWeight.__new__(PackedWeight)
    fwd.blob = torch.empty((nvfp4_packed_weight_bytes([n], k),), dtype=torch.uint8, device=w.device)
    bwd.blob = torch.empty((nvfp4_packed_weight_bytes([k], n),), dtype=torch.uint8, device=w.device)
    gt = torch.empty((1,), dtype=torch.float32, device=w.device)
    if g is None:
        ws = torch.empty((max(nvfp4_quantize_workspace_bytes(n, k), 1),), dtype=torch.uint8, device=w.device)
        fwd.desc, bwd.desc = nvfp4_pack_weights_train(w, gt, fwd.blob, bwd.blob, NVFP4_G_COMPUTE, ws, stream)
    else:
        gt.fill_(float(g)) if not isinstance(g, torch.Tensor) else gt.copy_(g.reshape(1))
        fwd.desc, bwd.desc = nvfp4_pack_weights_train(w, gt, fwd.blob, bwd.blob, NVFP4_G_GIVEN, None, stream)
    fwd.module_rows, fwd.K = [n], k
    bwd.module_rows, bwd.K = [k], n
    return fwd, bwd, gt


def linear_workspace(M: int, x_dtype, w: "PackedWeight", device="cuda") -> torch.Tensor:
    """A zero-filled workspace for nvfp4_linear (reusable by later calls on the same stream)."""
    in_dtype = NVFP4_IN_BF16 if x_dtype == torch.bfloat16 else NVFP4_IN_F32
    return torch.zeros((nvfp4_linear_workspace_bytes(M, in_dtype, w.desc),), dtype=torch.uint8, device=device)


@_stream_ordered
def linear(x: torch.Tensor, w: "PackedWeight", workspace=None, g=None, stream=None, gates=None,
           out_dtype=torch.float32):
    """Y = NVFP4(x) . W^T in one call (through the GDN gate epilogue when gates are given; Y in float32 or
    bfloat16); returns (y, codes, scales, g)."""
    M, K = x.shape
    codes, scales, gt = empty_quantized(M, K, x.device)
    if g is not None:
        gt.fill_(float(g))
    if workspace is None:
        workspace = linear_workspace(M, x.dtype, w, x.device)
    y = torch.empty((M, w.n), dtype=out_dtype, device=x.device)
    nvfp4_linear(x, codes, scales, gt, w.desc, y, workspace, NVFP4_G_GIVEN if g is not None else NVFP4_G_COMPUTE,
                 stream, gates=gates)
    return y, codes, scales, gt


@_stream_ordered
def gemm(a_codes, a_scales, g_x, w: PackedWeight, y=None, stream=None, gates=None, out_dtype=torch.float32):
    M = a_codes.shape[0]
    if y is None:
        y = torch.empty((M, w.n), dtype=out_dtype, device=a_codes.device)
    ws_bytes = nvfp4_gemm_workspace_bytes(M, w.desc)
    ws = torch.zeros((ws_bytes,), dtype=torch.uint8, device=a_codes.device) if ws_bytes else None
    nvfp4_gemm(M, a_codes, a_scales, g_x, w.desc, y, None, ws, stream, gates=gates)
    return y
