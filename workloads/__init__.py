"""Seeded synthetic inputs for the NVFP4 W4A4 linear layer.

This module only draws random numbers and casts them to the input dtype; it holds
none of the quantization or GEMM arithmetic.  Both the CPU oracle and the HIP path
consume exactly the arrays it returns.

Generation is host-side and deterministic: ``numpy.random.Generator(PCG64(...))``
with child streams spawned from ``SeedSequence(seed)`` in a fixed order (the order
of the ``spawn`` indices below).  Draws are FP32 unless noted and are rounded to
bf16 with torch's CPU cast (round to nearest even).  bf16 inputs are returned as
FP32 numpy arrays whose values are exactly bf16-representable, plus a dtype tag.

The shapes and value distributions stand in for the statistics of the pages'
workloads: heavy-tailed activations with outlier channels for the hybrid Gated
DeltaNet projections ("Why Gated DeltaNet Survives 4-Bit Quantization", section
"Why the 'Fragile' Recurrence is Actually Robust": inputs with extreme outliers),
and rows on the unit hypersphere for nGPT ("Normalized Architectures are Natively
4-Bit", section "Approach").
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def _rng(seed_seq: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_seq))


def to_bf16_values(a: np.ndarray, chunk_rows: int = 4096) -> np.ndarray:
    """Round an FP32/FP64 array to bf16 (RNE, via torch's CPU cast) and return FP32 values."""
    import torch

    a = np.asarray(a)
    out = np.empty(a.shape, dtype=np.float32)
    flat_in = a.reshape(-1, a.shape[-1]) if a.ndim > 1 else a.reshape(1, -1)
    flat_out = out.reshape(flat_in.shape)
    for r0 in range(0, flat_in.shape[0], chunk_rows):
        t = torch.from_numpy(np.ascontiguousarray(flat_in[r0:r0 + chunk_rows], dtype=np.float32))
        flat_out[r0:r0 + chunk_rows] = t.to(torch.bfloat16).to(torch.float32).numpy()
    return out


@dataclass
class Workload:
    name: str
    x: np.ndarray                   # [M, K] FP32 values (bf16-exact when x_dtype == 'bf16')
    x_dtype: str                    # 'f32' or 'bf16'
    w: list                         # list of [N_s, K] FP32 arrays, one per sub-module
    w_dtype: str
    module_names: list = field(default_factory=list)
    quantize_w_in_step: bool = False  # weights quantized inside the timed step (tiny case)

    @property
    def M(self):
        return self.x.shape[0]

    @property
    def K(self):
        return self.x.shape[1]

    @property
    def N(self):
        return sum(w.shape[0] for w in self.w)


# name -> (M, K, [(module, rows)]) for the five workloads
SHAPES = {
    "tiny": (64, 512, [("w", 256)]),
    "decode": (16, 5120, [("w", 5120)]),
    "gdn": (4096, 5120, [("q", 4096), ("k", 4096), ("v", 4096), ("z", 4096), ("a", 48), ("b", 48)]),
    "ngpt": (8192, 4096, [("w", 4096)]),
    "large": (32768, 16384, [("w", 16384)]),
}

SEEDS = {"tiny": 101, "decode": 202, "gdn": 303, "ngpt": 404, "large": 505}


def _outliers(rng, a, count, values):
    """Set ``count`` distinct positions (drawn without replacement) to the cycled ``values``."""
    flat = a.reshape(-1)
    pos = rng.choice(flat.size, size=count, replace=False)
    flat[pos] = np.resize(np.asarray(values, dtype=a.dtype), count)
    return a


def make_tiny(seed: int = SEEDS["tiny"]) -> Workload:
    """FP32 X[64x512], W[256x512] ~ N(0,1), each with 4 outliers +40,-40,+40,-40 (amax exactly 40)."""
    c = np.random.SeedSequence(seed).spawn(4)
    M, K, mods = SHAPES["tiny"]
    x = _rng(c[0]).standard_normal((M, K), dtype=np.float32)
    _outliers(_rng(c[1]), x, 4, [40.0, -40.0])
    w = _rng(c[2]).standard_normal((mods[0][1], K), dtype=np.float32)
    _outliers(_rng(c[3]), w, 4, [40.0, -40.0])
    return Workload("tiny", x, "f32", [w], "f32", ["w"], quantize_w_in_step=True)


def make_decode(seed: int = SEEDS["decode"]) -> Workload:
    """bf16 X[16x5120] ~ N(0,1); bf16 W[5120x5120] = 0.02 N(0,1)."""
    c = np.random.SeedSequence(seed).spawn(2)
    M, K, mods = SHAPES["decode"]
    x = to_bf16_values(_rng(c[0]).standard_normal((M, K), dtype=np.float32))
    w = to_bf16_values(np.float32(0.02) * _rng(c[1]).standard_normal((mods[0][1], K), dtype=np.float32))
    return Workload("decode", x, "bf16", [w], "bf16", ["w"])


GDN_SIGMA = {"q": 0.02, "k": 0.02, "v": 0.02, "z": 0.02, "a": 0.2, "b": 0.002}


def make_gdn(seed: int = SEEDS["gdn"], M: int | None = None) -> Workload:
    """bf16 X[4096x5120] ~ Student-t(3) with 5 channels (0.1% of 5120) scaled x50;
    six weight sub-modules q,k,v,z [4096x5120] (sigma 0.02), a [48x5120] (0.2), b [48x5120] (0.002)."""
    c = np.random.SeedSequence(seed).spawn(3 + 6)
    M0, K, mods = SHAPES["gdn"]
    M = M0 if M is None else M
    x = _rng(c[0]).standard_t(3, size=(M, K)).astype(np.float32)
    ch = _rng(c[1]).choice(K, size=int(round(0.001 * K)), replace=False)
    x[:, ch] *= np.float32(50.0)
    x = to_bf16_values(x)
    ws = []
    for i, (name, rows) in enumerate(mods):
        ws.append(to_bf16_values(np.float32(GDN_SIGMA[name]) *
                                 _rng(c[3 + i]).standard_normal((rows, K), dtype=np.float32)))
    return Workload("gdn", x, "bf16", ws, "bf16", [m for m, _ in mods])


@dataclass
class GdnGates:
    """Parameters of the gate epilogue of the fused GDN projection: its decay columns
    [a_col, a_col + n_a) and write-strength columns [b_col, b_col + n_b), and per decay
    head the A parameter (entering as exp(A)) and the bias added inside the softplus."""
    a_col: int
    n_a: int
    b_col: int
    n_b: int
    a_log: np.ndarray     # FP32 [n_a]
    dt_bias: np.ndarray   # FP32 [n_a]


def gdn_gate_params(seed: int = SEEDS["gdn"] + 1000, modules=None) -> GdnGates:
    """A ~ log U(1, 16) per head (the usual initialisation of exp(A) in 1..16), bias ~ U(-6.9, -2.3)
    (softplus of it spans the usual 1e-3..0.1 step sizes).  Columns: the a and b modules of
    the fused projection (the 5th and 6th, after q, k, v, z)."""
    mods = SHAPES["gdn"][2] if modules is None else modules
    offs = np.cumsum([0] + [r for _, r in mods])
    names = [m for m, _ in mods]
    ia, ib = names.index("a"), names.index("b")
    n_a = mods[ia][1]
    c = np.random.SeedSequence(seed).spawn(2)
    a_log = np.log(_rng(c[0]).uniform(1.0, 16.0, n_a)).astype(np.float32)
    dt_bias = _rng(c[1]).uniform(-6.9, -2.3, n_a).astype(np.float32)
    return GdnGates(int(offs[ia]), n_a, int(offs[ib]), mods[ib][1], a_log, dt_bias)


def _hypersphere_rows(rng, rows, cols):
    z = rng.standard_normal((rows, cols))             # FP64
    z += 1e-3                                         # shared positive mean component
    z /= np.linalg.norm(z, axis=1, keepdims=True)     # each row onto the unit sphere (FP64)
    return to_bf16_values(z.astype(np.float32))


def make_ngpt(seed: int = SEEDS["ngpt"], M: int | None = None) -> Workload:
    """X[8192x4096], W[4096x4096]: rows of N(0,1)+1e-3 draws, L2-normalised in FP64, cast to bf16."""
    c = np.random.SeedSequence(seed).spawn(2)
    M0, K, mods = SHAPES["ngpt"]
    M = M0 if M is None else M
    x = _hypersphere_rows(_rng(c[0]), M, K)
    w = _hypersphere_rows(_rng(c[1]), mods[0][1], K)
    return Workload("ngpt", x, "bf16", [w], "bf16", ["w"])


def make_large(seed: int = SEEDS["large"], M: int | None = None) -> Workload:
    """bf16 X[32768x16384] ~ N(0,1) with 0.05% of elements x30; bf16 W[16384x16384] = 0.01 N(0,1)."""
    c = np.random.SeedSequence(seed).spawn(3)
    M0, K, mods = SHAPES["large"]
    M = M0 if M is None else M
    x = _rng(c[0]).standard_normal((M, K), dtype=np.float32)
    flat = x.reshape(-1)
    n_out = int(round(0.0005 * flat.size))
    pos = _rng(c[1]).choice(flat.size, size=n_out, replace=False)
    flat[pos] *= np.float32(30.0)
    x = to_bf16_values(x)
    w = to_bf16_values(np.float32(0.01) * _rng(c[2]).standard_normal((mods[0][1], K), dtype=np.float32))
    return Workload("large", x, "bf16", [w], "bf16", ["w"])


MAKERS = {"tiny": make_tiny, "decode": make_decode, "gdn": make_gdn, "ngpt": make_ngpt, "large": make_large}


def make(name: str, **kw) -> Workload:
    return MAKERS[name](**kw)


def kv_cache(seed: int = 707, tokens: int = 4096, width: int = 1024) -> np.ndarray:
    """A K-cache-shaped bf16 tensor [tokens x heads*head_dim]: N(0,1) per channel times a per-channel
    scale exp(U(-1, 1)), with 1% of the channels x20 (the outlier channels of keys)."""
    c = np.random.SeedSequence(seed).spawn(3)
    x = _rng(c[0]).standard_normal((tokens, width), dtype=np.float32)
    scale = np.exp(_rng(c[1]).uniform(-1.0, 1.0, width)).astype(np.float32)
    out = _rng(c[2]).choice(width, size=max(1, width // 100), replace=False)
    scale[out] *= np.float32(20.0)
    return to_bf16_values(x * scale)


def rht_signs(seed: int = 606) -> int:
    """A seeded random 16-bit sign mask for the randomized Hadamard transform (the method's random draw,
    passed to both sides as an input)."""
    return int(_rng(np.random.SeedSequence(seed)).integers(0, 1 << 16))


def random_matrix(seed: int, rows: int, cols: int, scale: float = 1.0, dtype: str = "f32") -> np.ndarray:
    """A plain seeded N(0, scale^2) matrix for edge-case tests (FP32, or bf16-exact FP32 values)."""
    a = np.float32(scale) * _rng(np.random.SeedSequence(seed)).standard_normal((rows, cols), dtype=np.float32)
    return to_bf16_values(a) if dtype == "bf16" else a
