"""The seeded input generators produce the stated shapes, dtypes and distributions."""
import numpy as np

import workloads


def _is_bf16(a):
    return np.array_equal(workloads.to_bf16_values(a), a)


def test_tiny():
    wl = workloads.make_tiny()
    assert wl.x.shape == (64, 512) and wl.w[0].shape == (256, 512)
    for a in (wl.x, wl.w[0]):
        assert np.abs(a).max() == 40.0
        assert np.sum(np.abs(a) == 40.0) == 4 and np.sum(a == 40.0) == 2
    assert np.array_equal(workloads.make_tiny().x, wl.x)          # deterministic


def test_decode():
    wl = workloads.make_decode()
    assert wl.x.shape == (16, 5120) and wl.w[0].shape == (5120, 5120)
    assert _is_bf16(wl.x) and _is_bf16(wl.w[0][:64])
    assert abs(float(wl.w[0].std()) - 0.02) < 1e-3


def test_gdn_small():
    wl = workloads.make_gdn(M=64)
    assert [w.shape[0] for w in wl.w] == [4096, 4096, 4096, 4096, 48, 48]
    assert wl.N == 16480 and wl.K == 5120
    col_max = np.abs(wl.x).max(axis=0)
    assert np.sum(col_max > 200) >= 4                               # the x50 outlier channels
    sig = [float(w.std()) for w in wl.w]
    assert abs(sig[4] / sig[0] - 10) < 1 and abs(sig[0] / sig[5] - 10) < 1


def test_ngpt_small():
    wl = workloads.make_ngpt(M=64)
    n = np.linalg.norm(wl.x.astype(np.float64), axis=1)
    assert np.all(np.abs(n - 1) < 1e-2)
    assert float(wl.x.mean()) > 0


def test_large_small_m():
    wl = workloads.make_large(M=64)
    assert wl.x.shape == (64, 16384) and _is_bf16(wl.x)
    assert np.abs(wl.x).max() > 30
