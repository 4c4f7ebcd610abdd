"""Shared helpers of the GPU parity tests: tolerance checks and oracle calls on the exact
(bf16- or fp32-rounded) values the device received."""
import numpy as np
import pytest

import mla_synth as S

torch = pytest.importorskip("torch")


def have_gpu() -> bool:
    return torch.cuda.is_available()


def check(got, ref, dtype: str, what: str):
    """bf16: max|d| <= 1e-2 max|ref| and cosine >= 0.9999; fp32: max|d| <= 1e-5 max|ref|."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.abs(got - ref)))
    if dtype == S.BF16:
        cos = float(np.sum(got * ref) / (np.linalg.norm(got) * np.linalg.norm(ref) + 1e-300))
        assert err <= 1e-2 * scale and cos >= 0.9999, f"{what}: max|d|={err:.3e} max|ref|={scale:.3e} cos={cos:.6f}"
        return err / scale, cos
    assert err <= 1e-5 * scale, f"{what}: max|d|={err:.3e} max|ref|={scale:.3e} rel={err / scale:.3e}"
    return err / scale, 1.0
