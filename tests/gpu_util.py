"""Shared helpers of the GPU parity tests (comparison against the oracle)."""
import numpy as np
import pytest

# Parity bars: max |gpu - ref| <= TOL * max |ref| per tensor.
TOL_F32_STATE = 2e-5   # FP32 state storage: outputs and states
TOL_BF16_STATE = 1e-2  # BF16 state storage, against the oracle in BF16 mode


def tol_for(state: str) -> float:
    return TOL_F32_STATE if state == "f32" else TOL_BF16_STATE


def rel_linf(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    scale = np.abs(ref).max()
    assert np.isfinite(scale) and scale > 0
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU result"
    return float(err.max() / scale)


def assert_parity(got, ref, tol, what=""):
    e = rel_linf(got, ref)
    print(f"  parity {what}: max|d|/max|ref| = {e:.3e} (bar {tol:.0e})", flush=True)
    assert e <= tol, f"{what}: relative L-inf error {e:.3e} exceeds {tol:.0e}"


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from hybrid_linear_attention_rule_amd import kda
    kda.load()   # raises if the HIP library is missing: no fallback
    return torch
