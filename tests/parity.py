"""Comparison helpers for the GPU parity tests (tolerances of the parity bar)."""
import numpy as np
import torch

OUT_ATOL = 1e-2      # bf16 outputs: |gpu - ref| <= 1e-2 + 1e-2 |ref|
OUT_RTOL = 1e-2
LSE_ATOL = 1e-3      # LSE: 1e-3 absolute; +inf must match exactly


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def check_out(gpu: np.ndarray, ref: np.ndarray, where=None, atol=OUT_ATOL, rtol=OUT_RTOL, what="out"):
    if where is not None:
        gpu, ref = gpu[where], ref[where]
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert not np.isnan(ref).any(), "oracle produced NaN"
    bad = ~(np.abs(gpu - ref) <= atol + rtol * np.abs(ref))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; "
                             f"first {idx.tolist()} gpu={gpu[tuple(idx.T)]} ref={ref[tuple(idx.T)]}; "
                             f"max err {np.nanmax(np.abs(gpu - ref))}")
    return float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0


def check_lse(gpu: np.ndarray, ref: np.ndarray, where=None, atol=LSE_ATOL):
    if where is not None:
        gpu, ref = gpu[where], ref[where]
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    inf = np.isposinf(ref)
    assert np.array_equal(np.isposinf(gpu), inf), "+inf pattern of the LSE differs"
    fin = ~inf
    err = np.abs(gpu[fin] - ref[fin])
    assert np.all(err <= atol), f"lse max err {err.max()}"
    return float(err.max()) if err.size else 0.0
