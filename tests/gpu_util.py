"""Helpers for the GPU parity tests: moving seeded inputs to the device and
comparing the HIP results with the oracle at the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np

# Tolerances of the parity bar.
FP32_MAX_ABS = 2e-6      # fp32 outputs: max |y_gpu - y_oracle|
FP32_ROW_SUM = 1e-5      # fp32 outputs: per-row |sum(y_gpu) - 1|
BF16_MAX_REL = 8e-3      # bf16 outputs: max |y_gpu - y_oracle| / y_oracle over y_oracle >= 2^-126
TOPK_PROB_ABS = 2e-6     # top-K probabilities; indices must match exactly
BF16_MIN_NORMAL = 2.0 ** -126


def say(msg: str):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_device(x: np.ndarray):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def to_host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def assert_fp32_parity(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = ""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    nan_ref = np.isnan(y_ref)
    assert np.array_equal(np.isnan(y_gpu), nan_ref), f"{what}: NaN pattern differs"
    ok = ~nan_ref
    err = np.abs(y_gpu[ok] - y_ref[ok])
    worst = float(err.max()) if err.size else 0.0
    assert worst <= FP32_MAX_ABS, f"{what}: max abs error {worst:.3e} > {FP32_MAX_ABS}"
    rows_ok = ~nan_ref.any(axis=1)
    if rows_ok.any():
        s = np.abs(y_gpu[rows_ok].sum(axis=1) - 1.0)
        assert float(s.max()) <= FP32_ROW_SUM, f"{what}: row sum off by {float(s.max()):.3e}"
    return worst


def assert_bf16_parity(y_gpu: np.ndarray, y_ref: np.ndarray, what: str = ""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    nan_ref = np.isnan(y_ref)
    assert np.array_equal(np.isnan(y_gpu), nan_ref), f"{what}: NaN pattern differs"
    sel = (~nan_ref) & (y_ref >= BF16_MIN_NORMAL)
    rel = np.abs(y_gpu[sel] - y_ref[sel]) / y_ref[sel]
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= BF16_MAX_REL, f"{what}: max rel error {worst:.3e} > {BF16_MAX_REL}"
    tiny = (~nan_ref) & (y_ref < BF16_MIN_NORMAL)
    if tiny.any():  # below the smallest normal the output may be 0 or a tiny value
        assert float(np.abs(y_gpu[tiny]).max()) <= 2.0 * BF16_MIN_NORMAL
    return worst


def assert_parity(y_gpu, y_ref, bf16: bool, what: str = ""):
    return assert_bf16_parity(y_gpu, y_ref, what) if bf16 else assert_fp32_parity(y_gpu, y_ref, what)
