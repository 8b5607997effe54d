"""Parity metrics between the HIP path and the fp64 oracle.

Bars (written here, used by every GPU parity test):
  fp32 inputs: max |gpu - oracle| <= 1e-4 over outputs and final states;
  bf16 inputs: rms(gpu - oracle) / rms(oracle) <= 2e-2, for outputs and final states
  separately, over the whole tensor and over every (sequence, head) unit.
"""

import numpy as np

FP32_MAX_ABS = 1e-4
BF16_RMS_REL = 2e-2


def rms(x):
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def rms_rel(a, ref):
    r = rms(ref)
    d = rms(np.asarray(a, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    return d / r if r > 0 else d


def check(dtype, got, ref, what, units=None):
    """Assert the bar for ``dtype`` ("fp32" | "bf16").  ``units`` optionally lists
    (label, got_slice, ref_slice) triples checked one by one (bf16 only)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values from the GPU"
    if dtype == "fp32":
        err = max_abs(got, ref)
        assert err <= FP32_MAX_ABS, f"{what}: max-abs {err:.3e} > {FP32_MAX_ABS}"
        return err
    err = rms_rel(got, ref)
    assert err <= BF16_RMS_REL, f"{what}: rms-rel {err:.3e} > {BF16_RMS_REL}"
    for label, gs, rs in units or []:
        e = rms_rel(gs, rs)
        assert e <= BF16_RMS_REL, f"{what} {label}: rms-rel {e:.3e} > {BF16_RMS_REL}"
    return err
