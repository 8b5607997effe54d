"""Parity metrics between the HIP path and the fp64 oracle.

Bars (written here, used by every GPU parity test):
  fp32 inputs: max |gpu - oracle| <= 1e-4 over outputs and final states;
  bf16 inputs: rms(gpu - oracle) / rms(oracle) <= 2e-2, for outputs and final states
  separately, over the whole tensor and over every (sequence, head) unit.
  Token-major units (outputs, per-token gradients) are also gated window by window:
  every run of 64 consecutive tokens (one chunk; the last may be shorter) must meet
  rms(delta) / rms(oracle) <= 2e-2 on its own, so an error confined to one chunk of a
  long sequence cannot hide in the sequence's average.  A window's oracle rms is
  floored at 1 % of its unit's (a window of near-zero outputs would otherwise turn
  rounding noise into a large ratio).  Diagnostic, bounded too: max |delta| over a
  unit divided by the unit's oracle rms, at most 0.25.  An output element six standard
  deviations out carries one or two percent of relative error from bf16 operands and
  rounding, about 0.1 of the rms (0.124 seen under strong decay); a corrupted chunk
  gives errors of the order of the rms itself.
"""

import numpy as np

FP32_MAX_ABS = 1e-4
BF16_RMS_REL = 2e-2
WINDOW = 64
WINDOW_RMS_FLOOR = 1e-2
BF16_MAX_REL = 0.25


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


def unit_stats(got, ref, window=WINDOW):
    """(rms-rel, worst window rms-rel, max|delta| / rms) of one token-major unit
    (tokens on the first axis)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    T = ref.shape[0]
    if T == 0:
        return 0.0, 0.0, 0.0
    d = (got - ref).reshape(T, -1)
    r = ref.reshape(T, -1)
    unit_rms = rms(r)
    pad = (-T) % window
    d2 = np.pad(d * d, ((0, pad), (0, 0))).reshape(-1, window * d.shape[1]).sum(1)
    r2 = np.pad(r * r, ((0, pad), (0, 0))).reshape(-1, window * d.shape[1]).sum(1)
    n = np.full(d2.shape, window * d.shape[1], dtype=np.float64)
    n[-1] = (window - pad) * d.shape[1]
    floor = (WINDOW_RMS_FLOOR * unit_rms) ** 2
    w_rel = np.sqrt((d2 / n) / np.maximum(r2 / n, floor)) if unit_rms > 0 else np.sqrt(d2 / n)
    rel = float(np.sqrt(np.mean(d * d)) / unit_rms) if unit_rms > 0 else rms(d)
    mx = float(np.max(np.abs(d))) / unit_rms if unit_rms > 0 else float(np.max(np.abs(d)))
    return rel, float(np.max(w_rel)), mx


def check_unit(got, ref, what):
    """The bf16 bars for one token-major unit: whole unit, every window, max/rms.
    Returns the three statistics."""
    rel, worst, mx = unit_stats(got, ref)
    assert rel <= BF16_RMS_REL, f"{what}: rms-rel {rel:.3e} > {BF16_RMS_REL}"
    assert worst <= BF16_RMS_REL, f"{what}: worst {WINDOW}-token window rms-rel {worst:.3e} > {BF16_RMS_REL}"
    assert mx <= BF16_MAX_REL, f"{what}: max|delta|/rms {mx:.3e} > {BF16_MAX_REL}"
    return rel, worst, mx


def check(dtype, got, ref, what, units=None, windows=False):
    """Assert the bar for ``dtype`` ("fp32" | "bf16").  ``units`` optionally lists
    (label, got_slice, ref_slice) triples checked one by one (bf16 only); with
    ``windows`` each unit is token-major and also gated per 64-token window and on
    max|delta|/rms."""
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
        if windows:
            check_unit(gs, rs, f"{what} {label}")
        else:
            e = rms_rel(gs, rs)
            assert e <= BF16_RMS_REL, f"{what} {label}: rms-rel {e:.3e} > {BF16_RMS_REL}"
    return err


def check_rows(got, ref, what):
    """The bf16 bar on every row of [units, n] arrays at once (one row per unit);
    returns the worst row's rms-rel."""
    got = np.asarray(got, dtype=np.float64).reshape(np.shape(ref)[0], -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(got.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values from the GPU"
    d = np.sqrt(np.mean((got - ref) ** 2, axis=1))
    r = np.sqrt(np.mean(ref ** 2, axis=1))
    rel = np.where(r > 0, d / np.where(r > 0, r, 1.0), d)
    worst = int(np.argmax(rel))
    assert rel[worst] <= BF16_RMS_REL, f"{what}: unit {worst} rms-rel {rel[worst]:.3e} > {BF16_RMS_REL}"
    return float(rel[worst])
