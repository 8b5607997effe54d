"""The parity metrics themselves (tests/parity.py), on synthetic errors: an error
confined to one 64-token chunk of a long unit passes the whole-unit gate but fails
the window gate; uniform rounding-sized noise passes every gate."""

import numpy as np
import pytest

import parity


def test_one_corrupted_chunk_fails_the_window_gate_only():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((65536, 128))
    got = ref + 4e-3 * rng.standard_normal(ref.shape)     # the typical bf16 error level
    got[64 * 700: 64 * 701] += 0.6 * rng.standard_normal((64, 128))   # one bad chunk
    rel, worst, mx = parity.unit_stats(got, ref)
    assert rel <= parity.BF16_RMS_REL               # the unit average hides it
    assert worst > parity.BF16_RMS_REL              # the window gate does not
    assert mx > parity.BF16_MAX_REL
    with pytest.raises(AssertionError, match="window"):
        parity.check_unit(got, ref, "planted")


def test_rounding_noise_passes_and_ragged_tail_is_a_window():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((1000, 64))                 # 15 full windows + 40 rows
    got = ref * (1 + 2 ** -8 * rng.uniform(-1, 1, ref.shape))
    rel, worst, mx = parity.check_unit(got, ref, "noise")
    assert rel < 5e-3 and worst < 5e-3 and mx < 2e-2
    got[-3:] += 1.0                                       # corrupt the short last window
    assert parity.unit_stats(got, ref)[1] > parity.BF16_RMS_REL


def test_window_floor_for_near_zero_windows():
    ref = np.ones((256, 8))
    ref[64:128] = 1e-9                                    # a window of near-zero outputs
    got = ref.copy()
    got[64:128] += 1e-4                                   # absolute noise there
    _, worst, _ = parity.unit_stats(got, ref)
    unit_rms = parity.rms(ref)
    # judged against 1 % of the unit rms, not against the window's own 1e-9
    assert worst == pytest.approx(1e-4 / (parity.WINDOW_RMS_FLOOR * unit_rms), rel=1e-6)
    assert worst < parity.BF16_RMS_REL
