"""Pin for oracle.pool.recurrence_parallel, which fans (sequence, head) units over
worker processes for the CPU baseline: its result must be the plain recurrence's,
element for element, whatever the split -- a dropped, duplicated or reordered unit
fails here."""

import numpy as np
import pytest

from oracle import recurrence
from oracle.pool import recurrence_parallel


def case(seed, U, T=40, d_k=6, d_v=5, decay="channel", init=True):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((U, T, d_k))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    g = {"channel": -rng.uniform(0.001, 0.1, (U, T, d_k)),
         "head": -rng.uniform(0.001, 0.1, (U, T)), "none": None}[decay]
    return dict(q=rng.standard_normal((U, T, d_k)), k=k, v=rng.standard_normal((U, T, d_v)),
                g=g, beta=rng.uniform(0.0, 1.0, (U, T)),
                initial_state=rng.standard_normal((U, d_v, d_k)) if init else None)


@pytest.mark.parametrize("U,procs,decay,init", [
    (7, 3, "channel", True),      # uneven slices
    (2, 5, "channel", True),      # fewer units than processes
    (1, 4, "head", False),
    (6, 6, "none", True),
    (5, 1, "channel", False),     # in-process path
])
def test_pool_equals_recurrence(U, procs, decay, init):
    c = case(U * 10 + procs, U, decay=decay, init=init)
    o_ref, s_ref = recurrence(c["q"], c["k"], c["v"], c["g"], c["beta"], scale=0.3,
                              initial_state=c["initial_state"])
    o, s, used = recurrence_parallel(c["q"], c["k"], c["v"], c["g"], c["beta"], scale=0.3,
                                     initial_state=c["initial_state"], processes=procs)
    assert used == min(procs, U)
    assert o.shape == o_ref.shape and s.shape == s_ref.shape
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(s, s_ref)


def test_pool_units_are_not_permuted():
    """Units with different inputs land in their own rows (a swapped or duplicated
    slice would put another unit's results there)."""
    c = case(99, 9, T=8)
    o, s, _ = recurrence_parallel(c["q"], c["k"], c["v"], c["g"], c["beta"],
                                  initial_state=c["initial_state"], processes=4)
    for u in range(9):
        ou, su = recurrence(c["q"][u], c["k"][u], c["v"][u], c["g"][u], c["beta"][u],
                            initial_state=c["initial_state"][u])
        np.testing.assert_array_equal(o[u], ou)
        np.testing.assert_array_equal(s[u], su)
