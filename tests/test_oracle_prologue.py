"""Pins for the oracle's prologue (raw projections -> unit keys, sigmoid write strength,
sigmoid retention gate), run on the oracle and on copies with planted mistakes.

What the pins rest on (step-by-step page, the key-normalisation warning and FAQ;
deep-dive page, "From attention to recurrent state", on how the gate is
parameterised; readings in ``oracle/kda_prologue.py``):

* closed forms of the normalisation: a Pythagorean key (2, 3, 6) has norm 7, so its
  unit key is (2, 3, 6) / 7 up to the eps term; every normalised row has norm
  |k| / sqrt(|k|^2 + eps); a zero key stays zero;
* exact sigmoid values: sigmoid(0) = 1/2, sigmoid(+-ln 3) = 3/4, 1/4; saturation
  without overflow at +-50;
* invariance: outputs do not change when a raw key is scaled by a positive factor;
* special cases that reduce to pinned or library results: retention and write logits
  of +40 (alpha, beta -> 1) with orthonormal keys build S_T = V^T K (a matmul); a
  retention logit of -40 (alpha -> 0) leaves only the last write, S_t = beta_t v_t
  k_t^T.
"""

import numpy as np
import pytest

from oracle import BETA_LOGIT, GATE_LOGIT, NORM_K, decode_step, forward, recurrence
from oracle import kda_prologue as kp

EPS = kp.EPS
LN3 = np.log(3.0)


def pin_pythagorean_key(pro):
    k = np.array([[2.0, 3.0, 6.0], [-6.0, 2.0, 3.0]])
    kn, _, _ = pro(k, None, np.zeros(2), NORM_K)
    return np.allclose(kn, k / 7.0, rtol=0, atol=1e-8)


def pin_norm_closed_form(pro):
    rng = np.random.default_rng(1)
    k = rng.standard_normal((5, 7, 16)) * rng.uniform(0.2, 5, (5, 7, 1))
    kn, _, _ = pro(k, None, np.zeros((5, 7)), NORM_K)
    n2 = np.sum(k * k, axis=-1)
    want = np.sqrt(n2) / np.sqrt(n2 + EPS)
    return np.allclose(np.linalg.norm(kn, axis=-1), want, rtol=1e-12, atol=0)


def pin_zero_key(pro):
    kn, _, _ = pro(np.zeros((3, 8)), None, np.zeros(3), NORM_K)
    return np.all(kn == 0.0)


def pin_sigmoid_values(pro):
    b = np.array([0.0, LN3, -LN3, 50.0, -50.0])
    _, g, beta = pro(np.ones((5, 4)), b.copy(), b.copy(), BETA_LOGIT | GATE_LOGIT)
    ok = np.allclose(beta[:3], [0.5, 0.75, 0.25], rtol=0, atol=1e-15)
    ok &= abs(beta[3] - 1.0) < 1e-15 and 0 < beta[4] < 1e-21
    ok &= np.allclose(np.exp(g[:3]), [0.5, 0.75, 0.25], rtol=0, atol=1e-15)
    ok &= -1e-20 < g[3] < 0 and abs(g[4] + 50.0) < 1e-12
    return bool(ok and np.all(np.isfinite(g)) and np.all(np.isfinite(beta)))


def _case(seed, U=2, T=12, d_k=6, d_v=5):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((U, T, d_k)), rng.standard_normal((U, T, d_k)) * 3,
            rng.standard_normal((U, T, d_v)), rng.standard_normal((U, T, d_k)),
            rng.standard_normal((U, T)), 0.3 * rng.standard_normal((U, d_v, d_k)))


def _run(pro, q, k, v, g, b, s0, flags):
    k2, g2, b2 = pro(k, g, b, flags)
    return recurrence(q, k2, v, g2, b2, scale=0.4, initial_state=s0)


def pin_scale_invariance(pro):
    q, k, v, g, b, s0 = _case(2)
    f = NORM_K | BETA_LOGIT | GATE_LOGIT
    o1, s1 = _run(pro, q, k, v, g, b, s0, f)
    ok = True
    for c in (0.5, 3.0):
        o2, s2 = _run(pro, q, c * k, v, g, b, s0, f)
        ok &= np.allclose(o2, o1, rtol=1e-5, atol=1e-6) and np.allclose(s2, s1, rtol=1e-5,
                                                                        atol=1e-6)
    return bool(ok)


def pin_saturated_gates_build_matmul(pro):
    rng = np.random.default_rng(3)
    d = 6
    K = np.linalg.qr(rng.standard_normal((d, d)))[0].T[None] * rng.uniform(0.5, 4)  # raw scale
    V = rng.standard_normal((1, d, 4))
    q = rng.standard_normal((1, d, d))
    _, s = _run(pro, q, K, V, np.full((1, d, d), 40.0), np.full((1, d), 40.0), None,
                NORM_K | BETA_LOGIT | GATE_LOGIT)
    # unit keys up to the eps term (pinned on its own above)
    Kn = K[0] / np.sqrt(np.linalg.norm(K[0], axis=1, keepdims=True) ** 2 + EPS)
    return np.allclose(s[0], V[0].T @ Kn, rtol=0, atol=1e-9)


def pin_forget_all_keeps_last_write(pro):
    q, k, v, _, b, s0 = _case(4)
    g = np.full(k.shape, -40.0)
    _, s = _run(pro, q, k, v, g, b, s0, NORM_K | BETA_LOGIT | GATE_LOGIT)
    kn = k[:, -1] / np.sqrt(np.sum(k[:, -1] ** 2, axis=-1, keepdims=True) + EPS)
    bt = 1 / (1 + np.exp(-b[:, -1]))
    want = bt[:, None, None] * v[:, -1, :, None] * kn[:, None, :]
    return np.allclose(s, want, rtol=0, atol=1e-12)


PINS = [pin_pythagorean_key, pin_norm_closed_form, pin_zero_key, pin_sigmoid_values,
        pin_scale_invariance, pin_saturated_gates_build_matmul,
        pin_forget_all_keeps_last_write]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_prologue_pinned(pin):
    assert pin(kp.prologue)


def _mutant(kind):
    def pro(k, g, beta, flags):
        k = np.asarray(k, dtype=np.float64)
        beta = np.asarray(beta, dtype=np.float64)
        if flags & NORM_K:
            if kind == "wrong_axis":
                k = k / np.sqrt(np.sum(k * k, axis=0, keepdims=True) + EPS)
            elif kind == "no_sqrt":
                k = k / (np.sum(k * k, axis=-1, keepdims=True) + EPS)
            else:
                k = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + EPS)
        if flags & BETA_LOGIT:
            beta = 1 / (1 + np.exp(beta if kind == "beta_sign" else -beta))
        if g is not None:
            g = np.asarray(g, dtype=np.float64)
            if flags & GATE_LOGIT:
                if kind == "gate_sign":
                    g = -np.logaddexp(0.0, g)
                elif kind == "gate_no_log":
                    g = 1 / (1 + np.exp(-g))
                else:
                    g = -np.logaddexp(0.0, -g)
        return k, g, beta
    return pro


def _all_pass(pro):
    with np.errstate(all="ignore"):
        return all(pin(pro) for pin in PINS)


def test_harness_accepts_the_faithful_copy():
    assert _all_pass(_mutant("none"))


@pytest.mark.parametrize("kind", ["wrong_axis", "no_sqrt", "beta_sign", "gate_sign",
                                  "gate_no_log"])
def test_planted_prologue_mistake_is_caught(kind):
    assert not _all_pass(_mutant(kind)), kind


def test_forward_and_decode_apply_the_prologue():
    """Wiring: forward / decode_step with flags equal the plain calls on the
    transformed inputs, for each decay form."""
    rng = np.random.default_rng(5)
    B, T, H, d = 1, 9, 2, 4
    q, k, v = (rng.standard_normal((B, T, H, d)) for _ in range(3))
    b = rng.standard_normal((B, T, H))
    f = NORM_K | BETA_LOGIT | GATE_LOGIT
    for g in (rng.standard_normal((B, T, H, d)), rng.standard_normal((B, T, H)), None):
        k2, g2, b2 = kp.prologue(k, g, b, f)
        o1, s1 = forward(q, k, v, g, b, flags=f)
        o2, s2 = forward(q, k2, v, g2, b2)
        assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
        st = rng.standard_normal((B, H, d, d))
        gt = None if g is None else g[:, 0]
        d1 = decode_step(q[:, 0], k[:, 0], v[:, 0], gt, b[:, 0], st, flags=f)
        k3, g3, b3 = kp.prologue(k[:, 0], gt, b[:, 0], f)
        d2 = decode_step(q[:, 0], k3, v[:, 0], g3, b3, st)
        assert np.array_equal(d1[0], d2[0]) and np.array_equal(d1[1], d2[1])
