"""Pins for the oracle's two simpler decay variants (Gated DeltaNet: one scalar decay
per token; DeltaNet: no decay), run on the oracle and on copies with planted mistakes.

What the pins rest on (step-by-step page, "From quadratic attention to fixed state: a
brief history" and "DeltaNet, Gated DeltaNet, and KDA: comparison table"; deep-dive
page, "From attention to recurrent state", for the forget-plus-write form):

* the forget-plus-write matrix form S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T)
  + beta_t v_t k_t^T with a scalar alpha_t (and alpha_t = 1 for DeltaNet), evaluated
  with plain matrix products in float64 and as exact rational brute force;
* closed forms: beta = 0 leaves S_t = (alpha_1 ... alpha_t) S_0;
* a special case that reduces to a matmul: DeltaNet with orthonormal keys and
  beta = 1 builds S_T = V^T K;
* exact one-hot retrieval with DeltaNet;
* reductions to the already pinned per-channel path: a scalar decay equals a
  per-channel decay with all channels equal, no decay equals g = 0;
* wrappers: the chunkwise algebra, packed varlen batches and decode steps agree with
  the recurrence for both variants.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import chunked, decode_step, default_scale, forward, recurrence


def unit_rows(rng, *shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def case(seed, U=2, T=31, d_k=6, d_v=6, s0=True):
    rng = np.random.default_rng(seed)
    return dict(q=rng.standard_normal((U, T, d_k)), k=unit_rows(rng, U, T, d_k),
                v=rng.standard_normal((U, T, d_v)), g=-rng.uniform(0.001, 0.3, (U, T)),
                beta=1 / (1 + np.exp(-rng.standard_normal((U, T)))),
                initial_state=0.5 * rng.standard_normal((U, d_v, d_k)) if s0 else None)


def forget_write_reference(q, k, v, alpha, beta, scale, s0):
    """S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T, o_t = S_t scale q_t."""
    U, T, d_k = k.shape
    S = np.zeros((U, v.shape[2], d_k)) if s0 is None else s0.copy()
    o = np.empty((U, T, v.shape[2]))
    eye = np.eye(d_k)
    for u in range(U):
        for t in range(T):
            kk = k[u, t][:, None]
            S[u] = alpha[u, t] * S[u] @ (eye - beta[u, t] * (kk @ kk.T)) \
                + beta[u, t] * np.outer(v[u, t], k[u, t])
            o[u, t] = S[u] @ q[u, t] * scale
    return o, S


# ------------------------------------------------------------------ scalar decay pins
def pin_scalar_forget_write(rec):
    c = case(1)
    s = default_scale(6)
    o, S = rec(scale=s, **c)
    o_ref, S_ref = forget_write_reference(c["q"], c["k"], c["v"], np.exp(c["g"]), c["beta"], s,
                                          c["initial_state"])
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)


def pin_scalar_beta_zero(rec):
    c = case(2)
    c["beta"] = np.zeros_like(c["beta"])
    o, S = rec(scale=0.3, **c)
    G = np.cumsum(c["g"], axis=1)                               # [U, T]
    S0 = c["initial_state"]
    o_ref = 0.3 * np.exp(G)[:, :, None] * np.einsum("uvk,utk->utv", S0, c["q"])
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, np.exp(G[:, -1])[:, None, None] * S0, rtol=1e-12, atol=1e-12)


def pin_scalar_exact_rational(rec):
    rng = np.random.default_rng(3)
    d_k, d_v, T = 3, 2, 4

    def rat(lo, hi, den=8):
        return Fraction(int(rng.integers(lo * den, hi * den + 1)), den)

    K = [[rat(-1, 1) for _ in range(d_k)] for _ in range(T)]
    V = [[rat(-2, 2) for _ in range(d_v)] for _ in range(T)]
    Qv = [[rat(-2, 2) for _ in range(d_k)] for _ in range(T)]
    AL = [Fraction(int(rng.integers(1, 9)), 8) for _ in range(T)]
    BE = [Fraction(int(rng.integers(0, 9)), 8) for _ in range(T)]
    S = [[rat(-1, 1) for _ in range(d_k)] for _ in range(d_v)]
    S0 = [row[:] for row in S]
    outs = []
    for t in range(T):
        F = [[(1 if i == j else 0) - BE[t] * K[t][i] * K[t][j] for j in range(d_k)]
             for i in range(d_k)]
        S = [[AL[t] * sum(S[i][m] * F[m][j] for m in range(d_k)) + BE[t] * V[t][i] * K[t][j]
              for j in range(d_k)] for i in range(d_v)]
        outs.append([sum(S[i][j] * Qv[t][j] for j in range(d_k)) for i in range(d_v)])
    f = lambda m: np.array([[float(x) for x in r] for r in m])
    o, s = rec(f(Qv)[None], f(K)[None], f(V)[None], np.log([[float(a) for a in AL]]),
               np.array([[float(b) for b in BE]]), scale=1.0, initial_state=f(S0)[None])
    np.testing.assert_allclose(o[0], f(outs), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s[0], f(S), rtol=1e-13, atol=1e-13)


def pin_scalar_equals_equal_channels(rec):
    c = case(4, d_k=5, d_v=3)
    o, S = rec(scale=0.7, **c)
    cc = dict(c, g=np.repeat(c["g"][:, :, None], 5, axis=2))
    o_ref, S_ref = recurrence(scale=0.7, **cc)          # the pinned per-channel path
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S, S_ref, rtol=1e-13, atol=1e-13)


SCALAR_PINS = [pin_scalar_forget_write, pin_scalar_beta_zero, pin_scalar_exact_rational,
               pin_scalar_equals_equal_channels]


# ---------------------------------------------------------------------- no-decay pins
def pin_none_forget_write(rec):
    c = case(5)
    s = default_scale(6)
    o, S = rec(c["q"], c["k"], c["v"], None, c["beta"], scale=s, initial_state=c["initial_state"])
    o_ref, S_ref = forget_write_reference(c["q"], c["k"], c["v"], np.ones_like(c["beta"]),
                                          c["beta"], s, c["initial_state"])
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, rtol=1e-12, atol=1e-12)


def pin_none_orthonormal_matmul(rec):
    rng = np.random.default_rng(6)
    d_k, d_v = 7, 4
    Qm, _ = np.linalg.qr(rng.standard_normal((d_k, d_k)))
    K, V = Qm.T, rng.standard_normal((d_k, d_v))
    q = rng.standard_normal((d_k, d_k))
    o, s = rec(q[None], K[None], V[None], None, np.ones((1, d_k)), scale=1.0, initial_state=None)
    np.testing.assert_allclose(s[0], V.T @ K, rtol=0, atol=1e-13)
    for t in range(d_k):
        np.testing.assert_allclose(o[0, t], V[: t + 1].T @ (K[: t + 1] @ q[t]), atol=1e-13)


def pin_none_one_hot_retrieval(rec):
    d_k, d_v, n_write = 8, 5, 6
    rng = np.random.default_rng(7)
    order = rng.permutation(d_k)[:n_write]
    vals = rng.standard_normal((n_write, d_v))
    for i in range(n_write):
        T = n_write + 1
        k = np.zeros((1, T, d_k))
        k[0, np.arange(n_write), order] = 1.0
        k[0, -1] = k[0, i]
        q = np.zeros((1, T, d_k))
        q[0, -1] = k[0, i]
        v = np.zeros((1, T, d_v))
        v[0, :n_write] = vals
        beta = np.ones((1, T))
        beta[0, -1] = 0.0
        o, s = rec(q, k, v, None, beta, scale=1.0, initial_state=None)
        assert np.array_equal(o[0, -1], vals[i])


def pin_none_equals_zero_gate(rec):
    c = case(8)
    o, S = rec(c["q"], c["k"], c["v"], None, c["beta"], scale=0.5, initial_state=c["initial_state"])
    o_ref, S_ref = recurrence(c["q"], c["k"], c["v"], np.zeros(c["k"].shape), c["beta"],
                              scale=0.5, initial_state=c["initial_state"])
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S, S_ref, rtol=1e-13, atol=1e-13)


NONE_PINS = [pin_none_forget_write, pin_none_orthonormal_matmul, pin_none_one_hot_retrieval,
             pin_none_equals_zero_gate]


@pytest.mark.parametrize("pin", SCALAR_PINS + NONE_PINS, ids=lambda p: p.__name__)
def test_oracle_variant_pinned(pin):
    pin(recurrence)


# ------------------------------------------------------------ planted mistakes are caught
def _mutant(kind):
    """A copy of the recurrence for scalar / absent decay with one planted mistake."""
    def rec(q, k, v, g, beta, scale=None, initial_state=None):
        q, k, v, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta))
        U, T, d_k = k.shape
        scale = d_k ** -0.5 if scale is None else scale
        S = np.zeros((U, v.shape[2], d_k)) if initial_state is None else np.array(initial_state, float)
        o = np.empty((U, T, v.shape[2]))
        for t in range(T):
            a = np.ones(U) if g is None else np.exp(np.asarray(g, dtype=np.float64)[:, t])
            if kind == "no_decay":
                a = np.ones(U)
            if kind == "decay_squared":
                a = a * a
            if kind == "none_decays":
                a = np.full(U, np.exp(-0.05)) if g is None else a
            kt, vt, b = k[:, t], v[:, t], beta[:, t, None]
            prev = S.copy()
            if kind != "decay_after_write":
                S = S * a[:, None, None]
            src = prev if kind == "predict_undecayed" else S
            e = b * (vt - np.einsum("uvk,uk->uv", src, kt))
            S = S + e[:, :, None] * kt[:, None, :]
            if kind == "decay_after_write":
                S = S * a[:, None, None]
            o[:, t] = np.einsum("uvk,uk->uv", S, q[:, t]) * scale
        return o, S
    return rec


def _all_pass(rec, pins):
    for pin in pins:
        try:
            pin(rec)
        except Exception:  # noqa: BLE001 - any failure means the pin caught it
            return False
    return True


def test_variant_harness_accepts_the_faithful_copy():
    assert _all_pass(_mutant("none"), SCALAR_PINS + NONE_PINS)


@pytest.mark.parametrize("kind", ["no_decay", "decay_squared", "decay_after_write",
                                  "predict_undecayed"])
def test_planted_scalar_mistake_is_caught(kind):
    assert not _all_pass(_mutant(kind), SCALAR_PINS), kind


def test_planted_none_mistake_is_caught():
    assert not _all_pass(_mutant("none_decays"), NONE_PINS)


# --------------------------------------------------------------------------- wrappers
@pytest.mark.parametrize("decay", ["scalar", "none"])
@pytest.mark.parametrize("chunk", [1, 7, 64])
def test_chunked_matches_recurrence(decay, chunk):
    c = case(9, U=1, T=150, d_k=8, d_v=5)
    g = c["g"][0] if decay == "scalar" else None
    o_r, s_r = recurrence(c["q"][0], c["k"][0], c["v"][0], g, c["beta"][0], scale=0.35,
                          initial_state=c["initial_state"][0])
    o_c, s_c = chunked(c["q"][0], c["k"][0], c["v"][0], g, c["beta"][0], 0.35,
                       c["initial_state"][0], chunk=chunk)
    np.testing.assert_allclose(o_c, o_r, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s_c, s_r, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("decay", ["scalar", "none"])
def test_forward_varlen_and_decode(decay):
    rng = np.random.default_rng(10)
    lengths, H, d_k, d_v = [9, 0, 14], 2, 5, 4
    T = sum(lengths)
    q = rng.standard_normal((1, T, H, d_k))
    k = unit_rows(rng, 1, T, H, d_k)
    v = rng.standard_normal((1, T, H, d_v))
    g = -rng.uniform(0.001, 0.2, (1, T, H)) if decay == "scalar" else None
    beta = rng.uniform(0, 1, (1, T, H))
    s0 = rng.standard_normal((3, H, d_v, d_k)) * 0.3
    cu = np.cumsum([0] + lengths).astype(np.int32)
    o, fin = forward(q, k, v, g, beta, cu_seqlens=cu, scale=0.4, initial_state=s0)
    for n in range(3):
        lo, hi = cu[n], cu[n + 1]
        for h in range(H):
            sl = (0, slice(lo, hi), h)
            o_ref, s_ref = recurrence(q[sl], k[sl], v[sl], None if g is None else g[sl], beta[sl],
                                      scale=0.4, initial_state=s0[n, h])
            np.testing.assert_allclose(o[sl], o_ref, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(fin[n, h], s_ref, rtol=1e-13, atol=1e-13)
            # the same tokens as decode steps (one sequence at a time)
            state = s0[n:n + 1]
            for t in range(lo, hi):
                od, state = decode_step(q[:, t], k[:, t], v[:, t],
                                        None if g is None else g[:, t], beta[:, t],
                                        state if t > lo else s0[n:n + 1], scale=0.4)
                np.testing.assert_allclose(od[0, h], o[0, t, h], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(state[0, h], fin[n, h], rtol=1e-12, atol=1e-13)
