"""Pins for the fp64 oracle: it is checked against things other than itself.

Every pin takes the recurrence as an argument, so the same pins are run on the
oracle (all must pass) and on copies of it with one planted mistake each (at
least one pin must fail for every planted mistake).  What each pin rests on:

* hand-derived worked example (tests/golden/kda_two_token_d2.txt);
* closed forms: beta = 0 decays only; one token from a zero state writes beta v k^T;
* a special case that reduces to a library routine: orthonormal keys with
  alpha = 1, beta = 1 build S_T = V^T K (a plain matmul);
* exact one-hot retrieval;
* the forget-plus-write (Householder) factorisation of the delta rule given on the
  deep-dive page ("From attention to recurrent state"), extended with the decay,
  both in float64 and as exact rational brute force;
* invariants: linearity in (V, S_0), the per-token write identity and the norm
  bound, split/resume, packed varlen = separate sequences, T decode steps = one
  prefill of T tokens, recurrence = chunkwise algebra.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import chunked, decode_step, default_scale, forward, recurrence

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kda_two_token_d2.txt")


# ----------------------------------------------------------------------------- helpers
def unit_rows(rng, *shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def random_case(seed, U=3, T=37, d_k=6, d_v=5, s0=True):
    rng = np.random.default_rng(seed)
    return dict(
        q=rng.standard_normal((U, T, d_k)),
        k=unit_rows(rng, U, T, d_k),
        v=rng.standard_normal((U, T, d_v)),
        g=-rng.uniform(0.001, 0.3, (U, T, d_k)),
        beta=1 / (1 + np.exp(-rng.standard_normal((U, T)))),
        initial_state=0.5 * rng.standard_normal((U, d_v, d_k)) if s0 else None,
    )


def parse_golden(path):
    vals = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        name, rhs = line.split(":", 1)
        rows = [[Fraction(x) for x in r.split()] for r in rhs.split(";")]
        vals[name.strip()] = rows if len(rows) > 1 else rows[0]
    return vals


def fr2np(x):
    return np.array([[float(e) for e in r] for r in x]) if isinstance(x[0], list) \
        else np.array([float(e) for e in x])


# ----------------------------------------------------------------------------- pins
def pin_golden(rec):
    gv = parse_golden(GOLDEN)
    q = np.stack([fr2np(gv["q1"]), fr2np(gv["q2"])])[None]
    k = np.stack([fr2np(gv["k1"]), fr2np(gv["k2"])])[None]
    v = np.stack([fr2np(gv["v1"]), fr2np(gv["v2"])])[None]
    g = np.log(np.stack([fr2np(gv["alpha1"]), fr2np(gv["alpha2"])]))[None]
    beta = np.array([[float(gv["beta1"][0]), float(gv["beta2"][0])]])
    s0 = fr2np(gv["S0"])[None]
    o, s = rec(q, k, v, g, beta, scale=1.0, initial_state=s0)
    np.testing.assert_allclose(o[0, 0], fr2np(gv["o1"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0, 1], fr2np(gv["o2"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(s[0], fr2np(gv["S2"]), rtol=0, atol=1e-14)


def pin_beta_zero_decays_only(rec):
    c = random_case(1)
    c["beta"] = np.zeros_like(c["beta"])
    scale = 0.37
    o, s = rec(scale=scale, **c)
    G = np.cumsum(c["g"], axis=1)                       # [U, T, d_k]
    S0 = c["initial_state"]
    # closed form: S_t = S0 Diag(exp(G_t)), o_t = S_t scale q_t
    o_ref = np.einsum("uvk,utk->utv", S0, np.exp(G) * c["q"]) * scale
    s_ref = S0 * np.exp(G[:, -1])[:, None, :]
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, s_ref, rtol=1e-12, atol=1e-12)


def pin_one_token_from_zero(rec):
    c = random_case(2, T=1, s0=False)
    scale = 0.61
    o, s = rec(scale=scale, **c)
    b = c["beta"][:, 0]
    k, v, q = c["k"][:, 0], c["v"][:, 0], c["q"][:, 0]
    s_ref = b[:, None, None] * v[:, :, None] * k[:, None, :]
    o_ref = (b * scale * np.sum(k * q, axis=1))[:, None] * v
    np.testing.assert_allclose(s, s_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o[:, 0], o_ref, rtol=1e-13, atol=1e-14)


def pin_one_hot_retrieval(rec):
    # alpha = 1, beta = 1, distinct one-hot keys from zero: S k_i = v_i exactly;
    # a later read token with beta = 0, g = 0, q = k_i, scale = 1 returns v_i.
    d_k, d_v, n_write = 8, 5, 6
    rng = np.random.default_rng(3)
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
        v[0, -1] = rng.standard_normal(d_v)       # ignored: beta = 0 on the read token
        beta = np.ones((1, T))
        beta[0, -1] = 0.0
        g = np.zeros((1, T, d_k))
        o, s = rec(q, k, v, g, beta, scale=1.0, initial_state=None)
        assert np.array_equal(o[0, -1], vals[i])
        assert np.array_equal(s[0] @ k[0, i], vals[i])


def householder_reference(q, k, v, g, beta, scale, s0):
    """Forget-plus-write form S_t = S_{t-1} Diag(alpha_t)(I - beta_t k_t k_t^T)
    + beta_t v_t k_t^T (deep-dive page, equivalent formulation, with the decay)."""
    U, T, d_k = k.shape
    S = np.zeros((U, v.shape[2], d_k)) if s0 is None else s0.copy()
    o = np.empty((U, T, v.shape[2]))
    eye = np.eye(d_k)
    for u in range(U):
        for t in range(T):
            kk = k[u, t][:, None]
            forget = eye - beta[u, t] * (kk @ kk.T)
            S[u] = S[u] @ np.diag(np.exp(g[u, t])) @ forget + beta[u, t] * np.outer(v[u, t], k[u, t])
            o[u, t] = S[u] @ q[u, t] * scale
    return o, S


def pin_householder_form(rec):
    c = random_case(4, U=2, T=29, d_k=6, d_v=6)   # square: a row/column mix-up is silent
    scale = default_scale(6)
    o, s = rec(scale=scale, **c)
    o_ref, s_ref = householder_reference(c["q"], c["k"], c["v"], c["g"], c["beta"], scale,
                                         c["initial_state"])
    np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s, s_ref, rtol=1e-12, atol=1e-12)


def pin_orthonormal_keys_matmul(rec):
    # alpha = 1, beta = 1, keys = rows of an orthogonal matrix, zero state:
    # every write lands in an untouched direction, so S_T = V^T K.
    rng = np.random.default_rng(5)
    d_k, d_v = 7, 4
    Qm, _ = np.linalg.qr(rng.standard_normal((d_k, d_k)))
    K = Qm.T                                      # rows orthonormal
    V = rng.standard_normal((d_k, d_v))
    q = rng.standard_normal((d_k, d_k))
    o, s = rec(q[None], K[None], V[None], np.zeros((1, d_k, d_k)), np.ones((1, d_k)),
               scale=1.0, initial_state=None)
    np.testing.assert_allclose(s[0], V.T @ K, rtol=0, atol=1e-13)
    # the read after t writes is (sum_{i<=t} v_i k_i^T) q_t
    for t in range(d_k):
        np.testing.assert_allclose(o[0, t], V[: t + 1].T @ (K[: t + 1] @ q[t]), atol=1e-13)


def pin_linearity(rec):
    a, b = 0.7, -1.3
    c1 = random_case(6)
    c2 = random_case(7)
    mix = dict(c1)
    mix["v"] = a * c1["v"] + b * c2["v"]
    mix["initial_state"] = a * c1["initial_state"] + b * c2["initial_state"]
    c2x = dict(c1, v=c2["v"], initial_state=c2["initial_state"])
    o1, s1 = rec(scale=0.5, **c1)
    o2, s2 = rec(scale=0.5, **c2x)
    om, sm = rec(scale=0.5, **mix)
    np.testing.assert_allclose(om, a * o1 + b * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sm, a * s1 + b * s2, rtol=1e-12, atol=1e-12)


def pin_identity_gate_no_write(rec):
    c = random_case(8)
    c["g"] = np.zeros_like(c["g"])
    c["beta"] = np.zeros_like(c["beta"])
    o, s = rec(scale=0.9, **c)
    assert np.array_equal(s, c["initial_state"])
    np.testing.assert_allclose(o, 0.9 * np.einsum("uvk,utk->utv", c["initial_state"], c["q"]),
                               rtol=1e-13, atol=1e-13)


def pin_write_identity_and_norm(rec):
    # With |k_t| = 1: S_t k_t = (1 - beta_t) (decayed S_{t-1}) k_t + beta_t v_t, and
    # |S_t|_F <= |S_{t-1}|_F + |beta_t| |v_t| for beta in [0, 2], alpha in (0, 1].
    c = random_case(9, U=2, T=25)
    c["beta"] = np.random.default_rng(10).uniform(0, 2, c["beta"].shape)
    prev = c["initial_state"].copy()
    for t in range(c["beta"].shape[1]):
        sl = slice(t, t + 1)
        _, s = rec(c["q"][:, sl], c["k"][:, sl], c["v"][:, sl], c["g"][:, sl],
                   c["beta"][:, sl], scale=1.0, initial_state=prev)
        for u in range(2):
            kt, b = c["k"][u, t], c["beta"][u, t]
            decayed = prev[u] * np.exp(c["g"][u, t])[None, :]
            np.testing.assert_allclose(s[u] @ kt, (1 - b) * (decayed @ kt) + b * c["v"][u, t],
                                       rtol=1e-12, atol=1e-12)
            assert np.linalg.norm(s[u]) <= np.linalg.norm(prev[u]) + abs(b) * np.linalg.norm(
                c["v"][u, t]) + 1e-12
        prev = s


def pin_exact_rational(rec):
    # Exact rational brute force of the forget-plus-write form on tiny inputs, with
    # alpha passed directly; the float oracle gets g = log(alpha).
    rng = np.random.default_rng(11)
    d_k, d_v, T = 3, 2, 4

    def rat(lo, hi, den=8):
        return Fraction(int(rng.integers(lo * den, hi * den + 1)), den)

    K = [[rat(-1, 1) for _ in range(d_k)] for _ in range(T)]
    V = [[rat(-2, 2) for _ in range(d_v)] for _ in range(T)]
    Qv = [[rat(-2, 2) for _ in range(d_k)] for _ in range(T)]
    AL = [[Fraction(int(rng.integers(1, 9)), 8) for _ in range(d_k)] for _ in range(T)]
    BE = [Fraction(int(rng.integers(0, 9)), 8) for _ in range(T)]
    S = [[rat(-1, 1) for _ in range(d_k)] for _ in range(d_v)]
    S0 = [row[:] for row in S]
    outs = []
    for t in range(T):
        # S <- S Diag(alpha) (I - beta k k^T) + beta v k^T, exactly
        D = [[S[i][j] * AL[t][j] for j in range(d_k)] for i in range(d_v)]
        F = [[(1 if i == j else 0) - BE[t] * K[t][i] * K[t][j] for j in range(d_k)]
             for i in range(d_k)]
        S = [[sum(D[i][m] * F[m][j] for m in range(d_k)) + BE[t] * V[t][i] * K[t][j]
              for j in range(d_k)] for i in range(d_v)]
        outs.append([sum(S[i][j] * Qv[t][j] for j in range(d_k)) for i in range(d_v)])
    f = lambda m: np.array([[float(x) for x in r] for r in m])
    o, s = rec(f(Qv)[None], f(K)[None], f(V)[None], np.log(f(AL))[None],
               np.array([[float(b) for b in BE]]), scale=1.0, initial_state=f(S0)[None])
    np.testing.assert_allclose(o[0], f(outs), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s[0], f(S), rtol=1e-13, atol=1e-13)


PINS = [pin_golden, pin_beta_zero_decays_only, pin_one_token_from_zero, pin_one_hot_retrieval,
        pin_householder_form, pin_orthonormal_keys_matmul, pin_linearity,
        pin_identity_gate_no_write, pin_write_identity_and_norm, pin_exact_rational]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_recurrence_pinned(pin):
    pin(recurrence)


# ------------------------------------------------------------------ chunked == recurrent
@pytest.mark.parametrize("chunk", [1, 4, 16, 64])
def test_chunked_matches_recurrence(chunk):
    c = random_case(12, U=2, T=203, d_k=8, d_v=6)
    scale = default_scale(8)
    o_r, s_r = recurrence(scale=scale, **c)
    for u in range(2):
        o_c, s_c = chunked(c["q"][u], c["k"][u], c["v"][u], c["g"][u], c["beta"][u], scale,
                           c["initial_state"][u], chunk=chunk)
        np.testing.assert_allclose(o_c, o_r[u], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(s_c, s_r[u], rtol=1e-11, atol=1e-12)


def test_chunked_pinned_through_recurrence_pins():
    # The chunked form, wrapped to the recurrence's signature, also passes every pin.
    def rec_chunked(q, k, v, g, beta, scale=None, initial_state=None):
        U = np.asarray(beta).shape[0]
        scale = default_scale(np.asarray(k).shape[2]) if scale is None else scale
        outs = [chunked(q[u], k[u], v[u], g[u], beta[u], scale,
                        None if initial_state is None else initial_state[u], chunk=16)
                for u in range(U)]
        return np.stack([x[0] for x in outs]), np.stack([x[1] for x in outs])

    for pin in PINS:
        pin(rec_chunked)


# --------------------------------------------------------- batch / varlen / decode wrappers
def _batch_case(seed, lengths, H=3, d_k=6, d_v=5, s0=True):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    return dict(q=rng.standard_normal((1, T, H, d_k)), k=unit_rows(rng, 1, T, H, d_k),
                v=rng.standard_normal((1, T, H, d_v)), g=-rng.uniform(0.001, 0.2, (1, T, H, d_k)),
                beta=rng.uniform(0, 1, (1, T, H)),
                initial_state=rng.standard_normal((len(lengths), H, d_v, d_k)) * 0.3 if s0 else None,
                cu_seqlens=np.cumsum([0] + list(lengths)).astype(np.int32))


def test_varlen_equals_separate_sequences_and_split_resume():
    lengths = [17, 0, 40, 1, 23]
    c = _batch_case(13, lengths)
    o, fin = forward(c["q"], c["k"], c["v"], c["g"], c["beta"], cu_seqlens=c["cu_seqlens"],
                     scale=0.4, initial_state=c["initial_state"])
    cu = c["cu_seqlens"]
    for n, L in enumerate(lengths):
        lo, hi = cu[n], cu[n + 1]
        for h in range(3):
            sl = (0, slice(lo, hi), h)
            o_ref, s_ref = recurrence(c["q"][sl], c["k"][sl], c["v"][sl], c["g"][sl],
                                      c["beta"][sl], scale=0.4,
                                      initial_state=c["initial_state"][n, h])
            np.testing.assert_allclose(o[sl], o_ref, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(fin[n, h], s_ref, rtol=1e-13, atol=1e-13)
            if L == 0:
                assert np.array_equal(fin[n, h], c["initial_state"][n, h])
            if L > 2:
                # split / resume: the final state of a prefix seeds the rest
                m = L // 2
                a = (0, slice(lo, lo + m), h)
                b = (0, slice(lo + m, hi), h)
                o1, s1 = recurrence(c["q"][a], c["k"][a], c["v"][a], c["g"][a], c["beta"][a],
                                    scale=0.4, initial_state=c["initial_state"][n, h])
                o2, s2 = recurrence(c["q"][b], c["k"][b], c["v"][b], c["g"][b], c["beta"][b],
                                    scale=0.4, initial_state=s1)
                np.testing.assert_allclose(np.concatenate([o1, o2]), o_ref, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(s2, s_ref, rtol=1e-12, atol=1e-12)


def test_batched_layout_and_unit_subset():
    rng = np.random.default_rng(14)
    B, T, H, d = 2, 11, 3, 4
    q = rng.standard_normal((B, T, H, d))
    k = unit_rows(rng, B, T, H, d)
    v = rng.standard_normal((B, T, H, d))
    g = -rng.uniform(0, 0.1, (B, T, H, d))
    beta = rng.uniform(0, 1, (B, T, H))
    o, fin = forward(q, k, v, g, beta)
    for b in range(B):
        for h in range(H):
            o_ref, s_ref = recurrence(q[b, :, h], k[b, :, h], v[b, :, h], g[b, :, h],
                                      beta[b, :, h])
            np.testing.assert_allclose(o[b, :, h], o_ref, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(fin[b, h], s_ref, rtol=1e-13, atol=1e-13)
    o_s, fin_s = forward(q, k, v, g, beta, units=[(1, 2)])
    np.testing.assert_array_equal(o_s[1, :, 2], o[1, :, 2])
    assert np.isnan(o_s[0]).all() and np.isnan(fin_s[0]).all()


def test_decode_steps_equal_prefill():
    rng = np.random.default_rng(15)
    N, H, d_k, d_v, steps = 3, 2, 6, 4, 9
    S = rng.standard_normal((N, H, d_v, d_k)) * 0.1
    q = rng.standard_normal((steps, N, H, d_k))
    k = unit_rows(rng, steps, N, H, d_k)
    v = rng.standard_normal((steps, N, H, d_v))
    g = -rng.uniform(0, 0.1, (steps, N, H, d_k))
    beta = rng.uniform(0, 1, (steps, N, H))
    state = S.copy()
    outs = []
    for t in range(steps):
        o, new = decode_step(q[t], k[t], v[t], g[t], beta[t], state)
        outs.append(o)
        state = new
    # the same tokens as one prefill per (sequence, head)
    o_pre, fin = forward(q.transpose(1, 0, 2, 3), k.transpose(1, 0, 2, 3),
                         v.transpose(1, 0, 2, 3), g.transpose(1, 0, 2, 3),
                         beta.transpose(1, 0, 2), initial_state=S)
    np.testing.assert_allclose(np.stack(outs, axis=1), o_pre, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(state, fin, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------- planted mistakes are caught
def _mutant(kind):
    def rec(q, k, v, g, beta, scale=None, initial_state=None):
        q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
        U, T, d_k = k.shape
        d_v = v.shape[2]
        scale = d_k ** -0.5 if scale is None else scale
        S = np.zeros((U, d_v, d_k)) if initial_state is None else np.array(initial_state, float)
        o = np.empty((U, T, d_v))
        for t in range(T):
            kt, qt, vt, b = k[:, t], q[:, t], v[:, t], beta[:, t, None]
            a = np.exp(-g[:, t] if kind == "exp_sign" else g[:, t])
            prev = S.copy()
            if kind == "decay_rows":
                S = S * a[:, :, None]
            else:
                S = S * a[:, None, :]
            src = prev if kind == "predict_undecayed" else S
            p = np.einsum("uvk,uk->uv", src, kt)
            if kind == "no_beta":
                e = vt - p
            elif kind == "err_sign":
                e = b * (p - vt)
            elif kind == "beta_on_pred_only":
                e = vt - b * p
            else:
                e = b * (vt - p)
            read_from = S.copy()
            if kind == "outer_transposed":
                S = S + np.einsum("uk,uv->ukv", kt, e)
            else:
                S = S + e[:, :, None] * kt[:, None, :]
            sc = 1.0 if kind == "no_scale" else scale
            if kind == "read_before_write":
                o[:, t] = np.einsum("uvk,uk->uv", read_from, qt) * sc
            elif kind == "read_prev_state":
                o[:, t] = np.einsum("uvk,uk->uv", prev, qt) * sc
            else:
                o[:, t] = np.einsum("uvk,uk->uv", S, qt) * sc
        return o, S
    return rec


MUTANTS = ["decay_rows", "exp_sign", "predict_undecayed", "no_beta", "err_sign",
           "beta_on_pred_only", "outer_transposed", "no_scale", "read_before_write",
           "read_prev_state"]


def _square_pins_pass(rec):
    """Run every pin (shape errors count as failures); True if all pass."""
    for pin in PINS:
        try:
            pin(rec)
        except Exception:  # noqa: BLE001 - any failure means the pin caught it
            return False
    return True


def test_mutant_harness_accepts_the_faithful_copy():
    assert _square_pins_pass(_mutant("none"))


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    assert not _square_pins_pass(_mutant(kind)), f"no pin catches planted mistake {kind}"


def _chunk_mutant(kind):
    from scipy.linalg import solve_triangular

    def run(q, k, v, g, beta, scale, S, chunk):
        T = k.shape[0]
        o = np.empty((T, v.shape[1]))
        for st in range(0, T, chunk):
            r = slice(st, min(st + chunk, T))
            n = r.stop - r.start
            G = np.cumsum(g[r], axis=0)
            if kind == "exclusive_prefix":
                G = G - g[r]
            Kg, Ki, Qg = k[r] * np.exp(G), k[r] * np.exp(-G), scale * q[r] * np.exp(G)
            Kh = k[r] * (np.exp(G[-1]) if kind == "khat_end_only" else np.exp(G[-1] - G))
            A = np.tril(beta[r, None] * (Kg @ Ki.T), k=0 if kind == "a_with_diag" else -1)
            Tm = solve_triangular(np.eye(n) + A, np.diag(beta[r]), lower=True,
                                  unit_diagonal=kind != "a_with_diag")
            E = Tm @ (v[r] - Kg @ S.T)
            M = np.tril(Qg @ Ki.T, k=-1 if kind == "m_strict" else 0)
            o[r] = Qg @ S.T + M @ E
            S = (S if kind == "no_state_decay" else S * np.exp(G[-1])[None, :]) + E.T @ Kh
        return o, S
    return run


@pytest.mark.parametrize("kind", ["exclusive_prefix", "khat_end_only", "a_with_diag",
                                  "m_strict", "no_state_decay"])
def test_planted_chunk_mistake_is_caught(kind):
    c = random_case(16, U=1, T=70, d_k=5, d_v=4)
    args = [c[x][0] for x in ("q", "k", "v", "g", "beta")]
    o_r, s_r = recurrence(*args, scale=0.3, initial_state=c["initial_state"][0])
    o_m, s_m = _chunk_mutant(kind)(*args, 0.3, c["initial_state"][0], 16)
    assert not (np.allclose(o_m, o_r, atol=1e-9) and np.allclose(s_m, s_r, atol=1e-9))
