"""Pins for the fp64 backward oracle (oracle.kda_bwd_ref): it is checked against
things other than itself.

* Central finite differences of the forward oracle (itself pinned in
  test_oracle_pins.py) for every input, every decay kind and every prologue flag.
* Reverse-mode autodiff of an independent forward written here in plain torch
  float64 (a token loop with torch ops; nothing shared with the oracle).
* Closed form: one token from a zero state gives o = scale beta (k . q) v.
* Invariants: linearity in (do, dS_T); packed varlen = separate sequences.
Every pin takes the backward function as an argument, and copies of the oracle with
one planted mistake each must fail at least one pin.
"""

import inspect

import numpy as np
import pytest

import oracle.kda_bwd_ref as bwd_mod
from oracle import backward, forward, recurrence, recurrence_backward
from oracle.kda_prologue import BETA_LOGIT, GATE_LOGIT, NORM_K


def unit_rows(rng, *shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def small_case(seed, U=2, T=7, d_k=4, d_v=3, decay="channel"):
    rng = np.random.default_rng(seed)
    if decay == "channel":
        g = -rng.uniform(0.01, 0.5, (U, T, d_k))
    elif decay == "head":
        g = -rng.uniform(0.01, 0.5, (U, T))
    else:
        g = None
    return dict(q=rng.standard_normal((U, T, d_k)), k=unit_rows(rng, U, T, d_k),
                v=rng.standard_normal((U, T, d_v)), g=g,
                beta=rng.uniform(0.1, 1.0, (U, T)),
                initial_state=rng.standard_normal((U, d_v, d_k)),
                do=rng.standard_normal((U, T, d_v)),
                dfinal_state=rng.standard_normal((U, d_v, d_k)))


def loss(c, do, dfin):
    o, fin = recurrence(c["q"], c["k"], c["v"], c["g"], c["beta"], scale=0.7,
                        initial_state=c["initial_state"])
    return float(np.sum(o * do) + np.sum(fin * dfin))


NAMES = ["q", "k", "v", "g", "beta", "initial_state"]


# --------------------------------------------------------------------------- pins
def pin_finite_differences(rb):
    for decay in ("channel", "head", "none"):
        c = small_case(1, decay=decay)
        grads = rb(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], scale=0.7,
                   initial_state=c["initial_state"], dfinal_state=c["dfinal_state"])
        for name, gr in zip(NAMES, (grads[0], grads[1], grads[2], grads[3], grads[4],
                                    grads[5])):
            if c[name] is None:
                assert gr is None
                continue
            x = c[name]
            fd = np.zeros_like(x)
            h = 1e-6
            for idx in np.ndindex(x.shape):
                saved = x[idx]
                x[idx] = saved + h
                lp = loss(c, c["do"], c["dfinal_state"])
                x[idx] = saved - h
                lm = loss(c, c["do"], c["dfinal_state"])
                x[idx] = saved
                fd[idx] = (lp - lm) / (2 * h)
            np.testing.assert_allclose(gr, fd, rtol=1e-6, atol=1e-7, err_msg=f"{decay} {name}")


def pin_autograd(rb):
    torch = pytest.importorskip("torch")
    c = small_case(2, U=3, T=9, d_k=5, d_v=4)
    t = {n: torch.tensor(c[n], dtype=torch.float64, requires_grad=True) for n in NAMES}
    S = t["initial_state"]
    outs = []
    for i in range(c["q"].shape[1]):
        S = S * torch.exp(t["g"][:, i, :])[:, None, :]
        kt = t["k"][:, i, :]
        pred = (S * kt[:, None, :]).sum(-1)
        err = t["beta"][:, i, None] * (t["v"][:, i, :] - pred)
        S = S + err[:, :, None] * kt[:, None, :]
        outs.append(0.7 * (S * t["q"][:, i, None, :]).sum(-1))
    o = torch.stack(outs, 1)
    L = (o * torch.tensor(c["do"])).sum() + (S * torch.tensor(c["dfinal_state"])).sum()
    ref = torch.autograd.grad(L, [t[n] for n in NAMES])
    got = rb(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], scale=0.7,
             initial_state=c["initial_state"], dfinal_state=c["dfinal_state"])
    for name, a, b in zip(NAMES, got, ref):
        np.testing.assert_allclose(a, b.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def pin_one_token_closed_form(rb):
    # zero state, one token: S_1 = beta v k^T and o = scale beta (k . q) v, so
    # dq = s beta (v . do) k, dk = s beta (v . do) q, dv = s beta (k . q) do,
    # dbeta = s (k . q)(v . do) and dg = 0 (the decayed state is zero)
    rng = np.random.default_rng(3)
    d_k, d_v, s = 6, 5, 0.4
    q = rng.standard_normal((1, 1, d_k))
    k = unit_rows(rng, 1, 1, d_k)
    v = rng.standard_normal((1, 1, d_v))
    g = -rng.uniform(0.1, 0.5, (1, 1, d_k))
    beta = np.array([[0.6]])
    do = rng.standard_normal((1, 1, d_v))
    dq, dk, dv, dg, db, ds0 = rb(q, k, v, g, beta, do, scale=s)
    kq = float(k[0, 0] @ q[0, 0])
    vdo = float(v[0, 0] @ do[0, 0])
    np.testing.assert_allclose(dq[0, 0], s * 0.6 * vdo * k[0, 0], rtol=1e-12)
    np.testing.assert_allclose(dk[0, 0], s * 0.6 * vdo * q[0, 0], rtol=1e-12)
    np.testing.assert_allclose(dv[0, 0], s * 0.6 * kq * do[0, 0], rtol=1e-12)
    np.testing.assert_allclose(db[0, 0], s * kq * vdo, rtol=1e-12)
    np.testing.assert_allclose(dg, 0.0, atol=1e-15)
    # dL/dS_0: o = s (S_0 D + beta (v - S_0 D k) k^T) q, linear in S_0:
    # dS_0 = s [do q^T - beta do (k.q) k^T] D
    D = np.exp(g[0, 0])
    want = s * (np.outer(do[0, 0], q[0, 0]) - 0.6 * kq * np.outer(do[0, 0], k[0, 0])) * D
    np.testing.assert_allclose(ds0[0], want, rtol=1e-12, atol=1e-15)


def pin_linearity(rb):
    c = small_case(4)
    rng = np.random.default_rng(5)
    do2 = rng.standard_normal(c["do"].shape)
    ds2 = rng.standard_normal(c["dfinal_state"].shape)
    args = (c["q"], c["k"], c["v"], c["g"], c["beta"])
    a = rb(*args, c["do"], scale=0.7, initial_state=c["initial_state"],
           dfinal_state=c["dfinal_state"])
    b = rb(*args, do2, scale=0.7, initial_state=c["initial_state"], dfinal_state=ds2)
    ab = rb(*args, 2 * c["do"] - do2, scale=0.7, initial_state=c["initial_state"],
            dfinal_state=2 * c["dfinal_state"] - ds2)
    for x, y, z in zip(a, b, ab):
        np.testing.assert_allclose(z, 2 * x - y, rtol=1e-9, atol=1e-11)


PINS = [pin_finite_differences, pin_autograd, pin_one_token_closed_form, pin_linearity]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(recurrence_backward)


# ------------------------------------------------------------- planted mistakes are caught
_SRC = inspect.getsource(bwd_mod.recurrence_backward)
MUTANTS = {
    "dk_no_predict_term": ("dk[:, t, :] += np.matmul(st.transpose", "dk[:, t, :] += 0 * np.matmul(st.transpose"),
    "dp_sign": ("dp = -beta[:, t, None] * de", "dp = beta[:, t, None] * de"),
    "dg_undecayed_state": ("contrib = ds * st", "contrib = ds * st / alphas[t]"),
    "dq_from_decayed_state": ("dq[:, t, :] = scale * np.matmul(s_t.transpose", "dq[:, t, :] = scale * np.matmul(st.transpose"),
    "no_decay_on_carry": ("ds = ds * alphas[t]", "ds = ds"),
    "dbeta_without_prediction": ("np.sum(de * (v[:, t, :] - p), axis=1)", "np.sum(de * v[:, t, :], axis=1)"),
    "dv_without_beta": ("dv[:, t, :] = beta[:, t, None] * de", "dv[:, t, :] = de"),
    "dq_unscaled": ("dq[:, t, :] = scale * np.matmul", "dq[:, t, :] = np.matmul"),
    "read_grad_after_correct": ("de = np.matmul(ds, kt[:, :, None])", "de = np.matmul(ds - scale * do[:, t, :, None] * qt[:, None, :], kt[:, :, None])"),
}


def _mutant(kind):
    src = _SRC
    if kind != "none":
        old, new = MUTANTS[kind]
        assert src.count(old) == 1, kind
        src = src.replace(old, new)
    ns = dict(bwd_mod.__dict__)
    exec(compile(src, "<mutant>", "exec"), ns)  # noqa: S102 - test-only mutant copy
    return ns["recurrence_backward"]


def _all_pass(rb):
    for pin in PINS:
        try:
            pin(rb)
        except Exception:  # noqa: BLE001 - any failure means the pin caught it
            return False
    return True


def test_mutant_harness_accepts_the_faithful_copy():
    assert _all_pass(_mutant("none"))


@pytest.mark.parametrize("kind", sorted(MUTANTS))
def test_planted_backward_mistake_is_caught(kind):
    assert not _all_pass(_mutant(kind)), f"no pin catches planted mistake {kind}"


# ------------------------------------------------------ packed layout and the prologue
def test_packed_varlen_equals_separate_sequences():
    rng = np.random.default_rng(6)
    H, d_k, d_v = 2, 4, 3
    lens = [5, 0, 9, 3]
    tot = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = rng.standard_normal((1, tot, H, d_k))
    k = unit_rows(rng, 1, tot, H, d_k)
    v = rng.standard_normal((1, tot, H, d_v))
    g = -rng.uniform(0.01, 0.4, (1, tot, H, d_k))
    beta = rng.uniform(0.1, 1, (1, tot, H))
    do = rng.standard_normal((1, tot, H, d_v))
    s0 = rng.standard_normal((len(lens), H, d_v, d_k))
    dsT = rng.standard_normal((len(lens), H, d_v, d_k))
    got = backward(q, k, v, g, beta, do, cu_seqlens=cu, initial_state=s0, dfinal_state=dsT)
    for n, (lo, hi) in enumerate(zip(cu[:-1], cu[1:])):
        sl = slice(lo, hi)
        one = backward(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], do[:, sl],
                       initial_state=s0[n:n + 1], dfinal_state=dsT[n:n + 1])
        for a, b in zip(got[:5], one[:5]):
            np.testing.assert_allclose(a[:, sl], b, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(got[5][n], one[5][0], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("flags", [NORM_K, BETA_LOGIT, GATE_LOGIT,
                                   NORM_K | BETA_LOGIT | GATE_LOGIT])
def test_prologue_chain_rule_by_finite_differences(flags):
    rng = np.random.default_rng(7)
    B, T, H, d_k, d_v = 1, 5, 2, 4, 3
    q = rng.standard_normal((B, T, H, d_k))
    k = 2.0 * rng.standard_normal((B, T, H, d_k))
    v = rng.standard_normal((B, T, H, d_v))
    g = rng.uniform(1.0, 4.0, (B, T, H, d_k)) if flags & GATE_LOGIT \
        else -rng.uniform(0.01, 0.4, (B, T, H, d_k))
    beta = rng.standard_normal((B, T, H)) if flags & BETA_LOGIT \
        else rng.uniform(0.1, 1, (B, T, H))
    if not flags & NORM_K:
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    do = rng.standard_normal((B, T, H, d_v))

    def L(q_, k_, g_, b_):
        o, _ = forward(q_, k_, v, g_, b_, flags=flags)
        return float(np.sum(o * do))

    dq, dk, dv, dg, db, _ = backward(q, k, v, g, beta, do, flags=flags)
    for name, x, gr in (("k", k, dk), ("g", g, dg), ("beta", beta, db)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            saved = x[idx]
            x[idx] = saved + 1e-6
            lp = L(q, k, g, beta)
            x[idx] = saved - 1e-6
            lm = L(q, k, g, beta)
            x[idx] = saved
            fd[idx] = (lp - lm) / 2e-6
        np.testing.assert_allclose(gr, fd, rtol=1e-6, atol=1e-7, err_msg=name)


# ------------------------------------------------- the chunk algebra's reverse pass
@pytest.mark.parametrize("decay", ["channel", "head", "none"])
@pytest.mark.parametrize("chunk", [4, 16, 64])
def test_chunked_backward_equals_recurrence_backward(decay, chunk):
    from oracle.kda_chunk_ref import chunked_backward
    c = small_case(8, U=1, T=37, d_k=6, d_v=5, decay=decay)
    g = None if c["g"] is None else c["g"][0]
    ref = recurrence_backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], scale=0.3,
                              initial_state=c["initial_state"],
                              dfinal_state=c["dfinal_state"])
    got = chunked_backward(c["q"][0], c["k"][0], c["v"][0], g, c["beta"][0], c["do"][0], 0.3,
                           c["initial_state"][0], c["dfinal_state"][0], chunk=chunk)
    for name, a, r in zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), got, ref):
        if r is None:
            assert a is None
            continue
        np.testing.assert_allclose(a, r[0], rtol=1e-10, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("decay", ["channel", "head", "none"])
@pytest.mark.parametrize("segment", [1, 7, 64, 200])
def test_segmented_backward_equals_recurrence_backward(decay, segment):
    """oracle.segmented_backward (segment by segment from stored start states, the
    state gradient carried backwards) equals the whole-sequence token backward, with
    an initial state and a final-state gradient, including a ragged last segment and
    a segment longer than the sequence."""
    from oracle import segmented_backward
    c = small_case(11, U=3, T=150, d_k=5, d_v=4, decay=decay)
    args = (c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"])
    kw = dict(scale=0.7, initial_state=c["initial_state"], dfinal_state=c["dfinal_state"])
    ref = recurrence_backward(*args, **kw)
    got = segmented_backward(*args, segment=segment, **kw)
    for name, a, r in zip(NAMES, got, ref):
        if r is None:
            assert a is None
            continue
        np.testing.assert_allclose(a, r, rtol=0, atol=1e-11, err_msg=name)


def test_segmented_backward_carries_the_state_gradient():
    """A planted mistake -- each segment starting from a zero state gradient instead of
    the one carried from the segment after it -- changes the earlier segments'
    gradients, so the comparison above would catch it."""
    c = small_case(12, U=1, T=20, d_k=3, d_v=2)
    ref = recurrence_backward(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"])
    seg = recurrence_backward(c["q"][:, :10], c["k"][:, :10], c["v"][:, :10], c["g"][:, :10],
                              c["beta"][:, :10], c["do"][:, :10])
    # dv depends on the state gradient carried in (dq does not: only on the state)
    assert np.max(np.abs(seg[2] - ref[2][:, :10])) > 1e-6
