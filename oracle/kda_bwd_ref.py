"""fp64 reverse-mode (backward) pass of the KDA recurrence (test infrastructure; see
the package docstring).

The pages tie chunkwise scans to training ("Kimi Delta Attention Technical Deep
Dive", "Systems and implementation tradeoffs" -> "Training") but print no gradient
formulas.  What is computed here is the plain definition: the exact gradient of the
forward recurrence of :mod:`oracle.kda_ref` (step-by-step page, "How Kimi Delta
Attention works step by step") with respect to every input, for a scalar loss L whose
gradients with respect to the outputs o_t and to the final state are given.

Forward step t (S has d_v rows and d_k columns):

    S~  = S_{t-1} Diag(alpha_t)         alpha_t = exp(g_t)
    p   = S~ k_t
    e   = beta_t (v_t - p)
    S_t = S~ + e k_t^T
    o_t = S_t (scale q_t)

Reverse step t, carrying dS = dL/dS_t (starting from the final-state gradient), is
the chain rule taken through those five lines in reverse order:

    read     dS  += scale do_t q_t^T           dq_t = scale S_t^T do_t
    correct  de   = dS k_t                     dk_t = dS^T e        dS~ = dS
    error    dbeta_t = de . (v_t - p)          dv_t = beta_t de     dp = -beta_t de
    predict  dS~ += dp k_t^T                   dk_t += S~^T dp
    decay    dg_t[j] = sum_i dS~[i, j] S~[i, j]        (d alpha / d g = alpha)
             dS_{t-1} = dS~ Diag(alpha_t)

For the one-scalar decay (Gated DeltaNet) dg_t sums that over j as well; without a
decay (DeltaNet) there is no dg.  The states S_{t-1} are those of the forward pass,
kept from a first forward sweep (the plainest reading; no recomputation scheme).

With prologue ``flags`` the gradients are with respect to the raw inputs: the chain
rule continues through the prologue of :mod:`oracle.kda_prologue`.
"""

from __future__ import annotations

import numpy as np

from .kda_prologue import BETA_LOGIT, EPS, GATE_LOGIT, NORM_K
from .kda_ref import _sequence_bounds, default_scale


def recurrence_backward(q, k, v, g, beta, do, scale=None, initial_state=None,
                        dfinal_state=None):
    """Gradients of the recurrence over T tokens for U units at once.

    Shapes as :func:`oracle.kda_ref.recurrence` ([U, T, ...]; g [U, T, d_k], [U, T]
    or None), plus do [U, T, d_v] and dfinal_state [U, d_v, d_k] or None (zero).
    Returns (dq, dk, dv, dg, dbeta, dinitial_state) in float64; dg is None when g is.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    if g is not None:
        g = np.asarray(g, dtype=np.float64)
    n_units, n_tok, d_k = k.shape
    d_v = v.shape[2]
    if scale is None:
        scale = default_scale(d_k)

    # forward sweep, keeping alpha_t, S~_t, p_t and S_t
    state = (np.zeros((n_units, d_v, d_k)) if initial_state is None
             else np.array(initial_state, dtype=np.float64, copy=True))
    alphas, decayed, preds, after = [], [], [], []
    for t in range(n_tok):
        if g is None:
            alpha = np.ones((n_units, 1, 1))
        elif g.ndim == 3:
            alpha = np.exp(g[:, t, :])[:, None, :]
        else:
            alpha = np.exp(g[:, t])[:, None, None]
        st = state * alpha
        p = np.matmul(st, k[:, t, :, None])[:, :, 0]
        e = beta[:, t, None] * (v[:, t, :] - p)
        state = st + e[:, :, None] * k[:, t, None, :]
        alphas.append(alpha)
        decayed.append(st)
        preds.append(p)
        after.append(state)

    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dbeta = np.zeros_like(beta)
    dg = None if g is None else np.zeros_like(g)
    ds = (np.zeros((n_units, d_v, d_k)) if dfinal_state is None
          else np.array(dfinal_state, dtype=np.float64, copy=True))
    for t in range(n_tok - 1, -1, -1):
        kt, qt = k[:, t, :], q[:, t, :]
        st, p, s_t = decayed[t], preds[t], after[t]
        # read: o_t = scale S_t q_t
        ds = ds + scale * do[:, t, :, None] * qt[:, None, :]
        dq[:, t, :] = scale * np.matmul(s_t.transpose(0, 2, 1), do[:, t, :, None])[:, :, 0]
        # correct: S_t = S~ + e k^T
        e = beta[:, t, None] * (v[:, t, :] - p)
        de = np.matmul(ds, kt[:, :, None])[:, :, 0]
        dk[:, t, :] = np.matmul(ds.transpose(0, 2, 1), e[:, :, None])[:, :, 0]
        # error: e = beta (v - p)
        dbeta[:, t] = np.sum(de * (v[:, t, :] - p), axis=1)
        dv[:, t, :] = beta[:, t, None] * de
        dp = -beta[:, t, None] * de
        # predict: p = S~ k
        ds = ds + dp[:, :, None] * kt[:, None, :]
        dk[:, t, :] += np.matmul(st.transpose(0, 2, 1), dp[:, :, None])[:, :, 0]
        # decay: S~ = S_{t-1} Diag(alpha)
        if g is not None:
            contrib = ds * st
            if g.ndim == 3:
                dg[:, t, :] = contrib.sum(axis=1)
            else:
                dg[:, t] = contrib.sum(axis=(1, 2))
        ds = ds * alphas[t]
    return dq, dk, dv, dg, dbeta, ds


def _prologue_backward(k_raw, g_raw, beta_raw, flags, dk, dg, dbeta):
    """Chain rule through the prologue: gradients of the normalised key, the log-decay
    and the write strength back to the raw projections."""
    if flags & NORM_K:
        kr = np.asarray(k_raw, dtype=np.float64)
        nrm = np.sqrt(np.sum(kr * kr, axis=-1, keepdims=True) + EPS)
        # khat_i = k_i / n with n^2 = |k|^2 + eps:  d khat_i / d k_j = delta_ij / n - k_i k_j / n^3
        dk = dk / nrm - kr * np.sum(kr * dk, axis=-1, keepdims=True) / nrm ** 3
    if flags & BETA_LOGIT:
        b = 1.0 / (1.0 + np.exp(-np.asarray(beta_raw, dtype=np.float64)))
        dbeta = dbeta * b * (1.0 - b)
    if (flags & GATE_LOGIT) and dg is not None:
        # g = log sigmoid(a): dg/da = 1 - sigmoid(a) = sigmoid(-a)
        a = np.asarray(g_raw, dtype=np.float64)
        dg = dg / (1.0 + np.exp(a))
    return dk, dg, dbeta


def backward(q, k, v, g, beta, do, cu_seqlens=None, scale=None, initial_state=None,
             dfinal_state=None, flags=0):
    """Gradients of the whole-batch prefill in the packed ``[B, T, H, d]`` layout.

    Inputs as :func:`oracle.kda_ref.forward`, plus do [B, T, H, d_v] (gradient of the
    output) and dfinal_state [N, H, d_v, d_k] or None (zero).  Token rows outside
    every sequence get zero gradients.
    Returns (dq, dk, dv, dg, dbeta, dinitial_state), float64, in the input layouts
    (dg None when g is None; dinitial_state [N, H, d_v, d_k]).
    """
    from .kda_prologue import prologue

    q = np.asarray(q)
    B, T, H, d_k = q.shape
    d_v = np.asarray(v).shape[3]
    tok = B * T
    k_raw, g_raw, b_raw = k, g, beta
    if flags:
        k, g, beta = prologue(k, g, beta, flags)
    per_channel = g is not None and np.ndim(g) == 4
    qf = np.asarray(q, dtype=np.float64).reshape(tok, H, d_k)
    kf = np.asarray(k, dtype=np.float64).reshape(tok, H, d_k)
    vf = np.asarray(v, dtype=np.float64).reshape(tok, H, d_v)
    dof = np.asarray(do, dtype=np.float64).reshape(tok, H, d_v)
    bf = np.asarray(beta, dtype=np.float64).reshape(tok, H)
    gf = None if g is None else np.asarray(g, dtype=np.float64).reshape(
        tok, H, d_k if per_channel else 1)
    seqs = _sequence_bounds(cu_seqlens, B, T)
    N = len(seqs)
    dq = np.zeros((tok, H, d_k))
    dk = np.zeros((tok, H, d_k))
    dv = np.zeros((tok, H, d_v))
    dbeta = np.zeros((tok, H))
    dg = None if g is None else np.zeros(gf.shape)
    ds0 = np.zeros((N, H, d_v, d_k))
    if scale is None:
        scale = default_scale(d_k)
    for n, lo, hi in seqs:
        s0 = None if initial_state is None else np.asarray(initial_state)[n]
        dsT = None if dfinal_state is None else np.asarray(dfinal_state)[n]
        gseq = None
        if gf is not None:
            gseq = (gf[lo:hi].transpose(1, 0, 2) if per_channel else gf[lo:hi, :, 0].T)
        r = recurrence_backward(
            qf[lo:hi].transpose(1, 0, 2), kf[lo:hi].transpose(1, 0, 2),
            vf[lo:hi].transpose(1, 0, 2), gseq, bf[lo:hi].T, dof[lo:hi].transpose(1, 0, 2),
            scale=scale, initial_state=s0, dfinal_state=dsT)
        dq[lo:hi] = r[0].transpose(1, 0, 2)
        dk[lo:hi] = r[1].transpose(1, 0, 2)
        dv[lo:hi] = r[2].transpose(1, 0, 2)
        if dg is not None:
            dg[lo:hi] = r[3].transpose(1, 0, 2) if per_channel else r[3].T[:, :, None]
        dbeta[lo:hi] = r[4].T
        ds0[n] = r[5]
    dk = dk.reshape(B, T, H, d_k)
    dbeta = dbeta.reshape(B, T, H)
    if dg is not None:
        dg = dg.reshape((B, T, H, d_k) if per_channel else (B, T, H))
    if flags:
        dk, dg, dbeta = _prologue_backward(k_raw, g_raw, b_raw, flags, dk, dg, dbeta)
    return (dq.reshape(B, T, H, d_k), dk, dv.reshape(B, T, H, d_v), dg, dbeta, ds0)


def segmented_backward(q, k, v, g, beta, do, segment=64, scale=None, initial_state=None,
                       dfinal_state=None):
    """:func:`recurrence_backward` over a long sequence, one segment of ``segment``
    tokens at a time, so that no more than one segment's token states are held.

    The state at a segment's start is all the later tokens depend on ("Kimi Delta
    Attention Technical Deep Dive", "Systems and implementation tradeoffs" ->
    "Training": the state at a chunk boundary is the next chunk's initial condition).
    So one forward pass keeps the state at every segment start; then, from the last
    segment back to the first, the exact token backward of the segment runs from its
    stored start state, with the state gradient carried in from the segment after it
    (the final-state gradient for the last), and hands the gradient of its start
    state to the segment before.  Same shapes and returns as
    :func:`recurrence_backward`.
    """
    from .kda_ref import recurrence
    q, k, v, beta, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, beta, do))
    g = None if g is None else np.asarray(g, dtype=np.float64)
    U, T, d_k = k.shape
    d_v = v.shape[2]
    starts = list(range(0, T, segment)) or [0]
    states = []
    s = (np.zeros((U, d_v, d_k)) if initial_state is None
         else np.array(initial_state, dtype=np.float64, copy=True))
    for t0 in starts:
        states.append(s)
        sl = slice(t0, t0 + segment)
        _, s = recurrence(q[:, sl], k[:, sl], v[:, sl], None if g is None else g[:, sl],
                          beta[:, sl], scale=scale, initial_state=s)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dg = None if g is None else np.zeros_like(g)
    dbeta = np.zeros_like(beta)
    ds = None if dfinal_state is None else np.asarray(dfinal_state, dtype=np.float64)
    for t0, s0 in zip(reversed(starts), reversed(states)):
        sl = slice(t0, t0 + segment)
        r = recurrence_backward(q[:, sl], k[:, sl], v[:, sl], None if g is None else g[:, sl],
                                beta[:, sl], do[:, sl], scale=scale, initial_state=s0,
                                dfinal_state=ds)
        dq[:, sl], dk[:, sl], dv[:, sl] = r[0], r[1], r[2]
        if dg is not None:
            dg[:, sl] = r[3]
        dbeta[:, sl] = r[4]
        ds = r[5]
    if ds is None:
        ds = np.zeros((U, d_v, d_k))
    return dq, dk, dv, dg, dbeta, ds
