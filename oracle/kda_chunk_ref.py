"""fp64 chunkwise form of the KDA recurrence (test infrastructure).

The pages say only that training and prefill run the recurrence "chunkwise": a
block of tokens is processed from a boundary state, and the state at the end of
the block is the initial condition of the next block ("Kimi Delta Attention
Technical Deep Dive", "Systems and implementation tradeoffs" -> "Training"; the
step-by-step page's remark that production kernels process the sequence in
blocks).  The per-block algebra below is derived here from the token recurrence
of oracle.kda_ref; it is exact (up to rounding) for any chunk size C, and the
tests check it against the recurrence for several C.

For one chunk of rows r = 1..n (n <= C) starting from state S (d_v x d_k):

  G_r   = g_1 + ... + g_r                    inclusive prefix per key channel
  Kg_r  = k_r * exp(G_r)                     keys decayed to the chunk start
  Ki_r  = k_r * exp(-G_r)                    keys "un-decayed" (inverse factor)
  Qg_r  = scale * q_r * exp(G_r)
  Kh_r  = k_r * exp(G_n - G_r)               keys decayed to the chunk end
  A     = strictly lower part of diag(beta) Kg Ki^T      (n x n)
  Tm    = (I + A)^{-1} diag(beta)
  E     = Tm (V - Kg S^T)                    row r equals the token error e_r
  M     = lower part (diagonal included) of Qg Ki^T
  O     = Qg S^T + M E
  S'    = S Diag(exp(G_n)) + E^T Kh

Why: unrolling the recurrence inside the chunk gives the decayed state seen by
row r as S Diag(e^{G_r}) + sum_{c<r} e_c (k_c * e^{G_r - G_c})^T, so
e_r = beta_r (v_r - Kg_r S^T - sum_{c<r} (Kg_r . Ki_c) e_c), i.e. (I + A) E =
diag(beta)(V - Kg S^T); the output and end state follow the same way with the
diagonal term included.  Rows of S (the d_v index) never mix.
"""

from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunked(q, k, v, g, beta, scale, initial_state=None, chunk=64):
    """Chunkwise evaluation for one unit.

    q, k: [T, d_k]; v: [T, d_v]; beta: [T]; initial_state [d_v, d_k] or None;
    g: [T, d_k] (per key channel), [T] (one scalar per token: every channel decays
    alike, so G, e^{G} are the same for all channels) or None (no decay, G = 0).
    Returns (o [T, d_v], final_state [d_v, d_k]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if g is None:
        g = np.zeros(k.shape)
    g = np.asarray(g, dtype=np.float64)
    if g.ndim == 1:
        g = np.repeat(g[:, None], k.shape[1], axis=1)
    beta = np.asarray(beta, dtype=np.float64)
    n_tok, d_k = k.shape
    d_v = v.shape[1]
    S = (np.zeros((d_v, d_k)) if initial_state is None
         else np.array(initial_state, dtype=np.float64, copy=True))
    o = np.empty((n_tok, d_v))
    for start in range(0, n_tok, chunk):
        rows = slice(start, min(start + chunk, n_tok))
        n = rows.stop - rows.start
        G = np.cumsum(g[rows], axis=0)                    # inclusive prefix
        Kg = k[rows] * np.exp(G)
        Ki = k[rows] * np.exp(-G)
        Qg = scale * q[rows] * np.exp(G)
        Kh = k[rows] * np.exp(G[-1] - G)
        b = beta[rows]
        A = np.tril(b[:, None] * (Kg @ Ki.T), k=-1)
        Tm = solve_triangular(np.eye(n) + A, np.diag(b), lower=True,
                              unit_diagonal=True)
        E = Tm @ (v[rows] - Kg @ S.T)
        M = np.tril(Qg @ Ki.T)
        o[rows] = Qg @ S.T + M @ E
        S = S * np.exp(G[-1])[None, :] + E.T @ Kh
    return o, S


def chunked_backward(q, k, v, g, beta, do, scale, initial_state=None, dfinal_state=None,
                     chunk=64):
    """Gradients of :func:`chunked` for one unit, through the same chunk algebra.

    This is the reverse of the chunk form written with H = S^T (d_k x d_v) and the
    WY factors W = Tm Kg = X diag(beta) Kg and U = Tm V = X diag(beta) V
    (X = (I + A)^{-1}):

      E = U - W H,   O = Qg H + M E,   H' = Diag(e^{G_n}) H + Kh^T E.

    Reverse step for one chunk, given dO and dH' (the gradient of the state after it):

      dE  = Kh dH' + M^T dO                 dH  = Diag(e^{G_n}) dH' + Qg^T dO - W^T dE
      dQg = dO H^T + dM Ki,  dM = lower(dO E^T)
      dW  = -dE H^T     dKh = E dH'^T     d e^{G_n}_j = sum_v dH'[j, v] H[j, v]
      dX  = dE (beta V)^T + dW (beta Kg)^T            dA = -strict_lower(X^T dX X^T)
      d(beta V) = X^T dE     d(beta Kg) = X^T dW + dA Ki     dKi = dA^T (beta Kg) + dM^T Qg
    then through Kg = k e^G, Ki = k e^{-G}, Qg = scale q e^G, Kh = k e^{G_n - G} and
    G = prefix sums of g.  Exact (up to rounding) for any chunk size; the tests check
    it against oracle.kda_bwd_ref.  Returns (dq, dk, dv, dg, dbeta, dS0) like
    :func:`oracle.kda_bwd_ref.recurrence_backward` for one unit (2-D arrays).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    g_kind = None if g is None else np.ndim(g)
    if g is None:
        g = np.zeros(k.shape)
    g = np.asarray(g, dtype=np.float64)
    if g.ndim == 1:
        g = np.repeat(g[:, None], k.shape[1], axis=1)
    beta = np.asarray(beta, dtype=np.float64)
    n_tok, d_k = k.shape
    d_v = v.shape[1]
    H = (np.zeros((d_k, d_v)) if initial_state is None
         else np.array(initial_state, dtype=np.float64).T.copy())
    starts = list(range(0, n_tok, chunk))
    states = []
    for start in starts:                     # forward: the state at each chunk start
        rows = slice(start, min(start + chunk, n_tok))
        n = rows.stop - rows.start
        G = np.cumsum(g[rows], axis=0)
        Kg, Ki = k[rows] * np.exp(G), k[rows] * np.exp(-G)
        Kh = k[rows] * np.exp(G[-1] - G)
        b = beta[rows]
        X = np.linalg.inv(np.eye(n) + np.tril(b[:, None] * (Kg @ Ki.T), k=-1))
        E = X @ (b[:, None] * v[rows]) - X @ (b[:, None] * Kg) @ H
        states.append(H)
        H = np.exp(G[-1])[:, None] * H + Kh.T @ E
    dq, dk = np.zeros(q.shape), np.zeros(k.shape)
    dv, dgm = np.zeros(v.shape), np.zeros(k.shape)
    dbeta = np.zeros(n_tok)
    dH = (np.zeros((d_k, d_v)) if dfinal_state is None
          else np.array(dfinal_state, dtype=np.float64).T.copy())
    for start, H in zip(reversed(starts), reversed(states)):
        rows = slice(start, min(start + chunk, n_tok))
        n = rows.stop - rows.start
        G = np.cumsum(g[rows], axis=0)
        eG, Gn = np.exp(G), G[-1]
        Kg, Ki = k[rows] * eG, k[rows] * np.exp(-G)
        Qg = scale * q[rows] * eG
        Kh = k[rows] * np.exp(Gn - G)
        D = np.exp(Gn)
        b = beta[rows]
        Bk, Bv = b[:, None] * Kg, b[:, None] * v[rows]
        X = np.linalg.inv(np.eye(n) + np.tril(Bk @ Ki.T, k=-1))
        W, U = X @ Bk, X @ Bv
        M = np.tril(Qg @ Ki.T)
        E = U - W @ H
        dO = do[rows]
        dE = Kh @ dH + M.T @ dO
        dQg = dO @ H.T
        dM = np.tril(dO @ E.T)
        dW = -dE @ H.T
        dKh = E @ dH.T
        dD = np.sum(dH * H, axis=1)
        dX = dE @ Bv.T + dW @ Bk.T
        dA = -np.tril(X.T @ dX @ X.T, k=-1)
        dBv = X.T @ dE
        dBk = X.T @ dW + dA @ Ki
        dKi = dA.T @ Bk + dM.T @ Qg
        dQg = dQg + dM @ Ki
        dH_prev = D[:, None] * dH + Qg.T @ dO - W.T @ dE
        dv[rows] = b[:, None] * dBv
        dbeta[rows] = np.sum(dBv * v[rows], axis=1) + np.sum(dBk * Kg, axis=1)
        dKg = b[:, None] * dBk
        dk[rows] = dKg * eG + dKi / eG + dKh * np.exp(Gn - G)
        dq[rows] = scale * dQg * eG
        dG = dKg * Kg + dQg * Qg - dKi * Ki - dKh * Kh
        dGn = np.sum(dKh * Kh, axis=0) + dD * D
        # G_r = g_1 + ... + g_r and G_n = G_last: dg_s = sum_{r >= s} dG_r + dG_n
        dgm[rows] = np.cumsum(dG[::-1], axis=0)[::-1] + dGn[None, :]
        dH = dH_prev
    if g_kind is None:
        dg = None
    elif g_kind == 1:
        dg = dgm.sum(axis=1)
    else:
        dg = dgm
    return dq, dk, dv, dg, dbeta, dH.T.copy()
