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
