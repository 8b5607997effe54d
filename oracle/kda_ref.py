"""fp64 token-by-token KDA recurrence (test infrastructure; see the package docstring).

What is computed, per independent unit (one sequence, one head): the delta rule of
"Kimi Delta Attention Technical Deep Dive", section "From attention to recurrent
state" (the memory's prediction for the key, the write error against the value, a
rank-1 correction along the key scaled by the write strength beta), with KDA's
per-channel gate applied to the memory before the prediction, as the cycle of "Kimi
Delta Attention: The Linear Attention Behind Kimi K2 and Qwen3", section "How Kimi
Delta Attention works step by step", orders the steps (its prose and flowchart):

    S holds d_v rows and d_k columns and maps keys to values.
    For each token t, with alpha_t = exp(g_t) in (0, 1]^{d_k}:
      1. decay   : every key channel j (column j of S) is multiplied by alpha_t[j];
                   the flowchart writes this as a right product with Diag(alpha_t).
      2. predict : the decayed state's value for the current key, S k_t.
      3. error   : beta_t times (v_t minus that prediction).
      4. correct : add the outer product error * k_t^T to the decayed state.
      5. read    : o_t is the corrected state applied to the query scaled by
                   d_k^{-1/2} (the same scaling as softmax attention).

Readings taken where the pages leave a step open:

* The gate arrives as g = log(alpha) in fp32 (the workloads give "log alpha");
  alpha = exp(g) exactly in fp64 here.
* beta is one scalar per (token, head).
* ``scale`` is an argument defaulting to d_k^{-1/2}.
* Keys are L2-normalised by the caller; the oracle uses k as given.
* The "conceptual" gate order on the deep-dive page ("How the Kimi gate changes
  memory": predict from the undecayed state, then decay) is a different function
  and is not what is built; the step-by-step page's order (decay first) is.

The two simpler members of the same family (step-by-step page, "From quadratic
attention to fixed state: a brief history" and "DeltaNet, Gated DeltaNet, and KDA:
comparison table"; its FAQ "What's the concrete difference between Gated DeltaNet
and KDA?") use the same cycle with a different step 1:

* Gated DeltaNet: one scalar decay per token for the whole state (every entry of
  S is multiplied by alpha_t = exp(g_t)); g has no key-channel axis.
* DeltaNet: no decay at all (g is None).

Everything is computed in float64 on whatever values are passed in; callers pass
inputs already rounded to the kernel's input dtype so that input quantisation is
not counted as error.
"""

from __future__ import annotations

import numpy as np

from .kda_prologue import prologue


def default_scale(d_k: int) -> float:
    """Query scaling d_k^{-1/2} (step-by-step page, "read" step)."""
    return float(d_k) ** -0.5


def recurrence(q, k, v, g, beta, scale=None, initial_state=None):
    """Run the recurrence over T tokens for U independent units at once.

    Shapes (any float dtype; promoted to float64):
      q, k : [U, T, d_k]      v : [U, T, d_v]      beta : [U, T]
      g    : [U, T, d_k] (KDA, per key channel), [U, T] (Gated DeltaNet, one scalar
             per token) or None (DeltaNet, no decay)
      initial_state : [U, d_v, d_k] or None (zeros)
    Returns (o [U, T, d_v], final_state [U, d_v, d_k]), both float64.

    A 2-D call (no unit axis: q [T, d_k], beta [T], g [T, d_k] or [T], state
    [d_v, d_k]) is accepted and returns 2-D results.
    """
    squeeze = np.ndim(beta) == 1
    if squeeze:
        q, k, v, beta = (np.asarray(x)[None] for x in (q, k, v, beta))
        if g is not None:
            g = np.asarray(g)[None]
        if initial_state is not None:
            initial_state = np.asarray(initial_state)[None]
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    if g is not None:
        g = np.asarray(g, dtype=np.float64)
        if g.ndim not in (2, 3) or g.shape[:2] != beta.shape:
            raise ValueError("g must be [U, T, d_k], [U, T] or None")
    n_units, n_tok, d_k = k.shape
    d_v = v.shape[2]
    if scale is None:
        scale = default_scale(d_k)
    if initial_state is None:
        state = np.zeros((n_units, d_v, d_k))
    else:
        state = np.array(initial_state, dtype=np.float64, copy=True)

    out = np.empty((n_units, n_tok, d_v))
    for t in range(n_tok):
        key = k[:, t, :]                                       # [U, d_k]
        # 1. decay: each key channel (column of S) by its own alpha_t = exp(g_t)
        #    (KDA), the whole state by one scalar alpha_t (Gated DeltaNet), or
        #    nothing (DeltaNet)
        if g is not None and g.ndim == 3:
            state *= np.exp(g[:, t, :])[:, None, :]
        elif g is not None:
            state *= np.exp(g[:, t])[:, None, None]
        # 2. what the decayed memory returns for this key
        predicted = np.matmul(state, key[:, :, None])[:, :, 0]  # [U, d_v]
        # 3. error between the true value and the prediction, times beta_t
        err = beta[:, t, None] * (v[:, t, :] - predicted)      # [U, d_v]
        # 4. delta-rule write: rank-1 correction along the key direction
        state += err[:, :, None] * key[:, None, :]
        # 5. read with the scaled query
        out[:, t, :] = np.matmul(state, scale * q[:, t, :, None])[:, :, 0]
    if squeeze:
        return out[0], state[0]
    return out, state


def _sequence_bounds(cu_seqlens, B, T):
    if cu_seqlens is None:
        return [(b, b * T, (b + 1) * T) for b in range(B)]
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    return [(n, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def forward(q, k, v, g, beta, cu_seqlens=None, scale=None, initial_state=None,
            units=None, flags=0):
    """Whole-batch prefill in the packed ``[B, T, H, d]`` layout.

    q, k: [B, T, H, d_k]; v: [B, T, H, d_v]; beta: [B, T, H]; g: [B, T, H, d_k]
    (KDA), [B, T, H] (Gated DeltaNet) or None (DeltaNet).
    With ``cu_seqlens`` ([N+1], non-decreasing, cu[0] = 0, cu[N] = B*T) the B*T
    token rows are split into N sequences; otherwise each batch row b is one
    sequence of length T.  Every sequence starts from its own initial state
    (``initial_state`` [N, H, d_v, d_k], or zeros).

    ``units`` optionally restricts the work to a list of (n, h) pairs; outputs of
    other units are left as NaN and their final states as NaN.

    ``flags`` (``oracle.kda_prologue``) marks k, beta and g as raw projections that
    the prologue turns into unit keys, sigmoid(beta) and log(sigmoid(g)) first.

    Returns (o [B, T, H, d_v] float64, final_state [N, H, d_v, d_k] float64).
    """
    q = np.asarray(q)
    B, T, H, d_k = q.shape
    d_v = np.asarray(v).shape[3]
    tok = B * T
    if flags:
        k, g, beta = prologue(k, g, beta, flags)
    qf = np.asarray(q, dtype=np.float64).reshape(tok, H, d_k)
    kf = np.asarray(k, dtype=np.float64).reshape(tok, H, d_k)
    vf = np.asarray(v, dtype=np.float64).reshape(tok, H, d_v)
    gf = None if g is None else np.asarray(g, dtype=np.float64).reshape(tok, H, -1)
    per_channel = gf is not None and np.ndim(g) == 4
    bf = np.asarray(beta, dtype=np.float64).reshape(tok, H)
    seqs = _sequence_bounds(cu_seqlens, B, T)
    N = len(seqs)
    o = np.full((tok, H, d_v), np.nan)
    final = np.full((N, H, d_v, d_k), np.nan)
    wanted = None if units is None else {}
    if units is not None:
        for n, h in units:
            wanted.setdefault(int(n), []).append(int(h))
    for n, lo, hi in seqs:
        heads = list(range(H)) if wanted is None else sorted(wanted.get(n, []))
        if not heads:
            continue
        s0 = None
        if initial_state is not None:
            s0 = np.asarray(initial_state, dtype=np.float64)[n, heads]
        # unit axis = heads of this sequence
        o_seq, s_seq = recurrence(
            qf[lo:hi, heads].transpose(1, 0, 2), kf[lo:hi, heads].transpose(1, 0, 2),
            vf[lo:hi, heads].transpose(1, 0, 2),
            None if gf is None else (gf[lo:hi, heads].transpose(1, 0, 2) if per_channel
                                     else gf[lo:hi, heads, 0].T),
            bf[lo:hi, heads].T, scale=scale if scale is not None else default_scale(d_k),
            initial_state=s0)
        o[lo:hi, heads] = o_seq.transpose(1, 0, 2)
        final[n, heads] = s_seq
    return o.reshape(B, T, H, d_v), final


def decode_step(q, k, v, g, beta, state, scale=None, flags=0):
    """One decode step: one token per (sequence, head), state advanced by one.

    q, k: [N, H, d_k]; v: [N, H, d_v]; beta: [N, H]; state: [N, H, d_v, d_k];
    g: [N, H, d_k] (KDA), [N, H] (Gated DeltaNet) or None (DeltaNet).
    This is the recurrence with T = 1 (deep-dive page, "Decoding": one state
    update plus one query-state product per token).  The input ``state`` is not
    modified; the new state is returned.  ``flags`` as for ``forward``.
    Returns (o [N, H, d_v], new_state [N, H, d_v, d_k]) in float64.
    """
    q = np.asarray(q)
    N, H, d_k = q.shape
    d_v = np.asarray(v).shape[2]
    U = N * H
    if flags:
        k, g, beta = prologue(k, g, beta, flags)
    o, s = recurrence(
        np.asarray(q).reshape(U, 1, d_k), np.asarray(k).reshape(U, 1, d_k),
        np.asarray(v).reshape(U, 1, d_v),
        None if g is None else (np.asarray(g).reshape(U, 1, d_k) if np.ndim(g) == 3
                                else np.asarray(g).reshape(U, 1)),
        np.asarray(beta).reshape(U, 1), scale=scale,
        initial_state=np.asarray(state).reshape(U, d_v, d_k))
    return o.reshape(N, H, d_v), s.reshape(N, H, d_v, d_k)
