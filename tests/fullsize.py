"""The fp64 oracle over every (sequence, head) unit of a full-size workload, fanned
over the host cores with oracle.pool (test infrastructure for the GPU parity tests).
"""

import numpy as np

import kda_inputs as ki


def seq_bounds(x):
    if x["cu_seqlens"] is None:
        return [(n, n * x["T"], (n + 1) * x["T"]) for n in range(x["B"])]
    cu = x["cu_seqlens"].tolist()
    return [(n, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def oracle_all_units(x, procs=16):
    """(o [B*T, H, d_v], final_state [N, H, d_v, d_k]) in fp64 for every unit of the
    prefill batch ``x`` (a kda_inputs dict), sequence by sequence."""
    from oracle.pool import host_cores, recurrence_parallel
    procs = max(1, min(procs, host_cores()))
    H, d_k, d_v = x["H"], x["d_k"], x["d_v"]
    rows = x["q"].shape[0] * x["q"].shape[1]
    o_ref = np.zeros((rows, H, d_v))
    s_ref = np.zeros((x["N"], H, d_v, d_k))
    s0_all = None if x["initial_state"] is None else ki.to_f64(x["initial_state"])
    for n, lo, hi in seq_bounds(x):
        s0 = None if s0_all is None else s0_all[n]
        if hi == lo:
            if s0 is not None:
                s_ref[n] = s0
            continue

        def units(t):   # [rows, H, d] -> this sequence's [H, T_n, d]
            return np.ascontiguousarray(ki.to_f64(t.reshape(rows, H, -1)[lo:hi]).transpose(1, 0, 2))

        q, k, v = units(x["q"]), units(x["k"]), units(x["v"])
        g = None
        if x["g"] is not None:
            g = units(x["g"]) if x["g"].dim() == 4 else units(x["g"][..., None])[..., 0]
        beta = np.ascontiguousarray(ki.to_f64(x["beta"].reshape(rows, H)[lo:hi]).T)
        o, s, _ = recurrence_parallel(q, k, v, g, beta, initial_state=s0, processes=procs)
        o_ref[lo:hi] = o.transpose(1, 0, 2)
        s_ref[n] = s
    return o_ref, s_ref
