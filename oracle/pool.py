"""Fan independent (sequence, head) units of the fp64 recurrence out over host cores.

Test infrastructure, used by the CPU-baseline leg of the benchmark.  Units are
independent (each head of each sequence has its own state), so splitting them
over processes changes nothing in what is computed.
"""

from __future__ import annotations

import os
import multiprocessing as mp

import numpy as np

from .kda_ref import recurrence


def _run(args):
    q, k, v, g, beta, scale, s0 = args
    # one thread per worker, so "cores used" is the worker count
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        return recurrence(q, k, v, g, beta, scale=scale, initial_state=s0)


def host_cores() -> int:
    """Cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def recurrence_parallel(q, k, v, g, beta, scale=None, initial_state=None,
                        processes=None):
    """Same contract as :func:`oracle.kda_ref.recurrence` (unit axis first), with
    the unit axis split into ``processes`` slices run in worker processes.

    Returns (o, final_state, processes_used).
    """
    U = np.asarray(beta).shape[0]
    procs = max(1, min(processes or host_cores(), U))
    bounds = np.linspace(0, U, procs + 1).astype(int)
    jobs = []
    for i in range(procs):
        sl = slice(bounds[i], bounds[i + 1])
        s0 = None if initial_state is None else np.asarray(initial_state)[sl]
        gs = None if g is None else np.asarray(g)[sl]   # no decay (DeltaNet): g is None
        jobs.append((np.asarray(q)[sl], np.asarray(k)[sl], np.asarray(v)[sl],
                     gs, np.asarray(beta)[sl], scale, s0))
    if procs == 1:
        outs = [_run(jobs[0])]
    else:
        ctx = mp.get_context("fork")
        with ctx.Pool(procs) as pool:
            outs = pool.map(_run, jobs)
    o = np.concatenate([x[0] for x in outs], axis=0)
    s = np.concatenate([x[1] for x in outs], axis=0)
    return o, s, procs
