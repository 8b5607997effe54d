"""Seeded randomized GPU parity of the backward over launch geometries the fixed cases do
not reach: many short packed sequences (units far from a multiple of 8), unit counts
where the forward sweep falls back to the fused kernel, odd head counts, d_k or d_v = 64,
every decay kind and the prologue.  Each case compares every gradient with the fp64
oracle (bf16 bar of tests/parity.py)."""

import zlib

import numpy as np
import pytest
import torch

import gated_delta_rule_39_amd as kda
import kda_inputs as ki
from test_gpu_backward import DEV, compare, grads_in, run_both

pytestmark = pytest.mark.gpu


def lengths_for(seed, n, hi):
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(0, hi + 1, size=n)]


CASES = [
    # name, sequences, max length, H, d_k, d_v, decay, prologue flags
    ("n20_h5_fused_sweep", 20, 260, 5, 128, 128, "channel", 0),
    ("n6_h3_coop_sweep", 6, 400, 3, 128, 128, "head", 7),
    ("n9_h11_dk64", 9, 300, 11, 64, 128, "channel", 1),
    ("n7_h7_dv64", 7, 330, 7, 128, 64, "none", 2),
    ("n30_h9_short", 30, 90, 9, 64, 64, "channel", 4),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_random_varlen(case):
    name, n, hi, H, d_k, d_v, decay, flags = case
    lengths = lengths_for(zlib.crc32(name.encode()) % 1000, n, hi)
    nc, np_, r = kda.prefill_coop_plan(torch.bfloat16, n, H, d_k, d_v)
    print(f"backward stress {name}: units {n * H}, tokens {sum(lengths)}, "
          f"coop plan NC={nc} NP={np_} R={r}", flush=True)
    x = ki.make_prefill(H=H, d_k=d_k, d_v=d_v, dtype="bf16", lengths=lengths,
                        init_state_std=0.02, seed=91 + len(name), device=DEV, decay=decay,
                        raw=flags != 0)
    if flags and not flags & 1:
        x["k"] = (x["k"].float() / x["k"].float().norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    if flags and not flags & 2:
        x["beta"] = torch.sigmoid(x["beta"])
    if flags and not flags & 4 and x["g"] is not None:
        x["g"] = -torch.nn.functional.softplus(-x["g"])
    do, ds = grads_in(x, 191 + len(name))
    got, ref = run_both(x, do, ds, flags)
    compare(x, got, ref, name)


def test_backward_is_deterministic():
    """Two calls on the same inputs give bit-identical gradients (no atomics, fixed
    reduction orders)."""
    x = ki.make_prefill(H=4, d_k=128, d_v=128, dtype="bf16", lengths=[200, 77], seed=97,
                        init_state_std=0.02, device=DEV)
    do, ds = grads_in(x, 197)
    a = kda.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, cu_seqlens=x["cu_seqlens"],
                     initial_state=x["initial_state"], dfinal_state=ds)
    b = kda.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, cu_seqlens=x["cu_seqlens"],
                     initial_state=x["initial_state"], dfinal_state=ds)
    torch.cuda.synchronize()
    for u, w in zip(a, b):
        assert torch.equal(u, w)
