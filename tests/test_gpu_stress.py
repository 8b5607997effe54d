"""Seeded randomized GPU parity over launch geometries the fixed cases do not reach:
many short packed sequences (units far from a multiple of 8, few workgroups per unit,
one producer), odd head counts, mixed head dimensions, every decay kind and the
prologue.  Each case compares the whole output and final state with the fp64 oracle."""

import zlib

import numpy as np
import pytest
import torch

import gated_delta_rule_39_amd as kda
import kda_inputs as ki
from test_gpu_prefill import DEV, compare_full, run_gpu
from test_gpu_prologue import ALL, run_oracle

pytestmark = pytest.mark.gpu


def lengths_for(seed, n, hi):
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(0, hi + 1, size=n)]


CASES = [
    # name, N (or lengths), H, d_k, d_v, decay, prologue
    ("n20_h5_one_producer", 20, 700, 5, 128, 128, "channel", False),
    ("n40_h3", 40, 300, 3, 128, 128, "head", False),
    ("n12_h7_dk64", 12, 900, 7, 64, 128, "channel", True),
    ("n9_h11_dv64", 9, 1200, 11, 128, 64, "none", False),
    ("n3_h16_long", 3, 5000, 16, 128, 128, "channel", True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_random_varlen(case):
    name, n, hi, H, d_k, d_v, decay, pro = case
    lengths = lengths_for(zlib.crc32(name.encode()) % 1000, n, hi)
    units = n * H
    nc, np_, r = kda.prefill_coop_plan(torch.bfloat16, n, H, d_k, d_v)
    print(f"stress {name}: units {units}, tokens {sum(lengths)}, plan NC={nc} NP={np_} R={r}",
          flush=True)
    x = ki.make_prefill(H=H, d_k=d_k, d_v=d_v, dtype="bf16", lengths=lengths, init_state_std=0.02,
                        seed=81 + len(name), device=DEV, decay=decay, raw=pro)
    kw = ALL if pro else {}
    o_ref, s_ref = run_oracle(x, kw)
    paths = ["fused", "coop"] if nc > 0 else ["fused"]
    for path in paths:
        o, fs = run_gpu(x, path, **kw)
        compare_full(x, o, fs, o_ref, s_ref, f"{name} {path}")


@pytest.mark.parametrize("N,H,d", [(16, 16, 64), (300, 1, 128)])
def test_coop_not_applicable_falls_back_to_fused(N, H, d):
    """More units than the grid can hold as co-resident producer/consumer groups, and
    no lane plan (d = 64, or more than 256 sequences): the plan reports none, the
    workspace size is 0 and the fused kernel runs."""
    nc, _, _ = kda.prefill_coop_plan(torch.bfloat16, N, H, d, d)
    assert nc == 0 and kda.prefill_coop_lanes(torch.bfloat16, N, H, d, d) == 0
    assert kda.workspace_bytes(torch.bfloat16, N, N * 70, H, d, d) == 0
    x = ki.make_prefill(B=N, T=70, H=H, d_k=d, d_v=d, dtype="bf16", seed=90, device=DEV)
    o, fs = run_gpu(x, "fused")
    o_ref, s_ref = run_oracle(x, {})
    compare_full(x, o, fs, o_ref, s_ref, "fallback")
