"""GPU parity of the one-token decode step (kda_decode_step through the C ABI) against
the fp64 oracle."""

import numpy as np
import pytest
import torch

import gated_delta_rule_39_amd as kda
import kda_inputs as ki
from oracle import decode_step as oracle_decode
from parity import check, check_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run_and_compare(dtype, N, H, d_k, d_v, steps, seed):
    d = ki.make_decode(N=N, H=H, d_k=d_k, d_v=d_v, steps=steps, dtype=dtype, seed=seed,
                       device=DEV)
    state = d["state"].clone()
    ref_state = ki.to_f64(d["state"])
    for t in range(steps):
        o = kda.decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t], state)
        o_ref, ref_state = oracle_decode(ki.to_f64(d["q"][t]), ki.to_f64(d["k"][t]),
                                         ki.to_f64(d["v"][t]), ki.to_f64(d["g"][t]),
                                         ki.to_f64(d["beta"][t]), ref_state)
        torch.cuda.synchronize()
        check(dtype, ki.to_f64(o), o_ref, f"decode o step {t}")
        # GPU and oracle states each evolve on their own from the same initial state
        check(dtype, ki.to_f64(state), ref_state, f"decode state step {t}")


@pytest.mark.parametrize("d_k,d_v", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_decode_fp32_small(d_k, d_v):
    print(f"decode fp32 N=3 H=2 d_k={d_k} d_v={d_v}", flush=True)
    _run_and_compare("fp32", 3, 2, d_k, d_v, steps=6, seed=21)


@pytest.mark.parametrize("d_k,d_v", [(64, 64), (128, 128)])
def test_decode_bf16_small(d_k, d_v):
    print(f"decode bf16 N=5 H=3 d_k={d_k} d_v={d_v}", flush=True)
    _run_and_compare("bf16", 5, 3, d_k, d_v, steps=6, seed=22)


@pytest.mark.parametrize("gate", ["strong", "edge", "extreme", "spiky"])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_strong_decay(gate, dtype):
    """Strong per-channel decay over 70 steps: |g| of 0.6 .. 1.25 per token (the
    per-chunk sums of the prefill's strong-decay tests), 2 .. 4 ("extreme"), and near
    resets of single channels ("spiky").  Decode multiplies the state by e^g directly,
    so no decay is out of its range."""
    print(f"decode strong decay {gate} {dtype}", flush=True)
    d = ki.make_decode(N=6, H=4, d_k=128, d_v=128, steps=70, dtype=dtype, gate=gate, seed=26,
                       device=DEV)
    state = d["state"].clone()
    ref_state = ki.to_f64(d["state"])
    for t in range(d["steps"]):
        o = kda.decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t], state)
        o_ref, ref_state = oracle_decode(*(ki.to_f64(d[n][t]) for n in ("q", "k", "v", "g", "beta")),
                                         ref_state)
        torch.cuda.synchronize()
        check(dtype, ki.to_f64(o), o_ref, f"strong decode o step {t}")
    check(dtype, ki.to_f64(state), ref_state, "strong decode final state")


def test_decode_full_workload_sampled():
    """Decode at full size (N=256, H=32, d=128, bf16, 1000 in-place steps): every unit
    checked on its own for the first two steps, a seeded sample of 256 units at every
    step and their final states (units are independent, so the sample is exact)."""
    w = ki.DECODE
    print(f"decode full workload {w.name}", flush=True)
    d = ki.make_decode_workload(w, device=DEV)
    N, H, steps = w.N, w.H, w.steps
    rng = np.random.default_rng(55)
    S = 256
    flat = rng.choice(N * H, size=S, replace=False)
    sn, sh = flat // H, flat % H
    idx_n = torch.tensor(sn, device=DEV)
    idx_h = torch.tensor(sh, device=DEV)
    s0 = d["state"]
    ref_state = ki.to_f64(s0[idx_n, idx_h])[:, None]          # [64, 1, d_v, d_k]
    ref_full = ki.to_f64(s0)
    state = s0.clone()
    o_samp = torch.empty((steps, S, w.d_v), dtype=torch.bfloat16, device=DEV)
    for t in range(steps):
        o = kda.decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t], state)
        o_samp[t] = o[idx_n, idx_h]
        if t < 2:
            torch.cuda.synchronize()
            o_ref, ref_full = oracle_decode(*(ki.to_f64(d[x][t]) for x in ("q", "k", "v", "g",
                                                                            "beta")), ref_full)
            o_h = ki.to_f64(o)
            check("bf16", o_h, o_ref, f"decode full o step {t}")
            check_rows(o_h.reshape(N * H, -1), o_ref.reshape(N * H, -1),
                       f"decode full o step {t} per unit")
            check_rows(ki.to_f64(state).reshape(N * H, -1), ref_full.reshape(N * H, -1),
                       f"decode full state step {t} per unit")
    torch.cuda.synchronize()
    # oracle over the sampled units for all steps
    o_ref_all = np.empty((steps, S, w.d_v))
    sel = lambda x, t: ki.to_f64(d[x][t][idx_n, idx_h])[:, None]
    for t in range(steps):
        o_ref, ref_state = oracle_decode(sel("q", t), sel("k", t), sel("v", t), sel("g", t),
                                         sel("beta", t), ref_state)
        o_ref_all[t] = o_ref[:, 0]
    got = ki.to_f64(o_samp)
    check("bf16", got, o_ref_all, "decode sampled o (all steps)", windows=True,
          units=[(f"unit {u}", got[:, u], o_ref_all[:, u]) for u in range(S)])
    fin = ki.to_f64(state[idx_n, idx_h])
    check("bf16", fin, ref_state[:, 0], "decode sampled final state")
    check_rows(fin.reshape(S, -1), ref_state[:, 0].reshape(S, -1), "decode sampled final state")


def test_decode_deterministic_and_in_place():
    d = ki.make_decode(N=64, H=8, d_k=128, d_v=128, steps=3, seed=23, device=DEV)
    s1 = d["state"].clone()
    s2 = d["state"].clone()
    ptr = s1.data_ptr()
    for t in range(3):
        o1 = kda.decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t], s1)
        o2 = kda.decode_step(d["q"][t], d["k"][t], d["v"][t], d["g"][t], d["beta"][t], s2)
        assert torch.equal(o1, o2)
    assert torch.equal(s1, s2) and s1.data_ptr() == ptr
    assert not torch.equal(s1, d["state"])


def test_decode_identity_gate_leaves_state_unchanged():
    # alpha = 1 (g = 0), beta = 0: the state must come back bit-for-bit
    d = ki.make_decode(N=4, H=2, d_k=128, d_v=128, steps=1, seed=24, device=DEV)
    state = d["state"].clone()
    o = kda.decode_step(d["q"][0], d["k"][0], d["v"][0], torch.zeros_like(d["g"][0]),
                        torch.zeros_like(d["beta"][0]), state)
    torch.cuda.synchronize()
    assert torch.equal(state, d["state"])
    ref = np.einsum("nhvk,nhk->nhv", ki.to_f64(d["state"]), ki.to_f64(d["q"][0])) * 128 ** -0.5
    check("bf16", ki.to_f64(o), ref, "identity-gate read")


def test_decode_empty_batch_is_noop():
    z = torch.zeros((0, 2, 64), device=DEV)
    o = kda.decode_step(z, z, z, z, torch.zeros((0, 2), device=DEV),
                        torch.zeros((0, 2, 64, 64), device=DEV))
    assert o.shape == (0, 2, 64)
