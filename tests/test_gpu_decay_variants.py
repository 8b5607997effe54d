"""GPU parity of the two other decay kinds the method's family has, against the fp64
oracle: Gated DeltaNet (one scalar decay per token and head, g [.., H]) and DeltaNet
(no decay, g None).  Comparison table of DeltaNet, Gated DeltaNet and KDA on the
step-by-step page ("DeltaNet, Gated DeltaNet, and KDA: comparison table"): the three
differ only in the forget gate applied before the delta-rule write."""

import numpy as np
import pytest
import torch

import gated_delta_rule_39_amd as kda
import kda_inputs as ki
from oracle import decode_step as oracle_decode
from parity import check
from test_gpu_prefill import DEV, PATHS, _every_unit, compare_full, run_gpu, run_oracle

pytestmark = pytest.mark.gpu
DECAYS = ["head", "none"]


@pytest.mark.parametrize("decay", DECAYS)
@pytest.mark.parametrize("dtype,d_k,d_v,path", [
    ("fp32", 64, 64, "fused"), ("fp32", 128, 128, "fused"), ("bf16", 128, 128, "fused"),
    ("bf16", 64, 128, "fused"), ("bf16", 128, 128, "coop"), ("bf16", 64, 64, "coop")])
def test_varlen_ragged(decay, dtype, d_k, d_v, path):
    """Packed sequences (empty, sub-chunk, exact-chunk, ragged), nonzero initial state."""
    lengths = [1, 63, 0, 64, 65, 130, 200]
    print(f"decay={decay} prefill varlen {dtype} d_k={d_k} d_v={d_v} {path}", flush=True)
    x = ki.make_prefill(H=3, d_k=d_k, d_v=d_v, dtype=dtype, gate="softplus", lengths=lengths,
                        init_state_std=0.02, seed=61, device=DEV, decay=decay)
    o, fs = run_gpu(x, path)
    o_ref, s_ref = run_oracle(x)
    compare_full(x, o, fs, o_ref, s_ref, f"{decay} varlen {dtype}")
    assert torch.equal(fs[2], x["initial_state"][2])


@pytest.mark.parametrize("decay", DECAYS)
@pytest.mark.parametrize("dtype,path", [("fp32", "fused"), ("bf16", "fused"), ("bf16", "coop")])
def test_batched_xcd_mapping(decay, dtype, path):
    """B=2, H=4 (N*H = 8), T=300: four full chunks and a ragged tail."""
    print(f"decay={decay} prefill batched {dtype} {path}", flush=True)
    x = ki.make_prefill(B=2, T=300, H=4, d_k=128, d_v=128, dtype=dtype, seed=62, device=DEV,
                        decay=decay)
    o, fs = run_gpu(x, path)
    o_ref, s_ref = run_oracle(x)
    compare_full(x, o, fs, o_ref, s_ref, f"{decay} batched {dtype}")


@pytest.mark.parametrize("dtype,path", [("fp32", "fused"), ("bf16", "fused"), ("bf16", "coop")])
def test_reductions_to_channel_decay_bitwise(dtype, path):
    """A per-head g is the per-channel g with equal channels, and no decay is g = 0:
    the kernels must give bit-identical outputs and states for the two encodings."""
    print(f"decay reductions {dtype} {path}", flush=True)
    x = ki.make_prefill(H=4, d_k=128, d_v=128, dtype=dtype, lengths=[150, 64, 7],
                        init_state_std=0.02, seed=63, device=DEV, decay="head")
    o_h, s_h = run_gpu(x, path)
    xc = dict(x, g=x["g"][..., None].expand(*x["g"].shape, 128).contiguous())
    o_c, s_c = run_gpu(xc, path)
    assert torch.equal(o_h, o_c) and torch.equal(s_h, s_c)
    xn = dict(x, g=None)
    o_n, s_n = run_gpu(xn, path)
    xz = dict(x, g=torch.zeros_like(xc["g"]))
    o_z, s_z = run_gpu(xz, path)
    assert torch.equal(o_n, o_z) and torch.equal(s_n, s_z)


@pytest.mark.parametrize("path", PATHS)
def test_deltanet_one_hot_retrieval_exact(path):
    """No decay, beta = 1, one-hot keys: S k_i = v_i exactly; reads after the writes
    (across chunks) return the written bf16 values bit for bit."""
    d, n_write, T = 128, 90, 160
    rng = np.random.default_rng(64)
    keys = rng.permutation(d)[:n_write]
    vals = torch.from_numpy(rng.standard_normal((n_write, d))).to(torch.bfloat16)
    q = torch.zeros((1, T, 1, d))
    k = torch.zeros((1, T, 1, d))
    v = torch.zeros((1, T, 1, d))
    beta = torch.zeros((1, T, 1))
    for i in range(n_write):
        k[0, i, 0, keys[i]] = 1.0
        v[0, i, 0] = vals[i].float()
        beta[0, i, 0] = 1.0
    reads = list(range(n_write, T))
    targets = [(r * 11) % n_write for r in reads]
    for r, tgt in zip(reads, targets):
        q[0, r, 0, keys[tgt]] = 1.0
        k[0, r, 0, keys[tgt]] = 1.0
    x = dict(q=q.to(torch.bfloat16).to(DEV), k=k.to(torch.bfloat16).to(DEV),
             v=v.to(torch.bfloat16).to(DEV), g=None, beta=beta.to(DEV), cu_seqlens=None,
             initial_state=None)
    print(f"deltanet one-hot retrieval {path}", flush=True)
    o, fs = run_gpu(x, path, scale=1.0)
    for r, tgt in zip(reads, targets):
        assert torch.equal(o[0, r, 0].cpu(), vals[tgt]), f"token {r} should read value {tgt}"
    for i in range(n_write):
        assert torch.equal(fs[0, 0][:, keys[i]].cpu(), vals[i].float())


@pytest.mark.parametrize("decay", DECAYS)
def test_training_workload_every_unit(decay):
    """B4 H16 T4096 d128 bf16, both kernels, every unit against the oracle."""
    _every_unit(ki.TRAIN_PREFILL, decay=decay)


def test_long_workload_head_decay_every_unit():
    """H32 T65536 d128 bf16 (the long-context shape) with per-head decay, every unit."""
    _every_unit(ki.LONG_PREFILL, decay="head")


# ------------------------------------------------------------------ decode
def _decode_run(decay, dtype, N, H, d_k, d_v, steps, seed):
    d = ki.make_decode(N=N, H=H, d_k=d_k, d_v=d_v, steps=steps, dtype=dtype, seed=seed,
                       device=DEV, decay=decay)
    state = d["state"].clone()
    ref_state = ki.to_f64(d["state"])
    for t in range(steps):
        g = None if d["g"] is None else d["g"][t]
        o = kda.decode_step(d["q"][t], d["k"][t], d["v"][t], g, d["beta"][t], state)
        o_ref, ref_state = oracle_decode(ki.to_f64(d["q"][t]), ki.to_f64(d["k"][t]),
                                         ki.to_f64(d["v"][t]),
                                         None if g is None else ki.to_f64(g),
                                         ki.to_f64(d["beta"][t]), ref_state)
        torch.cuda.synchronize()
        check(dtype, ki.to_f64(o), o_ref, f"{decay} decode o step {t}")
        check(dtype, ki.to_f64(state), ref_state, f"{decay} decode state step {t}")


@pytest.mark.parametrize("decay", DECAYS)
@pytest.mark.parametrize("dtype,d_k,d_v", [("fp32", 64, 64), ("fp32", 128, 64),
                                           ("bf16", 128, 128), ("bf16", 64, 128)])
def test_decode(decay, dtype, d_k, d_v):
    print(f"decay={decay} decode {dtype} d_k={d_k} d_v={d_v}", flush=True)
    _decode_run(decay, dtype, 5, 3, d_k, d_v, steps=6, seed=65)


@pytest.mark.parametrize("decay", DECAYS)
@pytest.mark.parametrize("path", PATHS)
def test_decode_steps_match_prefill(decay, path):
    N, H, T, d = 2, 4, 70, 128
    print(f"decay={decay} decode vs prefill {path}", flush=True)
    x = ki.make_prefill(B=N, T=T, H=H, d_k=d, d_v=d, dtype="bf16", init_state_std=0.02,
                        seed=66, device=DEV, decay=decay)
    o_pre, s_pre = run_gpu(x, path)
    state = x["initial_state"].clone()
    outs = []
    for t in range(T):
        g = None if x["g"] is None else x["g"][:, t].contiguous()
        outs.append(kda.decode_step(x["q"][:, t].contiguous(), x["k"][:, t].contiguous(),
                                    x["v"][:, t].contiguous(), g,
                                    x["beta"][:, t].contiguous(), state))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1)
    check("bf16", ki.to_f64(o_dec), ki.to_f64(o_pre), f"{decay} decode vs prefill o")
    check("bf16", ki.to_f64(state), ki.to_f64(s_pre), f"{decay} decode vs prefill state")
