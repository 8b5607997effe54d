"""GPU parity of the chunked prefill (kda_prefill through the C ABI) against the fp64
oracle: small cases compared element by element in full (several chunks, ragged
tails, empty sequences), the full-size workloads on sampled (sequence, head) units,
and the special cases the method has."""

import numpy as np
import pytest
import torch

import gated_delta_rule_39_amd as kda
import kda_inputs as ki
from oracle import forward as oracle_forward
from parity import check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
# bf16 prefill runs on two kernels: "fused" (each value tile computes the chunk tiles)
# and "coop" (producer workgroups hand the chunk tiles to the value tiles)
PATHS = ["fused", "coop"]


def run_gpu(x, path="fused", **kw):
    ws = None
    if path == "coop":
        N = x["cu_seqlens"].numel() - 1 if x["cu_seqlens"] is not None else x["q"].shape[0]
        B, T, H, d_k = x["q"].shape
        nb = kda.workspace_bytes(x["q"].dtype, N, B * T, H, d_k, x["v"].shape[-1])
        assert nb > 0, "producer/consumer kernel not applicable to this case"
        ws = torch.full((nb,), 0xA5, dtype=torch.uint8, device=DEV)   # contents must not matter
    o, fs = kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], cu_seqlens=x["cu_seqlens"],
                        initial_state=x["initial_state"], workspace=ws, **kw)
    torch.cuda.synchronize()
    if ws is not None:
        assert not kda.workspace_aborted(ws), "producer/consumer hand-off aborted"
    return o, fs


def run_oracle(x, units=None, scale=None):
    cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu().numpy()
    s0 = None if x["initial_state"] is None else ki.to_f64(x["initial_state"])
    g = None if x["g"] is None else ki.to_f64(x["g"])
    return oracle_forward(ki.to_f64(x["q"]), ki.to_f64(x["k"]), ki.to_f64(x["v"]),
                          g, ki.to_f64(x["beta"]), cu_seqlens=cu, scale=scale,
                          initial_state=s0, units=units)


def seq_bounds(x):
    if x["cu_seqlens"] is None:
        return [(n, n * x["T"], (n + 1) * x["T"]) for n in range(x["B"])]
    cu = x["cu_seqlens"].tolist()
    return [(n, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def compare_full(x, o, fs, o_ref, s_ref, label):
    dtype = x["dtype"]
    H, d_v = x["H"], x["d_v"]
    og = ki.to_f64(o).reshape(-1, H, d_v)
    orf = o_ref.reshape(-1, H, d_v)
    sg = ki.to_f64(fs)
    units_o, units_s = [], []
    for n, lo, hi in seq_bounds(x):
        for h in range(H):
            if hi > lo:
                units_o.append((f"seq {n} head {h}", og[lo:hi, h], orf[lo:hi, h]))
            units_s.append((f"seq {n} head {h}", sg[n, h], s_ref[n, h]))
    check(dtype, og, orf, f"{label} o", units=units_o)
    check(dtype, sg, s_ref, f"{label} final state", units=units_s)


# ------------------------------------------------------------------ small, whole-tensor cases
def test_tiny_fp32_workload():
    """B=1, H=2, T=256, d=64, fp32, zero initial state: every element vs the oracle."""
    print("prefill tiny fp32 workload", flush=True)
    x = ki.make_prefill_workload(ki.TINY_FP32, device=DEV)
    o, fs = run_gpu(x)
    o_ref, s_ref = run_oracle(x)
    compare_full(x, o, fs, o_ref, s_ref, "tiny fp32")


@pytest.mark.parametrize("dtype,d_k,d_v,path", [
    ("fp32", 64, 64, "fused"), ("fp32", 128, 128, "fused"), ("fp32", 64, 128, "fused"),
    ("bf16", 64, 64, "fused"), ("bf16", 128, 128, "fused"), ("bf16", 128, 64, "fused"),
    ("bf16", 64, 128, "fused"), ("bf16", 64, 64, "coop"), ("bf16", 128, 128, "coop"),
    ("bf16", 128, 64, "coop"), ("bf16", 64, 128, "coop")])
def test_varlen_ragged_with_initial_state(dtype, d_k, d_v, path):
    """Packed sequences with empty, sub-chunk, exact-chunk and ragged lengths, nonzero
    initial state, H=3 (N*H not a multiple of 8: plain workgroup mapping)."""
    lengths = [1, 63, 0, 64, 65, 130, 200]
    print(f"prefill varlen {dtype} d_k={d_k} d_v={d_v} {path} lengths={lengths}", flush=True)
    x = ki.make_prefill(H=3, d_k=d_k, d_v=d_v, dtype=dtype, gate="softplus", lengths=lengths,
                        init_state_std=0.02, seed=31, device=DEV)
    o, fs = run_gpu(x, path)
    o_ref, s_ref = run_oracle(x)
    compare_full(x, o, fs, o_ref, s_ref, f"varlen {dtype}")
    # the empty sequence returns its initial state untouched
    assert torch.equal(fs[2], x["initial_state"][2])


@pytest.mark.parametrize("dtype,path", [("fp32", "fused"), ("bf16", "fused"), ("bf16", "coop")])
def test_batched_multi_chunk_xcd_mapping(dtype, path):
    """B=2, H=4 (N*H = 8: XCD-grouped mapping), T=300 (4 full chunks + ragged tail)."""
    print(f"prefill batched {dtype} {path} B=2 H=4 T=300 d=128", flush=True)
    x = ki.make_prefill(B=2, T=300, H=4, d_k=128, d_v=128, dtype=dtype, gate="uniform", seed=32,
                        device=DEV)
    o, fs = run_gpu(x, path)
    o_ref, s_ref = run_oracle(x)
    compare_full(x, o, fs, o_ref, s_ref, f"batched {dtype}")


@pytest.mark.parametrize("bv", ["16", "32", "64"])
def test_value_tile_heights_agree(bv, monkeypatch):
    """Every value-tile height gives oracle parity (rows of S never mix)."""
    monkeypatch.setenv("KDA_PREFILL_BV", bv)
    x = ki.make_prefill(B=1, T=160, H=2, d_k=128, d_v=128, dtype="bf16", seed=33,
                        init_state_std=0.02, lengths=[70, 90], device=DEV)
    print(f"prefill BV={bv}", flush=True)
    o, fs = run_gpu(x, "fused")
    o_ref, s_ref = run_oracle(x)
    compare_full(x, o, fs, o_ref, s_ref, f"BV={bv}")


# ------------------------------------------------------------------ full-size workloads
def _sampled(w, units, label, path, decay="channel"):
    print(f"prefill full workload {w.name} {path} decay={decay}: units {units}", flush=True)
    x = ki.make_prefill_workload(w, device=DEV, decay=decay)
    o, fs = run_gpu(x, path)
    o_ref, s_ref = run_oracle(x, units=units)
    H, d_v = x["H"], x["d_v"]
    og = o.view(-1, H, d_v)
    orf = o_ref.reshape(-1, H, d_v)
    bounds = {n: (lo, hi) for n, lo, hi in seq_bounds(x)}
    for n, h in units:
        lo, hi = bounds[n]
        check("bf16", ki.to_f64(og[lo:hi, h]), orf[lo:hi, h], f"{label} o seq {n} head {h}")
        check("bf16", ki.to_f64(fs[n, h]), s_ref[n, h], f"{label} state seq {n} head {h}")
    # every output finite, nothing left unwritten
    assert torch.isfinite(o.float()).all()
    return x, o, fs


@pytest.mark.parametrize("path", PATHS)
def test_training_prefill_workload_sampled(path):
    _sampled(ki.TRAIN_PREFILL, [(0, 0), (1, 7), (2, 15), (3, 3), (3, 11)], "B4 H16 T4096", path)


@pytest.mark.parametrize("path", PATHS)
def test_long_prefill_workload_sampled(path):
    _sampled(ki.LONG_PREFILL, [(0, 0), (0, 17), (0, 31)], "H32 T65536", path)


@pytest.mark.parametrize("path", PATHS)
def test_varlen_prefill_workload_sampled(path):
    w = ki.VARLEN_PREFILL
    _sampled(w, [(0, 0), (1, 5), (3, 9), (5, 15), (7, 2)], "varlen N8", path)


# ------------------------------------------------------------------ method special cases
@pytest.mark.parametrize("path", PATHS)
def test_one_hot_retrieval_exact(path):
    """alpha = 1, beta = 1, distinct one-hot keys from a zero state, bf16-representable
    values; a later token with beta = 0, g = 0, q = k_i, scale = 1 reads v_i exactly.
    Writes in chunk 0 and 1, reads in chunk 2 (through the carried state) and in the
    writing chunk (through the intra-chunk term)."""
    d = 128
    n_write = 100
    T = 192
    rng = np.random.default_rng(41)
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
    targets = [(r * 7) % n_write for r in reads]
    for r, tgt in zip(reads, targets):
        q[0, r, 0, keys[tgt]] = 1.0
        k[0, r, 0, keys[tgt]] = 1.0
    # a read inside the first chunk: token 10 reads what token 3 wrote
    q[0, 10, 0, keys[3]] = 1.0
    x = dict(q=q.to(torch.bfloat16).to(DEV), k=k.to(torch.bfloat16).to(DEV),
             v=v.to(torch.bfloat16).to(DEV), g=torch.zeros((1, T, 1, d), device=DEV),
             beta=beta.to(DEV), cu_seqlens=None, initial_state=None)
    o, fs = run_gpu(x, path, scale=1.0)
    for r, tgt in zip(reads, targets):
        assert torch.equal(o[0, r, 0].cpu(), vals[tgt]), f"token {r} should read value {tgt}"
    assert torch.equal(o[0, 10, 0].cpu(), vals[3])
    # S k_i = v_i for every written key, exactly, in the fp32 final state
    for i in range(n_write):
        assert torch.equal(fs[0, 0][:, keys[i]].cpu(), vals[i].float())


@pytest.mark.parametrize("dtype,path", [("fp32", "fused"), ("bf16", "fused"), ("bf16", "coop")])
def test_beta_zero_decays_only(dtype, path):
    """beta = 0: the state only decays (closed form), and with g = 0 too it comes back
    bit-for-bit."""
    x = ki.make_prefill(B=1, T=150, H=2, d_k=64, d_v=64, dtype=dtype, init_state_std=0.1,
                        seed=42, device=DEV)
    x["beta"] = torch.zeros_like(x["beta"])
    o, fs = run_gpu(x, path)
    s0 = ki.to_f64(x["initial_state"])
    G = np.cumsum(ki.to_f64(x["g"])[0], axis=0)                      # [T, H, d_k]
    s_ref = s0[0] * np.exp(G[-1])[:, None, :]
    o_ref = np.einsum("hvk,thk->thv", s0[0], np.exp(G) * ki.to_f64(x["q"])[0]) * 64 ** -0.5
    check(dtype, ki.to_f64(fs[0]), s_ref, "beta=0 state")
    check(dtype, ki.to_f64(o[0]), o_ref, "beta=0 o")
    x["g"] = torch.zeros_like(x["g"])
    o, fs = run_gpu(x, path)
    assert torch.equal(fs, x["initial_state"])


@pytest.mark.parametrize("path", PATHS)
def test_split_resume_and_state_aliasing(path):
    """run(0..T) == run(0..t) then run(t..T) with initial = final; bit-for-bit when t is
    a chunk boundary.  final_state may alias initial_state."""
    x = ki.make_prefill(B=1, T=320, H=4, d_k=128, d_v=128, dtype="bf16", init_state_std=0.02,
                        seed=43, device=DEV)
    o_full, s_full = run_gpu(x, path)
    for t in (128, 100):
        a = {kk: (vv[:, :t].contiguous() if kk in ("q", "k", "v", "g", "beta") else vv)
             for kk, vv in x.items()}
        b = {kk: (vv[:, t:].contiguous() if kk in ("q", "k", "v", "g", "beta") else vv)
             for kk, vv in x.items()}
        o1, s1 = run_gpu(a, path)
        st = s1.clone()
        o2, _ = kda.prefill(b["q"], b["k"], b["v"], b["g"], b["beta"], initial_state=st,
                            final_state=st, workspace=None if path == "fused" else "auto")
        torch.cuda.synchronize()
        o_cat = torch.cat([o1, o2], dim=1)
        if t % 64 == 0:
            assert torch.equal(o_cat, o_full) and torch.equal(st, s_full)
        else:
            o_ref, s_ref = run_oracle(x)
            check("bf16", ki.to_f64(o_cat), o_ref, f"split at {t} o")
            check("bf16", ki.to_f64(st), s_ref, f"split at {t} state")


@pytest.mark.parametrize("path", PATHS)
def test_packed_equals_separate_calls_and_deterministic(path):
    lengths = [77, 200, 5]
    x = ki.make_prefill(H=8, d_k=128, d_v=128, dtype="bf16", lengths=lengths,
                        init_state_std=0.02, seed=44, device=DEV)
    o, fs = run_gpu(x, path)
    o2, fs2 = run_gpu(x, path)
    assert torch.equal(o, o2) and torch.equal(fs, fs2)          # run-to-run deterministic
    cu = x["cu_seqlens"].tolist()
    for n in range(len(lengths)):
        lo, hi = cu[n], cu[n + 1]
        y = {kk: (x[kk][:, lo:hi].contiguous()) for kk in ("q", "k", "v", "g", "beta")}
        y.update(cu_seqlens=None, initial_state=x["initial_state"][n:n + 1].contiguous())
        on, fsn = run_gpu(y, path)
        check("bf16", ki.to_f64(on), ki.to_f64(o[:, lo:hi]), f"separate seq {n} o")
        check("bf16", ki.to_f64(fsn[0]), ki.to_f64(fs[n]), f"separate seq {n} state")


@pytest.mark.parametrize("path", PATHS)
def test_decode_steps_match_prefill(path):
    """T decode steps from S_0 give the same outputs and state as one prefill of the
    same T tokens (both against the oracle too)."""
    N, H, T, d = 4, 4, 70, 128
    x = ki.make_prefill(B=N, T=T, H=H, d_k=d, d_v=d, dtype="bf16", init_state_std=0.02,
                        seed=45, device=DEV)
    o_pre, s_pre = run_gpu(x, path)
    state = x["initial_state"].clone()
    outs = []
    for t in range(T):
        outs.append(kda.decode_step(x["q"][:, t].contiguous(), x["k"][:, t].contiguous(),
                                    x["v"][:, t].contiguous(), x["g"][:, t].contiguous(),
                                    x["beta"][:, t].contiguous(), state))
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1)
    check("bf16", ki.to_f64(o_dec), ki.to_f64(o_pre), "decode vs prefill o")
    check("bf16", ki.to_f64(state), ki.to_f64(s_pre), "decode vs prefill state")


def test_no_final_state_and_scale_argument():
    x = ki.make_prefill(B=1, T=90, H=2, d_k=64, d_v=64, dtype="fp32", seed=46, device=DEV)
    o, fs = kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], scale=0.3,
                        output_final_state=False)
    torch.cuda.synchronize()
    assert fs is None
    o_ref, _ = run_oracle(x, scale=0.3)
    check("fp32", ki.to_f64(o), o_ref, "scale=0.3 o")
