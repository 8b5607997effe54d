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
from parity import check, check_rows, check_unit

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
    check(dtype, og, orf, f"{label} o", units=units_o, windows=True)
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
def _every_unit(w, decay="channel"):
    """A full-size workload in the launch configuration the benchmark times, on both
    kernels, against the oracle over EVERY (sequence, head) unit: o per unit and per
    64-token window (plus max|delta|/rms), final state per unit."""
    import time
    from fullsize import oracle_all_units
    print(f"prefill full workload {w.name} decay={decay}: every unit", flush=True)
    x = ki.make_prefill_workload(w, device=DEV, decay=decay)
    t0 = time.perf_counter()
    o_ref, s_ref = oracle_all_units(x)
    print(f"  oracle over {x['N'] * x['H']} units: {time.perf_counter() - t0:.1f} s", flush=True)
    H, d_v = x["H"], x["d_v"]
    bounds = seq_bounds(x)
    for path in PATHS:
        o, fs = run_gpu(x, path)
        og = ki.to_f64(o).reshape(-1, H, d_v)
        sg = ki.to_f64(fs)
        worst = [0.0, 0.0, 0.0]
        for n, lo, hi in bounds:
            for h in range(H):
                st = check_unit(og[lo:hi, h], o_ref[lo:hi, h], f"{w.name} {path} o seq {n} head {h}")
                worst = [max(a, b) for a, b in zip(worst, st)]
        ws = check_rows(sg.reshape(-1, sg.shape[-2] * sg.shape[-1]),
                        s_ref.reshape(-1, sg.shape[-2] * sg.shape[-1]), f"{w.name} {path} final state")
        print(f"  {path}: o worst unit rms-rel {worst[0]:.2e}, worst window {worst[1]:.2e}, "
              f"worst max|d|/rms {worst[2]:.2e}; final state worst unit {ws:.2e}", flush=True)
        del o, fs, og, sg
    return x


def test_training_prefill_workload_every_unit():
    _every_unit(ki.TRAIN_PREFILL)


def test_long_prefill_workload_every_unit():
    _every_unit(ki.LONG_PREFILL)


def test_varlen_prefill_workload_every_unit():
    _every_unit(ki.VARLEN_PREFILL)


# ------------------------------------------------------------------ strong decay
@pytest.mark.parametrize("gate", ["strong", "edge"])
@pytest.mark.parametrize("dtype,path", [("fp32", "fused"), ("bf16", "fused"), ("bf16", "coop")])
def test_strong_decay_within_documented_range(gate, dtype, path):
    """Per-channel decay whose per-chunk sum of |g| is about 54 ("strong") or 70
    ("edge"), inside the documented limit of about 80: the decay factors of a chunk
    then span e^-70 .. 1, and their reciprocals e^70."""
    lengths = [1, 64, 130, 300]
    print(f"prefill strong decay {gate} {dtype} {path}", flush=True)
    x = ki.make_prefill(H=4, d_k=128, d_v=128, dtype=dtype, gate=gate, lengths=lengths,
                        init_state_std=0.02, seed=47, device=DEV)
    if x["g"] is not None:   # sequence 1 is exactly one chunk: its per-channel |g| sums
        chunk = -x["g"][0, 1:65].sum(dim=0)
        assert 45.0 < float(chunk.min()) and float(chunk.max()) < 80.0
    o, fs = run_gpu(x, path)
    o_ref, s_ref = run_oracle(x)
    compare_full(x, o, fs, o_ref, s_ref, f"strong decay {gate} {dtype} {path}")


# ------------------------------------------------------------------ past the chunk-start range
def chunk_block_sums(x, rows):
    """Largest per-channel sum of |g| over an aligned group of ``rows`` tokens of any
    64-token chunk (chunks start at each sequence's first token)."""
    g = -ki.to_f64(x["g"])
    if g.ndim == 3:                      # one g per token and head
        g = g[..., None]
    worst = 0.0
    for _, lo, hi in seq_bounds(x):
        gs = g.reshape(-1, *g.shape[2:]) if x["cu_seqlens"] is not None else None
        for c0 in range(lo, hi, 64):
            for r0 in range(c0, min(c0 + 64, hi), rows):
                seg = gs[r0:min(r0 + rows, c0 + 64, hi)] if gs is not None else None
                if seg is not None and seg.size:
                    worst = max(worst, float(seg.sum(axis=0).max()))
    return worst


@pytest.mark.parametrize("gate,paths", [("spiky", ["fused", "coop"]), ("extreme", ["coop"])])
def test_strong_decay_block_factored(gate, paths):
    """Chunks in which some 8 tokens of a channel decay by more than e^-10 take the
    block-factored form on the producer/consumer kernel.  "spiky": near resets of
    single channels at a moderate total decay (both kernels); "extreme": about 190
    per chunk, past the range of chunk-start factors (producer/consumer kernel only;
    the documented limit of the block form is a 16-token sum of about 85)."""
    # no single-token sequence: one row's output is one query-key product, whose bf16
    # relative error is about 2^-8 / |cos(q, k)| once the decay factors are far from 1
    # (the per-unit bar needs rows to average over)
    lengths = [45, 64, 130, 300, 17]
    print(f"prefill strong decay {gate} {paths}", flush=True)
    x = ki.make_prefill(H=4, d_k=128, d_v=128, dtype="bf16", gate=gate, lengths=lengths,
                        init_state_std=0.02, seed=51, device=DEV)
    b8, b16, b64 = chunk_block_sums(x, 8), chunk_block_sums(x, 16), chunk_block_sums(x, 64)
    print(f"  largest 8-token sum {b8:.1f}, 16-token {b16:.1f}, chunk {b64:.1f}", flush=True)
    assert b8 > 10.0 and b16 < 80.0
    assert "fused" not in paths or b64 < 80.0   # the fused kernel's chunk-start range
    o_ref, s_ref = run_oracle(x)
    for path in paths:
        o, fs = run_gpu(x, path)
        compare_full(x, o, fs, o_ref, s_ref, f"strong decay {gate} {path}")


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


# ------------------------------------------------------------------ lanes
# With more (sequence, head) units than lanes of producer/consumer workgroups, a plan
# made on the device spreads the units over the lanes and each lane works through its
# units one after another.
LANE_LENGTHS = {
    # every kind of length (empty, sub-chunk, exact, ragged, several chunks), the
    # longest ones not first
    "mixed": [5, 0, 200, 64, 1, 130, 63, 0, 65, 300, 17, 128, 0, 90, 257, 2, 40, 191, 0, 64,
              33, 129, 7, 0, 150, 64, 11, 0, 250, 66, 3, 99, 0, 128, 45, 180, 0, 70, 1, 310],
    # fewer units with chunks than lanes: some lanes get no unit, the empty ones share
    "sparse": [0] * 17 + [130, 0, 1, 0, 64] + [0] * 18,
}


@pytest.mark.parametrize("kind", sorted(LANE_LENGTHS))
def test_lanes_many_units(kind):
    lengths = LANE_LENGTHS[kind]
    H = 4
    lanes = kda.prefill_coop_lanes(torch.bfloat16, len(lengths), H, 128, 128)
    print(f"prefill lanes {kind}: N={len(lengths)} H={H} lanes={lanes}", flush=True)
    assert 0 < lanes < len(lengths) * H, "the case must take the lane plan"
    x = ki.make_prefill(H=H, d_k=128, d_v=128, dtype="bf16", lengths=lengths,
                        init_state_std=0.02, seed=48, device=DEV)
    o, fs = run_gpu(x, "coop")
    o_ref, s_ref = run_oracle(x)
    compare_full(x, o, fs, o_ref, s_ref, f"lanes {kind}")
    for n, ln in enumerate(lengths):
        if ln == 0:   # empty sequences return their initial state untouched
            assert torch.equal(fs[n], x["initial_state"][n]), f"sequence {n}"


def test_lanes_at_plan_limits():
    """The largest lane plan: 256 sequences x 32 heads = 8192 units -- 248 short
    sequences of 0 .. 48 tokens (most units are one partial chunk, so lanes switch
    units at nearly every chunk) and 8 of 150 .. 300 -- every unit and window against
    the oracle."""
    rng = np.random.default_rng(53)
    lengths = [int(n) for n in rng.integers(0, 49, size=248)] + \
              [int(n) for n in rng.integers(150, 301, size=8)]
    lengths = [lengths[i] for i in rng.permutation(len(lengths))]
    H = 32
    assert 0 < kda.prefill_coop_lanes(torch.bfloat16, len(lengths), H, 128, 128) < len(lengths) * H
    print(f"prefill lanes at the plan limits: N=256 H=32, {sum(lengths)} tokens", flush=True)
    x = ki.make_prefill(H=H, d_k=128, d_v=128, dtype="bf16", lengths=lengths,
                        init_state_std=0.02, seed=53, device=DEV)
    o, fs = run_gpu(x, "coop")
    o_ref, s_ref = run_oracle(x)
    compare_full(x, o, fs, o_ref, s_ref, "lanes at the plan limits")


@pytest.mark.parametrize("kind", sorted(LANE_LENGTHS))
def test_lane_plan_is_longest_first_greedy(kind):
    """The plan the kernel writes into the workspace (after a 256-byte header:
    lane_off[lanes + 1], the lanes' unit lists, then each lane's chunk total, int32) is
    the stated rule:
    sequences by chunk count, longest first (ties: lower index), each of a sequence's
    units to the lane with the fewest chunks so far (ties: lower lane).  Recomputed
    here on the host and compared exactly; so every unit is in exactly one lane."""
    lengths = LANE_LENGTHS[kind]
    H, N = 4, len(LANE_LENGTHS[kind])
    x = ki.make_prefill(H=H, d_k=128, d_v=128, dtype="bf16", lengths=lengths, seed=48, device=DEV)
    L = kda.prefill_coop_lanes(torch.bfloat16, N, H, 128, 128)
    U = N * H
    assert 0 < L < U
    nb = kda.workspace_bytes(torch.bfloat16, N, sum(lengths), H, 128, 128)
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    kda.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], cu_seqlens=x["cu_seqlens"], workspace=ws)
    torch.cuda.synchronize()
    plan = ws[256:256 + 4 * (2 * L + 1 + U)].view(torch.int32).cpu().numpy()
    nch = [(n + 63) // 64 for n in lengths]
    load, lists = [0] * L, [[] for _ in range(L)]
    for n in sorted(range(N), key=lambda m: (-nch[m], m)):
        for h in range(H):
            lane = min(range(L), key=lambda i: (load[i], i))
            lists[lane].append(n * H + h)
            load[lane] += nch[n]
    off = np.cumsum([0] + [len(li) for li in lists])
    assert np.array_equal(plan[:L + 1], off), "lane offsets"
    assert np.array_equal(plan[L + 1:L + 1 + U],
                          np.concatenate([np.array(li, dtype=np.int64) for li in lists])), "unit lists"
    assert np.array_equal(plan[L + 1 + U:], np.array(load)), "lane totals"


@pytest.mark.parametrize("kind", ["one unit per lane", "lanes"])
def test_plain_dispatch_equals_cooperative(kind, monkeypatch):
    """KDA_COOP_LAUNCH=plain (the same grid as an ordinary dispatch, when the device
    holds all of it resident) gives bit-for-bit the cooperative launch's results."""
    lengths = [300, 64, 130, 0, 5, 190] if kind == "lanes" else [300, 64, 130]
    H = 12 if kind == "lanes" else 4
    x = ki.make_prefill(H=H, d_k=128, d_v=128, dtype="bf16", lengths=lengths,
                        init_state_std=0.02, seed=52, device=DEV)
    print(f"prefill plain dispatch, {kind}", flush=True)
    o, fs = run_gpu(x, "coop")
    monkeypatch.setenv("KDA_COOP_LAUNCH", "plain")
    o1, fs1 = run_gpu(x, "coop")
    assert torch.equal(o, o1) and torch.equal(fs, fs1)


def test_lanes_bit_identical_to_one_unit_per_lane(monkeypatch):
    """The lane plan only changes which workgroups process a unit, not its arithmetic:
    o and final state equal, bit for bit, those of one unit per lane (the same
    consumer, forced by KDA_COOP_LANES=0 and KDA_COOP_NC=2)."""
    lengths = [300, 64, 130, 0, 5, 190]
    H = 12
    x = ki.make_prefill(H=H, d_k=128, d_v=128, dtype="bf16", lengths=lengths,
                        init_state_std=0.02, seed=49, device=DEV)
    assert 0 < kda.prefill_coop_lanes(torch.bfloat16, len(lengths), H, 128, 128) < len(lengths) * H
    print("prefill lanes vs one unit per lane", flush=True)
    o, fs = run_gpu(x, "coop")
    monkeypatch.setenv("KDA_COOP_LANES", "0")
    monkeypatch.setenv("KDA_COOP_NC", "2")
    assert kda.prefill_coop_lanes(torch.bfloat16, len(lengths), H, 128, 128) == len(lengths) * H
    assert kda.prefill_coop_plan(torch.bfloat16, len(lengths), H, 128, 128)[0] == 2
    o1, fs1 = run_gpu(x, "coop")
    assert torch.equal(o, o1) and torch.equal(fs, fs1)


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
