"""GPU parity of the backward (kda_backward) against the fp64 backward oracle.

The oracle (oracle.kda_bwd_ref) is the exact gradient of the token recurrence, pinned
by finite differences, independent autodiff and closed forms (test_oracle_backward.py).
The HIP path computes through the chunk algebra in bf16 MFMA with fp32 accumulation,
so the bar is the bf16 one of tests/parity.py: rms(gpu - oracle) / rms(oracle) <= 2e-2
for each of dq, dk, dv, dg, dbeta and dL/dS_0, over the whole tensor and per
(sequence, head) unit.  Inputs: the seeded workload generator (kda_inputs) with bf16
q, k, v; dL/do and dL/d(final state) drawn here from their own seeded generator.
"""

import numpy as np
import pytest
import torch

import gated_delta_rule_39_amd as kda
import kda_inputs as ki
from oracle import backward as oracle_backward
from parity import BF16_RMS_REL, check, rms_rel

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def grads_in(x, seed, dfinal=True):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    do = torch.randn(x["v"].shape, generator=gen).to(torch.bfloat16).to(DEV)
    ds = None
    if dfinal:
        N = x["initial_state"].shape[0] if x["initial_state"] is not None else (
            x["cu_seqlens"].numel() - 1 if x["cu_seqlens"] is not None else x["q"].shape[0])
        H, d_v, d_k = x["q"].shape[2], x["v"].shape[3], x["q"].shape[3]
        ds = (0.1 * torch.randn((N, H, d_v, d_k), generator=gen)).to(DEV)
    return do, ds


def run_both(x, do, ds, flags=0):
    got = kda.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do,
                       cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"],
                       dfinal_state=ds, normalize_k=bool(flags & 1), beta_logit=bool(flags & 2),
                       gate_logit=bool(flags & 4))
    torch.cuda.synchronize()
    f = ki.to_f64
    ref = oracle_backward(
        f(x["q"]), f(x["k"]), f(x["v"]), None if x["g"] is None else f(x["g"]), f(x["beta"]),
        f(do), cu_seqlens=None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu().numpy(),
        initial_state=None if x["initial_state"] is None else f(x["initial_state"]),
        dfinal_state=None if ds is None else f(ds), flags=flags)
    return got, ref


NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


def compare(x, got, ref, label, dg_bar=BF16_RMS_REL):
    cu = x["cu_seqlens"]
    for name, a, r in zip(NAMES, got, ref):
        if r is None:
            assert a is None, name
            continue
        a = a.float().cpu().numpy().astype(np.float64)
        if name == "dg" and dg_bar != BF16_RMS_REL:
            err = rms_rel(a, r)
            print(f"  {label} {name}: rms-rel {err:.2e} (bound {dg_bar})", flush=True)
            assert np.isfinite(a).all() and err <= dg_bar, f"{label} dg: rms-rel {err:.3e}"
            continue
        err = check("bf16", a, r, f"{label} {name}")
        print(f"  {label} {name}: rms-rel {err:.2e}", flush=True)
        # per (sequence, head): token rows of each sequence, or the state of each unit.
        # A unit's relative error is only meaningful over enough elements: units with
        # fewer than 64 (a sequence shorter than a chunk, for dbeta) are covered by the
        # whole-tensor check above and printed.
        if name == "dS0":
            units = [(n, h) for n in range(r.shape[0]) for h in range(r.shape[1])]
            for n, h in units:
                if np.any(r[n, h]):
                    e = rms_rel(a[n, h], r[n, h])
                    assert e <= BF16_RMS_REL, f"{label} {name} unit ({n},{h}): {e:.3e}"
        elif cu is not None:
            bounds = cu.cpu().numpy()
            for n in range(len(bounds) - 1):
                lo, hi = bounds[n], bounds[n + 1]
                for h in range(r.shape[2]):
                    rs = r[0, lo:hi, h]
                    if rs.size and np.any(rs):
                        e = rms_rel(a[0, lo:hi, h], rs)
                        if rs.size < 64:
                            if e > BF16_RMS_REL:
                                print(f"  {label} {name} unit ({n},{h}) of {rs.size} values: "
                                      f"rms-rel {e:.2e} (gpu {a[0, lo:hi, h].ravel()[:4]}, "
                                      f"oracle {rs.ravel()[:4]})", flush=True)
                            continue
                        assert e <= BF16_RMS_REL, f"{label} {name} unit ({n},{h}): {e:.3e}"


@pytest.mark.parametrize("d_k,d_v", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_backward_varlen_ragged(d_k, d_v):
    """Packed sequences (empty, sub-chunk, exact-chunk, ragged, several chunks) with a
    nonzero initial state and a nonzero final-state gradient."""
    lengths = [1, 63, 0, 64, 65, 200]
    print(f"backward varlen d_k={d_k} d_v={d_v}", flush=True)
    x = ki.make_prefill(H=3, d_k=d_k, d_v=d_v, dtype="bf16", gate="softplus", lengths=lengths,
                        init_state_std=0.02, seed=71, device=DEV)
    do, ds = grads_in(x, 171)
    got, ref = run_both(x, do, ds)
    compare(x, got, ref, f"varlen {d_k}x{d_v}")


@pytest.mark.parametrize("decay", ["channel", "head", "none"])
def test_backward_decay_kinds(decay):
    """KDA, Gated DeltaNet and DeltaNet gradients, B=2 batch rows of 300 tokens (four
    full chunks and a ragged tail), H=4."""
    print(f"backward batched decay={decay}", flush=True)
    x = ki.make_prefill(B=2, T=300, H=4, d_k=128, d_v=128, dtype="bf16", seed=72, device=DEV,
                        init_state_std=0.02, decay=decay)
    do, ds = grads_in(x, 172)
    got, ref = run_both(x, do, ds)
    compare(x, got, ref, f"batched {decay}")


def test_backward_without_states():
    """No initial state and no final-state gradient (the common training call)."""
    print("backward zero states", flush=True)
    x = ki.make_prefill(H=2, d_k=128, d_v=128, dtype="bf16", lengths=[257, 31], seed=73,
                        device=DEV)
    do, _ = grads_in(x, 173, dfinal=False)
    got, ref = run_both(x, do, None)
    compare(x, got, ref, "zero states")


def test_backward_only_final_state_gradient():
    """dL/do = 0: every gradient comes through the final state alone."""
    print("backward final-state gradient only", flush=True)
    x = ki.make_prefill(H=2, d_k=128, d_v=128, dtype="bf16", lengths=[130], seed=74,
                        init_state_std=0.02, device=DEV)
    _, ds = grads_in(x, 174)
    do = torch.zeros_like(x["v"])
    got, ref = run_both(x, do, ds)
    compare(x, got, ref, "final-state only")


def test_backward_empty_batch_passes_state_gradient_through():
    """With no tokens the final state is the initial state: dL/dS_0 = dL/dS_T exactly."""
    print("backward empty sequences", flush=True)
    x = ki.make_prefill(H=2, d_k=64, d_v=64, dtype="bf16", lengths=[0, 0], seed=75,
                        init_state_std=0.02, device=DEV)
    _, ds = grads_in(x, 175)
    do = torch.zeros_like(x["v"])
    got = kda.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, cu_seqlens=x["cu_seqlens"],
                       initial_state=x["initial_state"], dfinal_state=ds)
    torch.cuda.synchronize()
    assert torch.equal(got[5], ds)


def test_backward_dv_matches_directional_derivative_of_forward_kernel():
    """Directional check with the GPU forward itself: the outputs and the final state are
    linear in v, so the central difference (L(v + eps u) - L(v - eps u)) / (2 eps) of the
    forward kernel (fp32 path) is exact up to rounding and must agree with <dv, u>.  The
    direction is dv itself (a random direction would make the projection small against
    |dv| |u| and the comparison ill-conditioned)."""
    print("backward directional derivative vs forward kernel", flush=True)
    x = ki.make_prefill(H=2, d_k=64, d_v=64, dtype="bf16", lengths=[150], seed=76,
                        init_state_std=0.02, device=DEV)
    do, ds = grads_in(x, 176)
    got = kda.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, cu_seqlens=x["cu_seqlens"],
                       initial_state=x["initial_state"], dfinal_state=ds)
    direction = got[2].float()
    direction = direction / direction.norm()
    eps = 1e-2

    def loss(vv):
        o, fs = kda.prefill(x["q"].float(), x["k"].float(), vv, x["g"], x["beta"],
                            cu_seqlens=x["cu_seqlens"], initial_state=x["initial_state"],
                            workspace=None)
        return float((o * do.float()).sum() + (fs * ds).sum())

    v32 = x["v"].float()
    fd = (loss(v32 + eps * direction) - loss(v32 - eps * direction)) / (2 * eps)
    an = float((got[2].float() * direction).sum())
    assert abs(fd - an) <= 2e-2 * max(abs(fd), 1.0), (fd, an)


def _segmented_head(args):
    from oracle import segmented_backward
    return segmented_backward(*args, segment=64)


def test_backward_lanes_many_units():
    """More (sequence, head) units than lanes: the forward sweep of the backward runs
    on the lane plan (units one after another per lane).  All gradients vs the oracle."""
    lengths = [5, 0, 200, 64, 1, 130, 63, 0, 65, 140, 17, 128, 0, 90, 100, 2, 40, 70, 0, 64]
    H = 4
    assert 0 < kda.prefill_coop_lanes(torch.bfloat16, len(lengths), H, 128, 128) < len(lengths) * H
    print(f"backward lanes N={len(lengths)} H={H}", flush=True)
    x = ki.make_prefill(H=H, d_k=128, d_v=128, dtype="bf16", lengths=lengths,
                        init_state_std=0.02, seed=80, device=DEV)
    do, ds = grads_in(x, 180)
    got, ref = run_both(x, do, ds)
    compare(x, got, ref, "lanes")


def test_backward_full_size_every_token():
    """The long-context workload (B=1, H=32, T=65536, d=128, bf16) in the launch
    configuration bench.py times, four heads compared over ALL 65536 tokens: the oracle
    runs the exact token backward segment by segment (one fp64 forward pass stores the
    state every 64 tokens; each segment's backward starts from its stored state and
    the state gradient carried back from the segment after it), one head per process.
    Every gradient is gated per head and per 64-token window."""
    import multiprocessing as mp
    import time
    from parity import check_unit
    heads = [0, 9, 21, 31]
    print("backward full size, every token of four heads", flush=True)
    x = ki.make_prefill_workload(ki.LONG_PREFILL, device=DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(178)
    do = torch.randn(x["v"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    got = kda.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, need_dinitial_state=False)
    torch.cuda.synchronize()
    f = lambda t, h: np.ascontiguousarray(ki.to_f64(t[0, :, h]))          # [T, d]
    jobs = [(f(x["q"], h)[None], f(x["k"], h)[None], f(x["v"], h)[None], f(x["g"], h)[None],
             ki.to_f64(x["beta"][0, :, h])[None], f(do, h)[None]) for h in heads]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(len(heads)) as pool:
        refs = pool.map(_segmented_head, jobs)
    print(f"  segmented oracle: {time.perf_counter() - t0:.1f} s", flush=True)
    for i, h in enumerate(heads):
        for name, a, r in zip(NAMES[:5], got[:5], refs[i][:5]):
            a = ki.to_f64(a[0, :, h])
            rel, worst, mx = check_unit(a, r[0], f"full-size head {h} {name}")
            print(f"  head {h} {name}: rms-rel {rel:.2e}, worst window {worst:.2e}, "
                  f"max|d|/rms {mx:.2e}", flush=True)


# The gradient kernel forms dL/dG per element as dKg Kg + dQg Qg - dKi Ki - dKh Kh
# (products of bf16-operand MFMA results with e^{+-G} factors) and dg by suffix sums
# over the chunk's rows, in which most of those terms cancel.  The stronger the decay,
# the larger the terms against what is left, so dg meets the bf16 bar up to a per-chunk
# decay of about 24 and is bounded at 5e-2 beyond (measured: 2.7e-2 at about 54); the
# other gradients meet the bar throughout.
DG_STRONG_BOUND = 5e-2


@pytest.mark.parametrize("gate", ["moderate", "strong", "edge"])
def test_backward_strong_decay(gate):
    """Gradients with per-chunk sums of |g| of about 24, 54 and 70 (inside the
    documented range)."""
    print(f"backward strong decay {gate}", flush=True)
    x = ki.make_prefill(H=3, d_k=128, d_v=128, dtype="bf16", gate=gate, lengths=[64, 130, 300],
                        init_state_std=0.02, seed=74, device=DEV)
    do, ds = grads_in(x, 174)
    got, ref = run_both(x, do, ds)
    compare(x, got, ref, f"strong decay {gate}",
            dg_bar=BF16_RMS_REL if gate == "moderate" else DG_STRONG_BOUND)


@pytest.mark.parametrize("decay,flags", [("channel", 7), ("head", 7), ("none", 7),
                                         ("channel", 1), ("channel", 2), ("channel", 4)])
def test_backward_prologue(decay, flags):
    """Gradients with respect to the raw projections of the fused prologue: raw keys
    (through the L2 normalisation), beta logits (through the sigmoid) and retention
    logits (through g = log sigmoid(a)); the oracle chains its own prologue."""
    print(f"backward prologue decay={decay} flags={flags}", flush=True)
    x = ki.make_prefill(H=3, d_k=128, d_v=128, dtype="bf16", lengths=[70, 1, 130], seed=79,
                        init_state_std=0.02, device=DEV, decay=decay, raw=True)
    if not flags & 1:   # keys as the plain entry points take them: unit rows
        x["k"] = (x["k"].float() / x["k"].float().norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    if not flags & 2:
        x["beta"] = torch.sigmoid(x["beta"])
    if not flags & 4 and x["g"] is not None:
        x["g"] = -torch.nn.functional.softplus(-x["g"])
    do, ds = grads_in(x, 179)
    got, ref = run_both(x, do, ds, flags)
    compare(x, got, ref, f"prologue {decay} {flags}")
