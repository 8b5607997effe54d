"""The allocation-free prefill entry point (kda_prefill_noalloc, include/kda_noalloc.h)
through the C ABI: on two calls in a row, the second with a smaller input, its outputs
equal those of kda_prefill_ex with a caller workspace (the same kernels and plan), and
both meet the bf16 bar against the oracle.  Also: a request beyond the fixed scratch
is rejected before anything is launched."""

import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_39_amd as kda
import kda_inputs as ki
from oracle import forward as oracle_forward
from parity import check

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _noalloc():
    L = kda.lib()
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.kda_prefill_noalloc.restype = ctypes.c_int
    L.kda_prefill_noalloc.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp,
                                      vp, i32, i32, i64, i32, i32, i32, ctypes.c_float, vp, vp,
                                      vp, vp]
    L.kda_noalloc_scratch_bytes.restype = ctypes.c_size_t
    return L


def _call(fn_ex, x, o, fs, ws=None):
    N = x["N"]
    B, T, H, d_k = x["q"].shape
    d_v = x["v"].shape[-1]
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [1, kda.KDA_DECAY_CHANNEL, 0, p(x["q"]), p(x["k"]), p(x["v"]), p(x["g"]),
            p(x["beta"]), p(x["cu_seqlens"]), N, B, T, H, d_k, d_v, d_k ** -0.5,
            p(x["initial_state"]), p(fs), p(o)]
    if fn_ex:
        st = kda.lib().kda_prefill_ex(*args, p(ws), 0 if ws is None else ws.numel(), stream)
    else:
        st = _noalloc().kda_prefill_noalloc(*args, stream)
    assert st == 0, kda.lib().kda_status_string(st).decode()


@pytest.mark.parametrize("shape", [dict(B=1, T=4096, H=32), dict(B=2, T=700, H=8)])
def test_noalloc_equals_workspace_entry_point(shape):
    """Two calls in a row (the second smaller) through kda_prefill_noalloc and through
    kda_prefill_ex with a workspace give identical outputs; both meet the oracle bar."""
    big = ki.make_prefill(**shape, d_k=128, d_v=128, dtype="bf16", init_state_std=0.02,
                          seed=91, device=DEV)
    small = ki.make_prefill(H=shape["H"], d_k=128, d_v=128, dtype="bf16", init_state_std=0.02,
                            lengths=[130, 0, 65, 1], seed=92, device=DEV)
    print(f"noalloc vs workspace entry point {shape}", flush=True)
    for x in (big, small):
        N, H = x["N"], x["H"]
        B, T = x["q"].shape[:2]
        nb = kda.workspace_bytes(torch.bfloat16, N, B * T, H, 128, 128)
        assert 0 < nb <= _noalloc().kda_noalloc_scratch_bytes()
        ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
        o1, o2 = torch.empty_like(x["v"]), torch.empty_like(x["v"])
        f1 = torch.empty((N, H, 128, 128), device=DEV)
        f2 = torch.empty_like(f1)
        _call(True, x, o1, f1, ws)
        _call(False, x, o2, f2)
        torch.cuda.synchronize()
        assert not kda.workspace_aborted(ws)
        assert torch.equal(o1, o2) and torch.equal(f1, f2)
        # the oracle bar on the no-alloc outputs (units 0 and the last)
        units = [(0, 0), (N - 1, H - 1)]
        cu = None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu().numpy()
        o_ref, s_ref = oracle_forward(ki.to_f64(x["q"]), ki.to_f64(x["k"]), ki.to_f64(x["v"]),
                                      ki.to_f64(x["g"]), ki.to_f64(x["beta"]), cu_seqlens=cu,
                                      initial_state=ki.to_f64(x["initial_state"]), units=units)
        og = ki.to_f64(o2).reshape(-1, H, 128)
        orf = o_ref.reshape(-1, H, 128)
        bounds = ([(n, n * T, (n + 1) * T) for n in range(B)] if cu is None
                  else [(n, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)])
        for n, h in units:
            lo, hi = bounds[n][1], bounds[n][2]
            if hi > lo:
                check("bf16", og[lo:hi, h], orf[lo:hi, h], f"noalloc o seq {n} head {h}")
            check("bf16", ki.to_f64(f2[n, h]), s_ref[n, h], f"noalloc state seq {n} head {h}")


def test_noalloc_rejects_more_than_its_scratch(monkeypatch):
    """A ring deeper than the scratch holds is rejected with KDA_ERR_SCRATCH (7) and
    nothing is launched: the outputs keep their contents."""
    monkeypatch.setenv("KDA_COOP_R", "2000")
    x = ki.make_prefill(B=1, T=128, H=32, d_k=128, d_v=128, dtype="bf16", seed=93, device=DEV)
    nb = kda.workspace_bytes(torch.bfloat16, 1, 128, 32, 128, 128)
    L = _noalloc()
    assert nb > L.kda_noalloc_scratch_bytes()
    o = torch.full_like(x["v"], 3.0)
    fs = torch.full((1, 32, 128, 128), 5.0, device=DEV)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = L.kda_prefill_noalloc(1, 0, 0, p(x["q"]), p(x["k"]), p(x["v"]), p(x["g"]), p(x["beta"]),
                               None, 1, 1, 128, 32, 128, 128, 128 ** -0.5, None, p(fs), p(o), None)
    torch.cuda.synchronize()
    assert st == 7 and "scratch" in L.kda_status_string(7).decode()
    assert bool((o == 3.0).all()) and bool((fs == 5.0).all())
