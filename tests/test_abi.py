"""C ABI: the library loads, exports every declared symbol, and validates arguments
before any HIP call (so these run without a GPU and launch nothing)."""

import ctypes
import os
import re

import pytest

import gated_delta_rule_39_amd as kda

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADER = os.path.join(INCLUDE, "kda.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kda.LIB_PATH),
                                reason="libkda.so not built (run __graft_entry__.build())")


def declared_functions():
    """Every function declared in include/*.h (kda.h and the headers beside it)."""
    names = set()
    for f in sorted(os.listdir(INCLUDE)):
        if f.endswith(".h"):
            text = re.sub(r"/\*.*?\*/", "", open(os.path.join(INCLUDE, f)).read(), flags=re.S)
            names |= set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"kda_prefill", "kda_decode_step", "kda_abi_version", "kda_status_string",
            "kda_prefill_workspace_bytes", "kda_prefill_plan", "kda_prefill_coop_plan",
            "kda_prefill_ex", "kda_decode_step_ex", "kda_backward",
            "kda_backward_workspace_bytes", "kda_probe_hbm_copy", "kda_probe_hbm_read",
            "kda_probe_mfma_bf16", "kda_probe_read_sink_words"} <= set(names)
    L = kda.lib()
    for name in names:
        assert hasattr(L, name), f"{name} declared in kda.h but not exported"


def test_phase_stamps_only_in_the_timing_build():
    """The per-phase s_memtime stamps exist only in the timing build
    (_lib/phase/libkda.so, `python -m gated_delta_rule_39_amd.build --phases`): the
    product library exports no kda_phase_* function, the timing build (when built)
    exports all three."""
    names = ("kda_phase_read", "kda_phase_clear", "kda_phase_words", "kda_grad_phase_read",
             "kda_grad_phase_clear", "kda_grad_phase_words")
    L = kda.lib()
    for name in names:
        assert not hasattr(L, name), f"{name} in the product library"
    from gated_delta_rule_39_amd import build as kbuild
    if os.path.exists(kbuild.PHASE_LIB):
        P = ctypes.CDLL(kbuild.PHASE_LIB)
        for name in names:
            assert hasattr(P, name), f"{name} missing from the timing build"
        P.kda_phase_words.restype = ctypes.c_int
        assert P.kda_phase_words() == 4096 * 16


def test_version_and_status_strings():
    L = kda.lib()
    assert L.kda_abi_version() == 4
    for code in range(7):
        s = L.kda_status_string(code).decode()
        assert s.startswith("KDA")
    assert "unknown" in L.kda_status_string(99).decode()
    # fp32 inputs always take the fused kernel: no workspace
    assert L.kda_prefill_workspace_bytes(0, 8, 1 << 20, 16, 128, 128) == 0
    assert L.kda_prefill_workspace_bytes(1, 0, 0, 16, 128, 128) == 0


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def prefill_status(dtype=1, N=1, B=1, T=64, H=2, dk=64, dv=64, cu=None, q=FAKE, o=FAKE,
                   state=None):
    L = kda.lib()
    return L.kda_prefill(dtype, q, FAKE, FAKE, FAKE, FAKE, cu, N, B, T, H, dk, dv, 0.125,
                         state, state, o, None, 0, None)


def test_prefill_validation_codes():
    assert prefill_status(dtype=7) == 4                 # bad dtype
    assert prefill_status(dk=96) == 3                   # unsupported head dim
    assert prefill_status(dv=256) == 3
    assert prefill_status(N=-1) == 2                    # bad shape
    assert prefill_status(T=-5) == 2
    assert prefill_status(H=0) == 2
    assert prefill_status(N=2, B=1) == 2                # N != B without cu_seqlens
    assert prefill_status(cu=FAKE, N=2, B=2) == 2       # packed needs B == 1
    assert prefill_status(q=None) == 1                  # NULL input
    assert prefill_status(o=None) == 1
    assert prefill_status(N=0, B=0) == 0                # nothing to do: no launch
    assert prefill_status(T=0) == 0                     # empty and no final state


def test_decode_validation_codes():
    L = kda.lib()

    def st(dtype=1, N=4, H=2, dk=128, dv=128, state=FAKE):
        return L.kda_decode_step(dtype, FAKE, FAKE, FAKE, FAKE, FAKE, state, FAKE, N, H, dk, dv,
                                 0.1, None)

    assert st(dtype=3) == 4
    assert st(dk=32) == 3
    assert st(N=-1) == 2
    assert st(H=0) == 2
    assert st(state=None) == 1
    assert st(N=0) == 0


def test_decay_kind_validation_codes():
    L = kda.lib()

    def pf(decay, g=FAKE):
        return L.kda_prefill_ex(1, decay, 0, FAKE, FAKE, FAKE, g, FAKE, None, 1, 1, 64, 2, 64,
                                64, 0.125, None, None, FAKE, None, 0, None)

    def dc(decay, g=FAKE):
        return L.kda_decode_step_ex(1, decay, 0, FAKE, FAKE, FAKE, g, FAKE, FAKE, FAKE, 4, 2, 64,
                                    64, 0.1, None)

    for f in (pf, dc):
        assert f(3) == 3 and f(-1) == 3          # unknown decay kind: unsupported
        assert f(0, g=None) == 1                 # per-channel decay needs g
        assert f(1, g=None) == 1                 # per-head decay needs g
    # no decay with g NULL passes validation; with T = 0 and no final state nothing launches
    assert L.kda_prefill_ex(1, 2, 0, FAKE, FAKE, FAKE, None, FAKE, None, 1, 1, 0, 2, 64, 64,
                            0.125, None, None, FAKE, None, 0, None) == 0
    assert L.kda_decode_step_ex(1, 2, 0, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 0, 2, 64, 64,
                                0.1, None) == 0


def test_prologue_flag_validation():
    L = kda.lib()
    # known flags pass validation (T = 0 / N = 0: nothing launches); unknown bits are refused
    for f in (1, 2, 4, 7):
        assert L.kda_prefill_ex(1, 0, f, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 0, 2, 64, 64,
                                0.125, None, None, FAKE, None, 0, None) == 0
        assert L.kda_decode_step_ex(1, 0, f, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 64,
                                    64, 0.1, None) == 0
    for f in (8, 16, -1):
        assert L.kda_prefill_ex(1, 0, f, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 2, 64, 64,
                                0.125, None, None, FAKE, None, 0, None) == 3
        assert L.kda_decode_step_ex(1, 0, f, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 64,
                                    64, 0.1, None) == 3
    assert kda._flags(True, False, True) == kda.KDA_PRO_NORM_K | kda.KDA_PRO_GATE_LOGIT


def test_binding_decay_kind_from_g_shape():
    assert kda._decay_kind(None, (1, 4, 2, 8)) == kda.KDA_DECAY_NONE
    import torch
    assert kda._decay_kind(torch.zeros(1, 4, 2, 8), (1, 4, 2, 8)) == kda.KDA_DECAY_CHANNEL
    assert kda._decay_kind(torch.zeros(1, 4, 2), (1, 4, 2, 8)) == kda.KDA_DECAY_HEAD
    with pytest.raises(ValueError, match="g must have shape"):
        kda._decay_kind(torch.zeros(1, 4, 8), (1, 4, 2, 8))


def test_python_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError, match="device"):
        kda.prefill(x, x, x, x, torch.zeros(1, 4, 1))


def backward_status(dtype=1, decay=0, flags=0, N=1, B=1, T=64, H=2, dk=64, dv=64, cu=None,
                    dq=FAKE, ws=FAKE, ws_bytes=1 << 40, g=FAKE, dg=FAKE):
    L = kda.lib()
    return L.kda_backward(dtype, decay, flags, FAKE, FAKE, FAKE, g, FAKE, cu, N, B, T, H, dk, dv,
                          0.125, None, FAKE, None, dq, FAKE, FAKE, dg, FAKE, None, ws, ws_bytes,
                          None)


def test_backward_validation_codes():
    assert backward_status(dtype=7) == 4                # bad dtype
    assert backward_status(dtype=0) == 3                # fp32 backward: unsupported
    assert backward_status(decay=5) == 3
    assert backward_status(flags=8) == 3                # unknown prologue flag
    assert backward_status(dk=96) == 3
    assert backward_status(N=2, B=1) == 2               # N != B without cu_seqlens
    assert backward_status(dq=None) == 1
    assert backward_status(g=None) == 1                 # per-channel decay needs g and dg
    assert backward_status(dg=None) == 1
    assert backward_status(ws=None) == 6                # no workspace
    assert backward_status(ws_bytes=16) == 6            # too small
    assert backward_status(N=0, B=0) == 0               # nothing to do
    L = kda.lib()
    # two bf16 buffers of (T_total / 64 + N + 1) chunk slots of d_v x d_k per head, and
    # the factor tiles of every slot (bf16 KD, Qg, W [64][d_k], M [64][64]; fp32 e^{G_n})
    slots = (1000 // 64 + 4) * 4
    tiles = 3 * 64 * 128 * 2 + 64 * 64 * 2 + 128 * 4
    assert tiles == 388 * 128 + 8192
    assert L.kda_backward_workspace_bytes(1, 3, 1000, 4, 128, 64) == \
        slots * (2 * 64 * 128 * 2 + tiles)
    assert L.kda_backward_workspace_bytes(0, 3, 1000, 4, 128, 64) == 0


class _FakeLib:
    """Stands in for libkda.so: every call succeeds and launches nothing; the
    producer/consumer plan applies with a 1 KiB workspace."""

    def kda_prefill_workspace_bytes(self, *a):
        return 1024

    def kda_prefill_ex(self, *a):
        return 0

    def kda_backward_workspace_bytes(self, *a):
        return 1024

    def kda_backward(self, *a):
        return 0

    def kda_prefill_coop_plan(self, dtype, N, H, dk, dv, nc, np_, r):
        nc._obj.value, np_._obj.value, r._obj.value = 2, 5, 9
        return 0

    def kda_status_string(self, s):
        return b"KDA fake"


@pytest.mark.parametrize("word,raises", [(0, False), (1, True)])
def test_aborted_hand_off_makes_the_python_call_raise(monkeypatch, word, raises):
    """A workspace whose abort word is set after the call makes kda.prefill and
    kda.backward raise instead of returning the outputs (CPU tensors; the library
    and the device checks are replaced, only the binding's logic runs)."""
    import torch
    monkeypatch.setattr(kda, "lib", lambda: _FakeLib())
    monkeypatch.setattr(kda, "_need", lambda *a, **k: None)
    monkeypatch.setattr(kda, "_stream", lambda dev: None)
    B, T, H, d = 1, 64, 2, 128
    x = torch.zeros(B, T, H, d, dtype=torch.bfloat16)
    g = torch.zeros(B, T, H, d)
    beta = torch.zeros(B, T, H)
    ws = torch.zeros(1024, dtype=torch.uint8)
    ws[:4].view(torch.int32)[0] = word
    if raises:
        with pytest.raises(kda.KDAError, match="aborted|timed out"):
            kda.prefill(x, x, x, g, beta, workspace=ws)
        with pytest.raises(kda.KDAError, match="timed out"):
            kda.backward(x, x, x, g, beta, x, workspace=ws)
    else:
        o, fs = kda.prefill(x, x, x, g, beta, workspace=ws)
        assert o.shape == (B, T, H, d) and fs.shape == (1, H, d, d)
        kda.backward(x, x, x, g, beta, x, workspace=ws)
    # check=False leaves it to the caller
    kda.prefill(x, x, x, g, beta, workspace=ws, check=False)
    assert kda.workspace_aborted(ws) == raises


def test_sticky_abort_word():
    import torch
    ws = torch.zeros(64, dtype=torch.uint8)
    assert not kda.workspace_aborted(ws, sticky=True)
    ws[4:8].view(torch.int32)[0] = 1
    assert kda.workspace_aborted(ws, sticky=True) and not kda.workspace_aborted(ws)
    kda.clear_workspace_abort(ws)
    assert not kda.workspace_aborted(ws, sticky=True)


def test_probe_validation_codes():
    L = kda.lib()
    L.kda_probe_hbm_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.kda_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    L.kda_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    assert L.kda_probe_hbm_copy(None, FAKE, 1024, None) == 1
    assert L.kda_probe_hbm_copy(FAKE, FAKE, 1000, None) == 2      # not a multiple of 16
    assert L.kda_probe_hbm_read(FAKE, 0, FAKE, None) == 2
    assert L.kda_probe_mfma_bf16(FAKE, 0, 10, None) == 2
    assert L.kda_probe_mfma_bf16(None, 4, 10, None) == 1
    assert L.kda_probe_read_sink_words() > 0
