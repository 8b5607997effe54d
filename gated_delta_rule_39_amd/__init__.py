"""MI355X (gfx950) Kimi Delta Attention: chunked prefill, in-place decode and the
prefill's backward (gradients for training).

Thin Python binding over the C ABI in ``include/kda.h`` (``libkda.so``).  It only
marshals arguments: checks dtypes, devices and contiguity, allocates outputs with
torch, and passes device pointers plus the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback, and a missing
library raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# KDA_LIB_PATH selects another build of the library (e.g. the host-sanitized copy)
LIB_PATH = os.environ.get("KDA_LIB_PATH") or os.path.join(_PKG, "_lib", "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
_DTYPE_CODE = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}
# decay kinds: per key channel (KDA), one scalar per token and head (Gated DeltaNet), none
# (DeltaNet)
KDA_DECAY_CHANNEL, KDA_DECAY_HEAD, KDA_DECAY_NONE = 0, 1, 2
# prologue flags: k raw (L2-normalised in the kernel), beta and g given as logits
KDA_PRO_NORM_K, KDA_PRO_BETA_LOGIT, KDA_PRO_GATE_LOGIT = 1, 2, 4

_lib = None


class KDAError(RuntimeError):
    """A non-zero status from the KDA C ABI."""


def lib() -> ctypes.CDLL:
    """Load libkda.so (built in-tree by ``gated_delta_rule_39_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"KDA HIP library not built: {LIB_PATH} is missing; run "
            "`python -m gated_delta_rule_39_amd.build` (or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    L.kda_abi_version.restype = ctypes.c_int
    L.kda_abi_version.argtypes = []
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_status_string.argtypes = [ctypes.c_int]
    L.kda_prefill.restype = ctypes.c_int
    L.kda_prefill.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, i32, i32, i64, i32, i32, i32,
                              f32, vp, vp, vp, vp, sz, vp]
    L.kda_prefill_workspace_bytes.restype = sz
    L.kda_prefill_workspace_bytes.argtypes = [ctypes.c_int, i32, i64, i32, i32, i32]
    L.kda_prefill_plan.restype = ctypes.c_int
    L.kda_prefill_plan.argtypes = [ctypes.c_int, i32, i32, i32, i32,
                                   ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.kda_prefill_coop_plan.restype = ctypes.c_int
    L.kda_prefill_coop_plan.argtypes = [ctypes.c_int, i32, i32, i32, i32, ctypes.POINTER(i32),
                                        ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.kda_prefill_coop_lanes.restype = ctypes.c_int
    L.kda_prefill_coop_lanes.argtypes = [ctypes.c_int, i32, i32, i32, i32]
    L.kda_prefill_ex.restype = ctypes.c_int
    L.kda_prefill_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp,
                                 vp, i32, i32, i64, i32, i32, i32, f32, vp, vp, vp, vp, sz, vp]
    L.kda_decode_step.restype = ctypes.c_int
    L.kda_decode_step.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                  f32, vp]
    L.kda_backward.restype = ctypes.c_int
    L.kda_backward.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp,
                               i32, i32, i64, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp, vp, vp,
                               vp, vp, sz, vp]
    L.kda_backward_workspace_bytes.restype = sz
    L.kda_backward_workspace_bytes.argtypes = [ctypes.c_int, i32, i64, i32, i32, i32]
    L.kda_decode_step_ex.restype = ctypes.c_int
    L.kda_decode_step_ex.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp,
                                     vp, vp, i32, i32, i32, i32, f32, vp]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise KDAError(lib().kda_status_string(status).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (HIP) tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def prefill_plan(dtype: torch.dtype, N: int, H: int, d_k: int, d_v: int) -> Tuple[int, int]:
    """(v_tiles, workgroups) the prefill launch uses for these sizes."""
    nv, wg = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().kda_prefill_plan(_DTYPE_CODE[dtype], N, H, d_k, d_v, ctypes.byref(nv),
                                  ctypes.byref(wg)))
    return nv.value, wg.value


def prefill_coop_plan(dtype: torch.dtype, N: int, H: int, d_k: int, d_v: int):
    """(consumers, producers, ring_slots) of the producer/consumer prefill, or zeros."""
    a, b, c = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().kda_prefill_coop_plan(_DTYPE_CODE[dtype], N, H, d_k, d_v, ctypes.byref(a),
                                       ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def prefill_coop_lanes(dtype: torch.dtype, N: int, H: int, d_k: int, d_v: int) -> int:
    """Lanes of the producer/consumer prefill (0: not applicable)."""
    return int(lib().kda_prefill_coop_lanes(_DTYPE_CODE[dtype], N, H, d_k, d_v))


def workspace_bytes(dtype: torch.dtype, N: int, T_total: int, H: int, d_k: int, d_v: int) -> int:
    """Workspace size that selects the producer/consumer prefill (0: not applicable)."""
    return int(lib().kda_prefill_workspace_bytes(_DTYPE_CODE[dtype], N, T_total, H, d_k, d_v))


_workspaces = {}


def _auto_workspace(device, nbytes: int, purpose: str = "prefill"):
    """A workspace of at least ``nbytes`` cached per (purpose, device, stream): calls
    that share it are ordered on that stream."""
    key = (purpose, device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _decay_kind(g, qshape) -> int:
    """Decay kind from g's shape: q's shape = per key channel, q's shape without the
    last axis = one scalar per (token, head), None = no decay."""
    if g is None:
        return KDA_DECAY_NONE
    if tuple(g.shape) == tuple(qshape):
        return KDA_DECAY_CHANNEL
    if tuple(g.shape) == tuple(qshape[:-1]):
        return KDA_DECAY_HEAD
    raise ValueError(f"g must have shape {tuple(qshape)} (per key channel), "
                     f"{tuple(qshape[:-1])} (per head) or be None, got {tuple(g.shape)}")


def _flags(normalize_k: bool, beta_logit: bool, gate_logit: bool) -> int:
    return ((KDA_PRO_NORM_K if normalize_k else 0) | (KDA_PRO_BETA_LOGIT if beta_logit else 0)
            | (KDA_PRO_GATE_LOGIT if gate_logit else 0))


def workspace_aborted(ws: torch.Tensor, sticky: bool = False) -> bool:
    """True if the last producer/consumer call on ``ws`` stopped early (its outputs
    are invalid); with ``sticky``, if any call did since ``clear_workspace_abort``
    (synchronises)."""
    w = ws[:8].view(torch.int32)
    return int(w[1 if sticky else 0].item()) != 0


def clear_workspace_abort(ws: torch.Tensor) -> None:
    """Zero the sticky abort word of a producer/consumer workspace (enqueued)."""
    ws[4:8].zero_()


def _raise_if_aborted(ws: torch.Tensor, what: str) -> None:
    """Raise when the producer/consumer call that last used ``ws`` stopped early."""
    if workspace_aborted(ws):
        raise KDAError(f"{what}: a producer/consumer hand-off wait timed out and the call "
                       "stopped early; its outputs are invalid (NaN where not computed)")


def prefill(q, k, v, g, beta, *, cu_seqlens=None, scale=None, initial_state=None,
            output_final_state=True, out=None, final_state=None, workspace="auto",
            normalize_k=False, beta_logit=False, gate_logit=False, check=True):
    """Chunked KDA forward over packed sequences.

    q, k: [B, T, H, d_k]; v: [B, T, H, d_v] (all fp32 or all bf16); g (log alpha) fp32:
    [B, T, H, d_k] (per key channel, KDA), [B, T, H] (one decay per token and head,
    Gated DeltaNet) or None (no decay, DeltaNet); beta: [B, T, H] fp32; cu_seqlens: int32 [N+1] device tensor
    (B must be 1) or None (N = B); initial_state: [N, H, d_v, d_k] fp32 or None.
    ``final_state`` may be passed (and may be ``initial_state`` itself) to write the
    state in place.  ``workspace``: "auto" (a cached device buffer when the
    producer/consumer kernel applies), None (fused kernel), or a uint8 device tensor.
    Prologue (fused into the kernels): ``normalize_k`` L2-normalises each raw key row,
    ``beta_logit`` takes beta = sigmoid(beta), ``gate_logit`` takes the retention
    alpha = sigmoid(g) instead of exp(g).
    ``check``: when the producer/consumer kernel ran, wait for the call and raise
    ``KDAError`` if its hand-off aborted (outputs invalid).  ``check=False`` returns
    at once; the caller then reads ``workspace_aborted(ws)`` itself (the sticky word
    covers many calls: ``workspace_aborted(ws, sticky=True)``).
    Returns (o [B, T, H, d_v], final_state or None).
    """
    dev = q.device
    _need(q, "q", device=dev)
    dt = q.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"q/k/v must be float32 or bfloat16, got {dt}")
    for t, nm in ((k, "k"), (v, "v")):
        _need(t, nm, dtype=dt, device=dev)
    if g is not None:
        _need(g, "g", dtype=torch.float32, device=dev)
    _need(beta, "beta", dtype=torch.float32, device=dev)
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d_k]")
    B, T, H, d_k = q.shape
    d_v = v.shape[-1]
    decay = _decay_kind(g, q.shape)
    if k.shape != q.shape or v.shape != (B, T, H, d_v) or beta.shape != (B, T, H):
        raise ValueError("inconsistent q/k/v/g/beta shapes")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, device=dev)
        N = cu_seqlens.numel() - 1
        if B != 1:
            raise ValueError("packed sequences (cu_seqlens) need B == 1")
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", dtype=torch.float32, device=dev)
        if initial_state.shape != (N, H, d_v, d_k):
            raise ValueError("initial_state must be [N, H, d_v, d_k]")
    if scale is None:
        scale = d_k ** -0.5
    o = out if out is not None else torch.empty((B, T, H, d_v), dtype=dt, device=dev)
    _need(o, "out", dtype=dt, device=dev)
    fs = final_state
    if fs is None and output_final_state:
        fs = torch.empty((N, H, d_v, d_k), dtype=torch.float32, device=dev)
    if fs is not None:
        _need(fs, "final_state", dtype=torch.float32, device=dev)
        if fs.shape != (N, H, d_v, d_k):
            raise ValueError("final_state must be [N, H, d_v, d_k]")
    ws = None
    nb = workspace_bytes(dt, N, B * T, H, d_k, d_v)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a uint8 device tensor")
        ws = _auto_workspace(dev, nb) if nb > 0 else None
    elif workspace is not None:
        _need(workspace, "workspace", dtype=torch.uint8, device=dev)
        ws = workspace
    _check(lib().kda_prefill_ex(_DTYPE_CODE[dt], decay,
                                _flags(normalize_k, beta_logit, gate_logit), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                _ptr(beta), _ptr(cu_seqlens), N, B, T, H, d_k, d_v,
                                float(scale), _ptr(initial_state), _ptr(fs), _ptr(o), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(dev)))
    # the library reports a hand-off abort in the workspace only when it ran the
    # producer/consumer kernel, i.e. when the workspace is large enough for it
    if check and ws is not None and nb > 0 and ws.numel() >= nb and B * T > 0:
        _raise_if_aborted(ws, "kda.prefill")
    return o, fs


def decode_step(q, k, v, g, beta, state, *, scale=None, out=None, normalize_k=False,
                beta_logit=False, gate_logit=False):
    """One decode token per (sequence, head); ``state`` [N, H, d_v, d_k] fp32 is
    updated in place.  q, k: [N, H, d_k]; v: [N, H, d_v]; g fp32: [N, H, d_k] (per key
    channel), [N, H] (per head) or None (no decay); beta: [N, H] fp32.  The prologue
    flags are as for ``prefill``.  Returns o [N, H, d_v]."""
    dev = q.device
    _need(q, "q", device=dev)
    dt = q.dtype
    if dt not in _DTYPE_CODE:
        raise TypeError(f"q/k/v must be float32 or bfloat16, got {dt}")
    for t, nm in ((k, "k"), (v, "v")):
        _need(t, nm, dtype=dt, device=dev)
    if g is not None:
        _need(g, "g", dtype=torch.float32, device=dev)
    _need(beta, "beta", dtype=torch.float32, device=dev)
    _need(state, "state", dtype=torch.float32, device=dev)
    if q.dim() != 3:
        raise ValueError("q must be [N, H, d_k]")
    N, H, d_k = q.shape
    d_v = v.shape[-1]
    decay = _decay_kind(g, q.shape)
    if k.shape != q.shape or v.shape != (N, H, d_v) \
            or beta.shape != (N, H) or state.shape != (N, H, d_v, d_k):
        raise ValueError("inconsistent decode shapes")
    if scale is None:
        scale = d_k ** -0.5
    o = out if out is not None else torch.empty((N, H, d_v), dtype=dt, device=dev)
    _need(o, "out", dtype=dt, device=dev)
    _check(lib().kda_decode_step_ex(_DTYPE_CODE[dt], decay,
                                    _flags(normalize_k, beta_logit, gate_logit), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(beta), _ptr(state), _ptr(o), N, H, d_k, d_v,
                                    float(scale), _stream(dev)))
    return o


def backward_workspace_bytes(N: int, T_total: int, H: int, d_k: int, d_v: int) -> int:
    """Workspace bytes ``backward`` needs (bf16 chunk states and state gradients)."""
    return int(lib().kda_backward_workspace_bytes(KDA_BF16, N, T_total, H, d_k, d_v))


def _backward_uses_ring(N: int, H: int, d_k: int, d_v: int) -> bool:
    """Whether kda_backward's forward sweep runs on the producer/consumer kernel (its
    workspace then starts with the ring and the abort words): d_k = d_v = 128 and a
    producer/consumer plan with two consumers (include/kda.h, kda_backward)."""
    return d_k == 128 and d_v == 128 and prefill_coop_plan(torch.bfloat16, N, H, d_k, d_v)[0] == 2


def backward(q, k, v, g, beta, do, *, cu_seqlens=None, scale=None, initial_state=None,
             dfinal_state=None, need_dinitial_state=True, workspace="auto",
             normalize_k=False, beta_logit=False, gate_logit=False, check=True):
    """Gradients of ``prefill`` (bf16 inputs).  The prologue flags must be those of the
    forward call; the gradients are then with respect to the raw k, beta logits and
    retention logits.

    The inputs are those of the forward call; ``do`` [B, T, H, d_v] bf16 is dL/do and
    ``dfinal_state`` [N, H, d_v, d_k] fp32 (or None: zero) is dL/d(final state).
    ``workspace``: "auto" (a cached device buffer) or a uint8 device tensor of at least
    ``backward_workspace_bytes`` bytes.
    ``check``: as for ``prefill`` (raise if the forward sweep's hand-off aborted).
    Returns (dq, dk, dv [bf16], dg [fp32, g's shape, or None], dbeta [fp32],
    dinitial_state [fp32, or None]).
    """
    dev = q.device
    _need(q, "q", dtype=torch.bfloat16, device=dev)
    for t, nm in ((k, "k"), (v, "v"), (do, "do")):
        _need(t, nm, dtype=torch.bfloat16, device=dev)
    if g is not None:
        _need(g, "g", dtype=torch.float32, device=dev)
    _need(beta, "beta", dtype=torch.float32, device=dev)
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, d_k]")
    B, T, H, d_k = q.shape
    d_v = v.shape[-1]
    decay = _decay_kind(g, q.shape)
    if k.shape != q.shape or v.shape != (B, T, H, d_v) or do.shape != v.shape \
            or beta.shape != (B, T, H):
        raise ValueError("inconsistent q/k/v/do/g/beta shapes")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, device=dev)
        N = cu_seqlens.numel() - 1
        if B != 1:
            raise ValueError("packed sequences (cu_seqlens) need B == 1")
    else:
        N = B
    for t, nm in ((initial_state, "initial_state"), (dfinal_state, "dfinal_state")):
        if t is not None:
            _need(t, nm, dtype=torch.float32, device=dev)
            if t.shape != (N, H, d_v, d_k):
                raise ValueError(f"{nm} must be [N, H, d_v, d_k]")
    if scale is None:
        scale = d_k ** -0.5
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dg = None if g is None else torch.empty_like(g)
    dbeta = torch.empty_like(beta)
    ds0 = torch.empty((N, H, d_v, d_k), dtype=torch.float32, device=dev) \
        if need_dinitial_state else None
    nb = backward_workspace_bytes(max(N, 1), B * T, H, d_k, d_v)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto' or a uint8 device tensor")
        ws = _auto_workspace(dev, nb, "backward")
    else:
        _need(workspace, "workspace", dtype=torch.uint8, device=dev)
        ws = workspace
    _check(lib().kda_backward(KDA_BF16, decay, _flags(normalize_k, beta_logit, gate_logit),
                              _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                              _ptr(cu_seqlens), N, B, T, H, d_k, d_v, float(scale),
                              _ptr(initial_state), _ptr(do), _ptr(dfinal_state), _ptr(dq),
                              _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(ds0), _ptr(ws),
                              ws.numel(), _stream(dev)))
    if check and B * T > 0 and N > 0 and _backward_uses_ring(N, H, d_k, d_v):
        _raise_if_aborted(ws, "kda.backward")
    return dq, dk, dv, dg, dbeta, ds0
