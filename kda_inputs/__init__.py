"""Seeded synthetic inputs for the KDA prefill and decode workloads.

This module is shared by the tests and the benchmark, and serves both the HIP path
and the CPU oracle.  It holds none of the method's arithmetic: it only draws
random tensors with the shapes and distributions of the workloads below and
rounds them to the input dtype.

Recipe (every workload): q, v ~ N(0, 1); k ~ N(0, 1), then L2-normalised over
d_k per (token, head) in fp32 (the caller-side precondition of the delta rule,
step-by-step page, FAQ "Why does DeltaNet need keys to be normalized?"); then
q, k, v are rounded to the input dtype (bf16 with round-to-nearest-even).  The
gate is g = log(alpha) in fp32, either -U(0.001, 0.1) ("uniform") or
-softplus(N(0, 1)) * 0.1 ("softplus"); beta = sigmoid(N(0, 1)) in fp32.  Two
strong-decay recipes probe the documented range of the per-chunk decay (the sum of
|g| over 64 tokens, per key channel, below about 80): "moderate", -U(0.25, 0.5)
(about 24 per chunk), "strong", -U(0.6, 1.1) (about 54) and "edge", -U(0.95, 1.25)
(about 70).  Past that range: "extreme", -U(2, 4) (about 190 per chunk, 48 per 16
tokens), and "spiky", the uniform gate plus, with probability 0.01 per token and
channel, a drop of -U(5, 20) (a near reset of that channel).  Initial
states, where present, are N(0, 0.02^2) fp32 (0.02 read as the standard
deviation).  The draw order is fixed: sequence lengths (varlen only), q, k, v,
g, beta, initial state.

Decay kinds: "channel" (KDA: g per key channel, [.., H, d_k]), "head" (Gated
DeltaNet: one g per token and head, [.., H], same distribution) and "none"
(DeltaNet: no g is drawn and g is None).

Raw projections (``raw=True``, for the fused prologue): k ~ N(0, 1) is not
normalised, beta holds logits ~ N(0, 1) (sigmoid gives the recipe's beta) and g
holds retention logits a ~ U(2, 7), so that log(sigmoid(a)) spans about the same
range as the uniform gate, -0.127 .. -0.0009; with gate "extreme", strongly negative
logits a ~ U(-4, -1) (log(sigmoid(a)) from -4.02 to -1.31).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class PrefillWorkload:
    """Shape and distribution recipe of one prefill workload."""
    name: str
    B: int
    T: int
    H: int
    d_k: int
    d_v: int
    dtype: str = "bf16"
    gate: str = "uniform"                  # "uniform" | "softplus"
    init_state_std: Optional[float] = None  # None -> zero initial state
    n_seqs: int = 0                         # >0: varlen, lengths ~ U[len_lo, len_hi]
    len_lo: int = 0
    len_hi: int = 0
    seed: int = 0


@dataclass(frozen=True)
class DecodeWorkload:
    """Shape and distribution recipe of one decode workload."""
    name: str
    N: int
    H: int
    d_k: int
    d_v: int
    steps: int
    dtype: str = "bf16"
    gate: str = "uniform"
    state_std: float = 0.02
    seed: int = 0


# The five workloads of the method's measurement plan, numbered 1..5.
TINY_FP32 = PrefillWorkload("tiny_fp32_B1_H2_T256_d64", B=1, T=256, H=2, d_k=64, d_v=64,
                            dtype="fp32", gate="uniform", seed=1)
TRAIN_PREFILL = PrefillWorkload("prefill_B4_H16_T4096_d128", B=4, T=4096, H=16, d_k=128,
                                d_v=128, dtype="bf16", gate="softplus", seed=2)
LONG_PREFILL = PrefillWorkload("prefill_B1_H32_T65536_d128", B=1, T=65536, H=32, d_k=128,
                               d_v=128, dtype="bf16", gate="uniform", seed=3)
VARLEN_PREFILL = PrefillWorkload("varlen_N8_U512-16384_H16_d128", B=1, T=0, H=16, d_k=128,
                                 d_v=128, dtype="bf16", gate="uniform", init_state_std=0.02,
                                 n_seqs=8, len_lo=512, len_hi=16384, seed=4)
DECODE = DecodeWorkload("decode_N256_H32_d128_1000steps", N=256, H=32, d_k=128, d_v=128,
                        steps=1000, dtype="bf16", gate="uniform", state_std=0.02, seed=5)

WORKLOADS = {w.name: w for w in (TINY_FP32, TRAIN_PREFILL, LONG_PREFILL, VARLEN_PREFILL, DECODE)}


def _gen(seed: int, device) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return gen


def _randn(gen, shape, device):
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)


def _gate(gen, shape, kind, device):
    if kind == "uniform":
        u = torch.rand(*shape, generator=gen, device=device, dtype=torch.float32)
        return -(0.001 + 0.099 * u)
    if kind == "softplus":
        return -torch.nn.functional.softplus(_randn(gen, shape, device)) * 0.1
    if kind in ("moderate", "strong", "edge", "extreme"):
        lo, hi = {"moderate": (0.25, 0.5), "strong": (0.6, 1.1), "edge": (0.95, 1.25),
                  "extreme": (2.0, 4.0)}[kind]
        u = torch.rand(*shape, generator=gen, device=device, dtype=torch.float32)
        return -(lo + (hi - lo) * u)
    if kind == "spiky":
        u = torch.rand(*shape, generator=gen, device=device, dtype=torch.float32)
        hit = torch.rand(*shape, generator=gen, device=device, dtype=torch.float32) < 0.01
        drop = torch.rand(*shape, generator=gen, device=device, dtype=torch.float32)
        return -(0.001 + 0.099 * u) - hit.float() * (5.0 + 15.0 * drop)
    raise ValueError(f"unknown gate recipe {kind!r}")


def _unit_keys(gen, shape, device):
    k = _randn(gen, shape, device)
    return k / k.norm(dim=-1, keepdim=True)


def varlen_lengths(n_seqs: int, lo: int, hi: int, seed: int):
    """Integer lengths uniform on [lo, hi] inclusive, drawn first from the seed."""
    gen = _gen(seed, "cpu")
    return torch.randint(lo, hi + 1, (n_seqs,), generator=gen).tolist()


def _gate_for(gen, lead, d_k, kind, decay, device, raw=False):
    if raw and decay in ("channel", "head"):
        shape = (*lead, d_k) if decay == "channel" else lead
        u = torch.rand(*shape, generator=gen, device=device, dtype=torch.float32)
        return -4.0 + 3.0 * u if kind == "extreme" else 2.0 + 5.0 * u
    if decay == "channel":
        return _gate(gen, (*lead, d_k), kind, device)
    if decay == "head":
        return _gate(gen, lead, kind, device)
    if decay == "none":
        return None
    raise ValueError(f"unknown decay kind {decay!r}")


def make_prefill(B=1, T=64, H=1, d_k=64, d_v=64, dtype="fp32", gate="uniform",
                 init_state_std=None, lengths=None, seed=0, device="cpu", decay="channel",
                 raw=False):
    """Draw one prefill batch.

    With ``lengths`` (a list of sequence lengths, zeros allowed) the batch is
    packed: B = 1, T = sum(lengths), and ``cu_seqlens`` (int32, on ``device``)
    holds the offsets.  Otherwise ``cu_seqlens`` is None and each of the B rows is
    one sequence of length T.

    Returns a dict with q, k, v ([B, T, H, d], dtype), g ([B, T, H, d_k] fp32 for
    decay "channel", [B, T, H] for "head", None for "none"), beta ([B, T, H] fp32), cu_seqlens, initial_state ([N, H, d_v, d_k] fp32 or
    None), N, lengths and the shape fields.
    """
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        B, T = 1, sum(lengths)
    N = len(lengths) if lengths is not None else B
    gen = _gen(seed, device)
    tdt = _DTYPES[dtype]
    q = _randn(gen, (B, T, H, d_k), device).to(tdt)
    k = (_randn(gen, (B, T, H, d_k), device) if raw
         else _unit_keys(gen, (B, T, H, d_k), device)).to(tdt)
    v = _randn(gen, (B, T, H, d_v), device).to(tdt)
    g = _gate_for(gen, (B, T, H), d_k, gate, decay, device, raw)
    beta = _randn(gen, (B, T, H), device)
    if not raw:
        beta = torch.sigmoid(beta)
    s0 = None
    if init_state_std is not None:
        s0 = _randn(gen, (N, H, d_v, d_k), device) * float(init_state_std)
    cu = None
    if lengths is not None:
        offs = [0]
        for n in lengths:
            offs.append(offs[-1] + n)
        cu = torch.tensor(offs, dtype=torch.int32, device=device)
    return dict(q=q, k=k, v=v, g=g, beta=beta, cu_seqlens=cu, initial_state=s0,
                N=N, B=B, T=T, H=H, d_k=d_k, d_v=d_v, dtype=dtype, lengths=lengths,
                decay=decay, raw=raw)


def make_prefill_workload(w: PrefillWorkload, device="cpu", decay="channel", raw=False):
    """Draw the named workload (varlen lengths first, from the same seed); ``decay``
    selects the gate's form (see the module docstring)."""
    lengths = None
    if w.n_seqs:
        lengths = varlen_lengths(w.n_seqs, w.len_lo, w.len_hi, w.seed)
    return make_prefill(B=w.B, T=w.T, H=w.H, d_k=w.d_k, d_v=w.d_v, dtype=w.dtype,
                        gate=w.gate, init_state_std=w.init_state_std, lengths=lengths,
                        seed=w.seed, device=device, decay=decay, raw=raw)


def make_decode(N=4, H=2, d_k=64, d_v=64, steps=1, dtype="bf16", gate="uniform",
                state_std=0.02, seed=0, device="cpu", decay="channel", raw=False):
    """Draw a decode run: initial state plus ``steps`` one-token inputs per
    (sequence, head).

    Returns a dict with state ([N, H, d_v, d_k] fp32), q, k, v
    ([steps, N, H, d], dtype), g ([steps, N, H, d_k] fp32; [steps, N, H] for decay
    "head"; None for "none"), beta ([steps, N, H]).
    """
    gen = _gen(seed, device)
    tdt = _DTYPES[dtype]
    state = _randn(gen, (N, H, d_v, d_k), device) * float(state_std)
    q = _randn(gen, (steps, N, H, d_k), device).to(tdt)
    k = (_randn(gen, (steps, N, H, d_k), device) if raw
         else _unit_keys(gen, (steps, N, H, d_k), device)).to(tdt)
    v = _randn(gen, (steps, N, H, d_v), device).to(tdt)
    g = _gate_for(gen, (steps, N, H), d_k, gate, decay, device, raw)
    beta = _randn(gen, (steps, N, H), device)
    if not raw:
        beta = torch.sigmoid(beta)
    return dict(state=state, q=q, k=k, v=v, g=g, beta=beta, N=N, H=H, d_k=d_k, d_v=d_v,
                steps=steps, dtype=dtype, decay=decay, raw=raw)


def make_decode_workload(w: DecodeWorkload, device="cpu", steps=None, decay="channel"):
    return make_decode(N=w.N, H=w.H, d_k=w.d_k, d_v=w.d_v,
                       steps=w.steps if steps is None else steps, dtype=w.dtype,
                       gate=w.gate, state_std=w.state_std, seed=w.seed, device=device,
                       decay=decay)


def to_f64(t):
    """Upcast a tensor (any device, any float dtype) to a float64 NumPy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
