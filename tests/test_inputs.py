"""Seeded input generators: reproducible, with the recipe's shapes and ranges."""

import torch

import kda_inputs as ki


def test_prefill_reproducible_and_in_range():
    a = ki.make_prefill(B=2, T=33, H=3, d_k=16, d_v=8, dtype="bf16", gate="softplus", seed=7)
    b = ki.make_prefill(B=2, T=33, H=3, d_k=16, d_v=8, dtype="bf16", gate="softplus", seed=7)
    for name in ("q", "k", "v", "g", "beta"):
        assert torch.equal(a[name], b[name])
    assert a["q"].dtype == torch.bfloat16 and a["g"].dtype == torch.float32
    norms = a["k"].float().norm(dim=-1)
    assert torch.allclose(norms, torch.ones_like(norms), atol=1e-2)   # bf16-rounded unit keys
    assert (a["g"] < 0).all() and ((a["beta"] > 0) & (a["beta"] < 1)).all()
    c = ki.make_prefill(B=2, T=33, H=3, d_k=16, d_v=8, dtype="bf16", gate="softplus", seed=8)
    assert not torch.equal(a["q"], c["q"])


def test_uniform_gate_range_and_varlen_packing():
    w = ki.VARLEN_PREFILL
    lengths = ki.varlen_lengths(w.n_seqs, w.len_lo, w.len_hi, w.seed)
    assert len(lengths) == 8 and all(512 <= n <= 16384 for n in lengths)
    x = ki.make_prefill(H=2, d_k=8, d_v=8, lengths=[5, 0, 9], init_state_std=0.02, seed=3)
    assert x["cu_seqlens"].tolist() == [0, 5, 5, 14]
    assert x["q"].shape == (1, 14, 2, 8) and x["initial_state"].shape == (3, 2, 8, 8)
    assert ((x["g"] <= -0.001) & (x["g"] >= -0.1)).all()
    assert 0.01 < float(x["initial_state"].std()) < 0.03


def test_decode_shapes():
    d = ki.make_decode(N=3, H=2, d_k=8, d_v=4, steps=5, seed=1)
    assert d["state"].shape == (3, 2, 4, 8) and d["q"].shape == (5, 3, 2, 8)
    assert d["v"].shape == (5, 3, 2, 4) and d["beta"].shape == (5, 3, 2)


def test_decay_kinds():
    h = ki.make_prefill(B=1, T=9, H=3, d_k=8, d_v=4, decay="head", seed=2)
    assert h["g"].shape == (1, 9, 3) and (h["g"] < 0).all()
    n = ki.make_prefill(B=1, T=9, H=3, d_k=8, d_v=4, decay="none", seed=2)
    assert n["g"] is None and n["decay"] == "none"
    d = ki.make_decode(N=2, H=3, d_k=8, d_v=4, steps=2, decay="head", seed=1)
    assert d["g"].shape == (2, 2, 3)


def test_raw_projections():
    r = ki.make_prefill(B=1, T=20, H=2, d_k=16, d_v=4, raw=True, seed=3)
    norms = r["k"].float().norm(dim=-1)
    assert (norms > 1.5).any()                                  # keys are not unit
    assert (r["beta"] < 0).any() and (r["beta"] > 0).any()      # logits, both signs
    assert ((r["g"] >= 2) & (r["g"] <= 7)).all()                # retention logits
    d = ki.make_decode(N=2, H=2, d_k=8, d_v=4, steps=2, raw=True, decay="head", seed=1)
    assert d["g"].shape == (2, 2, 2) and (d["g"] >= 2).all()
