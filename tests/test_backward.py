"""Mask-router backward (straight-through estimator + sparsity term) against
the fp64 oracle, on the GPU's own routing (ids, softmax weights, hard mask,
float32 mask logits).  The slot gradients dL/dg_hat are seeded synthetic
inputs.  Float32 arithmetic (dz, d_gate, dx, and dW of float32 layers) is
checked to 1e-5 relative; dW of bf16 layers runs on the matrix cores with dz
rounded to bf16 (2^-9 relative per element, float32 accumulation) and is
checked to 1e-2 relative L2."""
import numpy as np
import pytest
import torch

import oracle
import dynamic_expert_sparsity_amd as B
from dynamic_expert_sparsity_amd import synth
from beamtest import host, need_gpu, rel_l2

pytestmark = pytest.mark.gpu


def _case(shape, T, seed, beta, **kw):
    L = synth.make_layer(shape, T, seed=seed, device="cuda", **kw)
    sh = synth.SHAPES[shape] if isinstance(shape, str) else shape
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], sh.K)
    lay(L["x"])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 17)
    sg = torch.randn((T, sh.K), generator=gen, device="cuda", dtype=torch.float32)
    G = lay.mask_backward(L["x"], sg, beta)
    torch.cuda.synchronize()
    R = {k: v.cpu().numpy() for k, v in lay.routing.items()}
    O = oracle.mask_backward(host(L["x"]), host(L["W_mask"]), R["topk_ids"], R["topk_weights"],
                             R["mask"], R["mask_logits"], sg.cpu().numpy(), beta)
    return L, sh, {k: (v.cpu().numpy() if v is not None else None) for k, v in G.items()}, O, R


def _close(got, ref, rel, name):
    scale = max(float(np.abs(ref).max()), 1e-30)
    assert float(np.abs(got - ref).max()) <= rel * scale, f"{name} max abs err"
    assert rel_l2(got, ref) <= rel, f"{name} rel-L2 {rel_l2(got, ref):.3e}"


@pytest.mark.parametrize("shape,T,beta,kw", [
    ("tiny", 16, 0.0, {"mask_bias": 0.0}),
    ("tiny", 16, 0.05, {"mask_bias": -0.5}),
    ("qwen3", 1, 0.0, {"mask_bias": -1.04}),
    ("qwen3", 64, 0.01, {"mask_bias": -1.04}),
    ("qwen3", 300, 0.01, {"mask_bias": 0.0}),       # ragged token chunk
    ("qwen3", 2048, 0.001, {"mask_bias": -1.04}),   # several token ranges
    ("qwen3", 700, 0.02, {"mask_mode": "zero"}),    # the zero-initialised mask router
    (synth.LayerShape(256, 40, 3, 64, torch.bfloat16), 129, 0.1, {"mask_bias": 0.3}),  # E % 16 != 0
])
def test_mask_backward_matches_oracle(shape, T, beta, kw):
    need_gpu()
    L, sh, G, O, R = _case(shape, T, 3100 + T, beta, **kw)
    fp32 = sh.dtype == torch.float32
    _close(G["dz"], O["dz"], 1e-5, "dz")
    _close(G["d_gate"], O["d_gate"], 1e-5, "d_gate")
    _close(G["dx"], O["dx"], 1e-5, "dx")
    _close(G["dW_mask"], O["dW_mask"], 1e-5 if fp32 else 1e-2, "dW_mask")
    # exact zeros off the Top-K candidates
    cand = np.zeros_like(O["dz"], dtype=bool)
    np.put_along_axis(cand, R["topk_ids"].astype(np.int64), True, axis=1)
    assert np.all(G["dz"][~cand] == 0.0) and np.all(G["d_gate"][~cand] == 0.0)


def test_mask_backward_optional_outputs():
    need_gpu()
    sh = synth.SHAPES["qwen3"]
    T = 96
    L = synth.make_layer("qwen3", T, seed=3200, mask_bias=-0.5, device="cuda")
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], sh.K)
    lay(L["x"])
    sg = torch.ones((T, sh.K), device="cuda")
    full = lay.mask_backward(L["x"], sg, 0.01)
    part = lay.mask_backward(L["x"], sg, 0.01, want_dW=False, want_dx=False, want_d_gate=False)
    torch.cuda.synchronize()
    assert part["dW_mask"] is None and part["dx"] is None and part["d_gate"] is None
    assert torch.equal(part["dz"], full["dz"])
    # repeat calls are bitwise equal (fixed summation orders, no atomics)
    again = lay.mask_backward(L["x"], sg, 0.01)
    torch.cuda.synchronize()
    for k in ("dz", "dW_mask", "dx", "d_gate"):
        assert torch.equal(again[k], full[k]), k


@pytest.mark.parametrize("T", [96, 3000])
def test_mask_backward_each_output_alone(T):
    """dW alone (its token-range partials added by a reduction of their own
    at T = 3000) and dx alone (no partials to add) equal, bit for bit, what
    a call asking for every output writes."""
    need_gpu()
    sh = synth.SHAPES["qwen3"]
    L = synth.make_layer("qwen3", T, seed=3300 + T, mask_bias=-0.5, device="cuda")
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], sh.K)
    lay(L["x"])
    gen = torch.Generator(device="cuda")
    gen.manual_seed(T)
    sg = torch.randn((T, sh.K), generator=gen, device="cuda", dtype=torch.float32)
    full = lay.mask_backward(L["x"], sg, 0.01)
    only_dw = lay.mask_backward(L["x"], sg, 0.01, want_dx=False, want_d_gate=False)
    only_dx = lay.mask_backward(L["x"], sg, 0.01, want_dW=False, want_d_gate=False)
    torch.cuda.synchronize()
    assert only_dw["dx"] is None and only_dx["dW_mask"] is None
    assert torch.equal(only_dw["dW_mask"], full["dW_mask"])
    assert torch.equal(only_dx["dx"], full["dx"])
    assert torch.equal(only_dw["dz"], full["dz"]) and torch.equal(only_dx["dz"], full["dz"])
