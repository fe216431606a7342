"""Shared (always-on) experts: parity of the HIP layer with the fp64 oracle.

Shared expert s is expert E + s of the grouping: every token, weight 1, no
mask (news article on the paper, sections 5-6: the DeepSeek and Qwen1.5-MoE
models keep their shared experts on; a token whose routed slots are all
masked still passes through them).  The routing outputs must equal the
oracle's decisions on the GPU's logits bit for bit (the grouping now covers
E + S experts and pads with T*(K+S)); y is checked on the GPU's routing.
"""
import numpy as np
import pytest
import torch

import dynamic_expert_sparsity_amd as B
from dynamic_expert_sparsity_amd import synth
from beamtest import (check_routing_exact, check_y, gpu_routing_host, need_gpu, sample_tokens)

pytestmark = pytest.mark.gpu


def _layer(shape, T, S, seed, **kw):
    L = synth.make_layer(shape, T, seed=seed, n_shared=S, device="cuda", **kw)
    L["W_gu_all"] = torch.cat([L["W_gu"], L["Ws_gu"]]).contiguous()
    L["W_dt_all"] = torch.cat([L["W_dt"], L["Ws_dt"]]).contiguous()
    return L


def _run(L, K, flags=0):
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu_all"], L["W_dt_all"], K, flags=flags)
    y, R = lay(L["x"])
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), {k: v.cpu() for k, v in R.items()}, lay


def _check(L, shape, S, T, tol, flags=0, n_sample=48):
    y, R, lay = _run(L, shape.K, flags)
    G = gpu_routing_host(R)
    O = check_routing_exact(G, shape.K, lay.sizes["block_m"], n_shared=S)
    counts = G["counts"]
    assert len(counts) == shape.E + S and np.all(counts[shape.E:] == T)
    check_y(y, L, shape.K, O, tol, tokens=sample_tokens(T, n_sample, seed=T))
    return y, O


@pytest.mark.parametrize("name,T,b", [
    ("dsv2lite", 1, -1.04), ("dsv2lite", 64, -1.04), ("dsv2lite", 256, -1.04),
    ("dsv2lite", 700, -0.5),        # per-call choice between kernel families
    ("dsv2lite", 3000, -1.04),      # several tiles, separate pair scatter
    ("qwen15", 33, 0.0), ("qwen15", 300, -1.04),
])
def test_shared_bf16(name, T, b):
    need_gpu()
    shape, S = synth.SHAPES[name], synth.N_SHARED[name]
    L = _layer(shape, T, S, seed=2600 + T, mask_bias=b)
    _check(L, shape, S, T, 1e-2)


@pytest.mark.parametrize("T", [2, 8])
def test_shared_small_batch_uneven_slots(T):
    # small decode batch, skewed per-token mask biases: the tokens' slot
    # counts (2 shared + 0..6 routed) differ, and so do their down workgroups
    need_gpu()
    shape, S = synth.SHAPES["dsv2lite"], synth.N_SHARED["dsv2lite"]
    L = _layer(shape, T, S, seed=2650 + T, skew=True)
    _check(L, shape, S, T, 1e-2, n_sample=T)


@pytest.mark.parametrize("T", [5, 300])
def test_shared_tiled_forced(T):
    need_gpu()
    shape = synth.SHAPES["dsv2lite"]
    L = _layer(shape, T, 2, seed=2700 + T, mask_bias=-0.3)
    _check(L, shape, 2, T, 1e-2, flags=B.BEAM_FORCE_PREFILL)


def test_shared_fp32_tiny():
    need_gpu()
    shape = synth.LayerShape(64, 8, 2, 128, torch.float32)
    L = _layer(shape, 40, 3, seed=2800, mask_bias=0.0)
    _check(L, shape, 3, 40, 1e-5)


def test_all_routed_masked_tokens_get_the_shared_experts():
    need_gpu()
    shape = synth.SHAPES["dsv2lite"]
    T = 40
    L = _layer(shape, T, 2, seed=2900, mask_bias=-8.0)
    y, O = _check(L, shape, 2, T, 1e-2, n_sample=T)
    assert np.asarray(O["mask"]).max() == 0
    assert np.abs(y).max() > 0
    # the same call without the routed experts' weights mattering: a layer
    # whose experts are the two shared ones, both routed with weight 1/2 by
    # an all-zero gate and mask router, gives y / 2 up to bf16 rounding
    Wz = torch.zeros((2, shape.d), dtype=shape.dtype, device="cuda")
    lay2 = B.MoELayer(Wz, Wz, L["Ws_gu"].contiguous(), L["Ws_dt"].contiguous(), 2)
    y2, _ = lay2(L["x"])
    torch.cuda.synchronize()
    y2 = y2.float().cpu().numpy()
    err = np.linalg.norm(y - 2 * y2) / np.linalg.norm(y)
    assert err < 1e-2, err


def test_no_shared_unchanged():
    # n_shared = 0 through the same code: identical to the plain layer
    need_gpu()
    shape = synth.SHAPES["qwen3"]
    L = synth.make_layer(shape, 100, seed=3000, mask_bias=-1.04, device="cuda")
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], shape.K)
    y, R = lay(L["x"])
    torch.cuda.synchronize()
    assert lay.S == 0 and lay.desc.n_shared == 0
    G = gpu_routing_host({k: v.cpu() for k, v in R.items()})
    O = check_routing_exact(G, shape.K, lay.sizes["block_m"])
    check_y(y.float().cpu().numpy(), L, shape.K, O, 1e-2, tokens=sample_tokens(100, 32))
