"""GPU properties of the HIP layer that hold at any size.

- determinism: repeated calls on the same inputs (same workspace) are
  bitwise equal;
- a token's output does not depend on the rest of the batch (the layer is
  per token, Eq. 8): rows of a batched call match single-token calls;
- tokens whose K slots are all masked produce exactly 0 (Eq. 6 note: the
  active count may reach zero; the residual path outside the layer carries
  such a token);
- W_mask = 0 (the paper's initialisation) activates every slot and gives the
  plain Top-K layer;
- the skewed-load workload (hot experts, 43% fully masked tokens) at full
  size, checked on sampled tokens.
"""
import numpy as np
import pytest
import torch

import dynamic_expert_sparsity_amd as B
from dynamic_expert_sparsity_amd import synth
from beamtest import (check_logits, check_routing_exact, check_y, gpu_routing_host, layer,
                      need_gpu, run, sample_tokens)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,T", [("qwen3", 1), ("qwen3", 256), ("qwen3", 2048),
                                     (synth.LayerShape(128, 8, 2, 64, torch.bfloat16), 300)])
def test_repeat_calls_bitwise_equal(shape, T):
    need_gpu()
    L = layer(shape, T, seed=900 + T, mask_bias=-0.5)
    K = (synth.SHAPES[shape] if isinstance(shape, str) else shape).K
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], K)
    outs = []
    for _ in range(3):
        y, R = lay(L["x"])
        torch.cuda.synchronize()
        outs.append((y.clone(), {k: v.clone() for k, v in R.items()}))
    for y, R in outs[1:]:
        assert torch.equal(y, outs[0][0])
        for k in R:
            n = R["num_active"][1].item() if k == "sorted_pairs" else None
            a, b = (R[k][:n], outs[0][1][k][:n]) if n is not None else (R[k], outs[0][1][k])
            if k in ("block_expert", "active_experts"):
                continue  # only the prefix is defined; compared below
            assert torch.equal(a, b), k
        na = R["num_active"].cpu()
        assert torch.equal(R["active_experts"][:na[2]], outs[0][1]["active_experts"][:na[2]])
        assert torch.equal(R["block_expert"][:na[3]], outs[0][1]["block_expert"][:na[3]])


def test_batch_rows_match_single_token_calls():
    need_gpu()
    T = 24
    L = layer("qwen3", T, seed=902, mask_bias=-0.3)
    yb, Rb, _ = run(L, 8)
    for t in (0, 5, 23):
        ys, Rs, _ = run(L, 8, x=L["x"][t:t + 1].contiguous())
        assert np.array_equal(Rs["masked_ids"].numpy()[0], Rb["masked_ids"].numpy()[t])
        ref = yb[t]
        err = np.linalg.norm(ys[0] - ref) / max(np.linalg.norm(ref), 1e-30)
        assert err <= 1e-2


def test_dead_tokens_exactly_zero_and_mixed_batch():
    need_gpu()
    T = 130
    L = layer("qwen3", T, seed=903, mask_bias=0.0)
    # make every third token fully masked through input channel 1
    L["W_mask"][:, 1] = 1.0
    L["x"][::3, 1] = -40.0
    L["x"][1::3, 1] = 0.0
    L["x"][2::3, 1] = 0.0
    y, R, _ = run(L, 8)
    G = gpu_routing_host(R)
    dead = np.where(G["mask"].sum(axis=1) == 0)[0]
    assert set(range(0, T, 3)) <= set(dead.tolist())
    assert np.all(y[dead] == 0.0)
    O = check_routing_exact(G, 8, 16)
    check_y(y, L, 8, O, 1e-2, tokens=sample_tokens(T, 40))


def test_zero_mask_router_is_plain_topk():
    need_gpu()
    L = layer("qwen3", 64, seed=904, mask_mode="zero")
    y, R, lay = run(L, 8)
    G = gpu_routing_host(R)
    assert G["mask"].min() == 1 and G["num_active"][0] == 64 * 8
    np.testing.assert_array_equal(G["g_hat"], G["topk_weights"])
    O = check_routing_exact(G, 8, lay.sizes["block_m"])
    check_y(y, L, 8, O, 1e-2, tokens=sample_tokens(64, 24))


def test_skewed_load_full_size():
    need_gpu()
    T = 16384
    L = layer("qwen3", T, seed=905, skew=True)
    y, R, lay = run(L, 8)
    G = gpu_routing_host(R)
    check_logits(G, L)
    O = check_routing_exact(G, 8, lay.sizes["block_m"])
    counts = G["counts"]
    assert counts.max() > 5 * counts.mean()          # hot experts
    frac_dead = (G["mask"].sum(axis=1) == 0).mean()
    assert 0.3 < frac_dead < 0.6                     # ~43% of tokens fully masked
    check_y(y, L, 8, O, 1e-2, tokens=sample_tokens(T, 48, seed=3))
