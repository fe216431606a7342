"""GPU: the Top-K tie rule and the mask at z = 0 exactly, through both select
kernels (one workgroup for a batch of at most 64 tokens; quarter-tile
workgroups above) and the router-logit tilings of small and large batches.

BEAM paper, section 3.2 Eq. 4 keeps the K largest router logits; equal logits
go to the lower expert index first (the slot order is descending logit, then
ascending index).  Eq. 6 keeps a slot iff sigmoid(z) >= 0.5, i.e. z >= 0, so
z = 0 (the zero-initialised mask router of the paper) keeps every slot.

Ties are forced by construction, not left to chance:
  * W_gate = 0: every router logit is 0, so the ids are 0..K-1 and every
    softmax weight is exactly 1/K;
  * twin experts: experts 2i and 2i+1 share a router row (twins inside one
    select lane's run of experts), or experts e and e + E/2 do (twins in
    different lanes).  With K odd, the K-th slot always splits a twin pair,
    so the lower twin must be kept and the higher one dropped;
  * W_mask = 0: every mask logit is exactly 0 and every slot is kept.
Every discrete output is compared bit for bit with the oracle on the GPU's own
logits, and y row by row with the oracle's Eq. 8.
"""
import numpy as np
import pytest
import torch

from dynamic_expert_sparsity_amd import synth
from beamtest import (check_logits, check_routing_exact, check_y, gpu_routing_host, layer,
                      need_gpu, run)

pytestmark = pytest.mark.gpu

# E = 128: 8 experts per select lane (16 lanes per token); d % 256 == 0 and
# I % 128 == 0: batches above 512 tokens take the tiled path
def _shape(K):
    return synth.LayerShape(256, 128, K, 128, torch.bfloat16)


TS = [1, 40, 300, 8200]


def _run_checked(L, K):
    need_gpu()
    y, R, lay = run(L, K)
    G = gpu_routing_host(R)
    check_logits(G, L)
    O = check_routing_exact(G, K, lay.sizes["block_m"])
    check_y(y, L, K, O, 1e-2, tokens=None if L["x"].shape[0] <= 512 else np.arange(0, 8200, 41))
    return G


@pytest.mark.parametrize("T", TS)
@pytest.mark.parametrize("K", [8, 3])
def test_zero_router_all_logits_tied(T, K):
    L = layer(_shape(K), T, seed=2000 + T + K, mask_bias=0.0)
    L["W_gate"].zero_()
    G = _run_checked(L, K)
    assert np.all(G["gate_logits"] == 0.0)
    np.testing.assert_array_equal(G["topk_ids"], np.tile(np.arange(K), (T, 1)))
    one_over_k = np.float32(1.0) / np.float32(K)
    assert np.all(G["topk_weights"] == one_over_k)


@pytest.mark.parametrize("T", TS)
@pytest.mark.parametrize("K", [3, 7])
@pytest.mark.parametrize("twins", ["in_lane", "across_lanes"])
def test_twin_experts_split_at_slot_k(T, K, twins):
    E = 128
    L = layer(_shape(K), T, seed=2100 + T + K, mask_bias=0.0)
    Wg = L["W_gate"]
    if twins == "in_lane":
        lo = torch.arange(0, E, 2, device=Wg.device)
        hi = lo + 1
    else:
        lo = torch.arange(0, E // 2, device=Wg.device)
        hi = lo + E // 2
    Wg[hi] = Wg[lo]
    G = _run_checked(L, K)
    r = G["gate_logits"]
    lo_n, hi_n = lo.cpu().numpy(), hi.cpu().numpy()
    # the twins' logits are bitwise equal (the tie exists on the device)
    np.testing.assert_array_equal(r[:, hi_n].view(np.uint32), r[:, lo_n].view(np.uint32))
    # K odd: the last slot holds the lower twin of a pair whose higher twin
    # is the next expert in logit order, and is dropped
    twin_of = np.empty(E, dtype=np.int64)
    twin_of[lo_n], twin_of[hi_n] = hi_n, lo_n
    last = G["topk_ids"][:, K - 1]
    assert np.all(np.isin(last, lo_n)), "slot K-1 holds a higher twin"
    assert not np.any(G["topk_ids"] == twin_of[last][:, None]), "both twins of the split pair kept"
    # within the kept set the twins sit side by side, lower first
    for k in range(0, K - 1, 2):
        a, b = G["topk_ids"][:, k], G["topk_ids"][:, k + 1]
        assert np.all(twin_of[a] == b) and np.all(a < b)


@pytest.mark.parametrize("T", TS)
def test_zero_mask_router_z_exactly_zero(T):
    K = 8
    L = layer(_shape(K), T, seed=2200 + T, mask_mode="zero")
    G = _run_checked(L, K)
    assert np.all(G["mask_logits"] == 0.0)
    assert G["mask"].min() == 1 and G["num_active"][0] == T * K
    np.testing.assert_array_equal(G["masked_ids"], G["topk_ids"])
    np.testing.assert_array_equal(G["g_hat"], G["topk_weights"])
