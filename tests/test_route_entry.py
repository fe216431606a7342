"""GPU: beam_moe_route alone (paper section 3.2 Eq. 4-7 and the grouping of
the news article's section 5) on the batch sizes that take each routing
kernel: one workgroup (T <= 64), quarter-tile select + one grouping
workgroup with the pairs placed there (65..1024) or by the separate scatter
(above).  Every routing field must equal, bit for bit, both what
beam_moe_forward writes for the same layer and the oracle's routing on the
GPU's own logits.  The router logits (Eq. 4-5) are checked against the
oracle's at every token tiling, also for E not a multiple of 16 (a column
group holds rows of one router only, the rest clamped) and d whose 64-wide
k-chunks do not split evenly over the waves."""
import numpy as np
import pytest
import torch

import dynamic_expert_sparsity_amd as B
from dynamic_expert_sparsity_amd import synth
from beamtest import check_logits, check_routing_exact, gpu_routing_host, layer, need_gpu

pytestmark = pytest.mark.gpu

# d % 256 == 0 and I % 128 == 0: above 512 tokens the tiled path and its
# 128-position blocks, as in beam_moe_forward
SHAPE = synth.LayerShape(256, 16, 4, 128, torch.bfloat16)


@pytest.mark.parametrize("T", [40, 300, 700, 2000, 8300])
def test_route_matches_forward_and_oracle(T):
    need_gpu()
    L = layer(SHAPE, T, seed=3200 + T, mask_bias=-0.3)
    R = B.route(L["x"], L["W_gate"], L["W_mask"], SHAPE.K, SHAPE.I)
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], SHAPE.K)
    _, Rf = lay(L["x"])
    torch.cuda.synchronize()
    assert R["_sizes"]["block_m"] == lay.sizes["block_m"]
    assert R["_sizes"]["path"] == lay.sizes["path"]
    Gr = gpu_routing_host({k: v.cpu() for k, v in R.items() if not k.startswith("_")})
    Gf = gpu_routing_host({k: v.cpu() for k, v in Rf.items()})
    for k in Gf:
        np.testing.assert_array_equal(Gr[k], Gf[k], err_msg=k)
    check_routing_exact(Gr, SHAPE.K, lay.sizes["block_m"])


# 100 / 700 / 1500 / 3000 / 5000 tokens: each of the five token tilings of the
# router logits; E = 40 and 60 leave part-filled column groups, d = 384 and
# 640 give 6 and 10 k-chunks (runs of unequal length; idle waves at d = 384
# with eight waves)
@pytest.mark.parametrize("E,d", [(40, 384), (60, 640)])
@pytest.mark.parametrize("T", [100, 700, 1500, 3000, 5000])
def test_router_tilings_odd_shapes(E, d, T):
    need_gpu()
    shape = synth.LayerShape(d, E, 4, 128, torch.bfloat16)
    L = layer(shape, T, seed=3300 + T + E, mask_bias=-0.3)
    R = B.route(L["x"], L["W_gate"], L["W_mask"], shape.K, shape.I)
    torch.cuda.synchronize()
    G = gpu_routing_host({k: v.cpu() for k, v in R.items() if not k.startswith("_")})
    check_logits(G, L)
    check_routing_exact(G, shape.K, R["_sizes"]["block_m"])
