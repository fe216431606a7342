"""GPU: the allocation-free entry point beam_moe_forward_noalloc against
beam_moe_forward on the same inputs, on two calls in a row whose second has
the smaller batch (the static workspace keeps the first call's contents).
Same kernels, so every output must be bitwise equal (stronger than the
layer's 1e-2 bound); y is also checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

import dynamic_expert_sparsity_amd as B
from dynamic_expert_sparsity_amd import synth
from beamtest import check_routing_exact, check_y, gpu_routing_host, layer, need_gpu

pytestmark = pytest.mark.gpu


def _noalloc(L, K, T):
    E, d = L["W_gate"].shape
    I = L["W_gu"].shape[1] // 2
    desc = B.make_desc(T, d, E, K, I, L["x"].dtype)
    sizes = B.query(desc)
    R = B.alloc_routing(desc, sizes, L["x"].device)
    y = torch.empty((T, d), dtype=L["x"].dtype, device=L["x"].device)
    B.forward_noalloc(desc, L["x"][:T], L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], y, R)
    return y, R, sizes


@pytest.mark.parametrize("shape,K,T1,T2", [("qwen3", 8, 256, 40), ("qwen3", 8, 512, 1),
                                           (synth.LayerShape(128, 8, 2, 64, torch.bfloat16), 2,
                                            300, 5)])
def test_noalloc_matches_forward(shape, K, T1, T2):
    need_gpu()
    L = layer(shape, T1, seed=3300 + T1, mask_bias=-0.5)
    for T in (T1, T2):
        x = L["x"][:T].contiguous()
        lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], K)
        y_ref, R_ref = lay(x)
        y, R, sizes = _noalloc({**L, "x": x}, K, T)
        torch.cuda.synchronize()
        assert sizes["workspace_bytes"] <= B.NOALLOC_SCRATCH_BYTES
        assert torch.equal(y, y_ref), f"T={T}: y differs from beam_moe_forward"
        Gn = gpu_routing_host({k: v.cpu() for k, v in R.items()})
        Gr = gpu_routing_host({k: v.cpu() for k, v in R_ref.items()})
        for k in Gr:
            np.testing.assert_array_equal(Gn[k], Gr[k], err_msg=f"T={T}: {k}")
        O = check_routing_exact(Gn, K, sizes["block_m"])
        check_y(y.float().cpu().numpy(), {**L, "x": x}, K, O, 1e-2)
