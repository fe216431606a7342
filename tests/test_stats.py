"""Device routing statistics (beam_moe_stats) against the oracle's counts on
the same routing, bit for bit; accumulation over calls; NULL outputs."""
import numpy as np
import pytest
import torch

import oracle
import dynamic_expert_sparsity_amd as B
from dynamic_expert_sparsity_amd import synth
from beamtest import layer, need_gpu

pytestmark = pytest.mark.gpu


def _oracle_stats(R, E):
    return oracle.routing_stats(R["mask"].cpu().numpy(), R["masked_ids"].cpu().numpy(), E)


@pytest.mark.parametrize("shape,T,kw", [
    ("tiny", 16, {"mask_bias": 0.0}),
    ("qwen3", 1, {"mask_bias": -1.04}),
    ("qwen3", 256, {"mask_bias": -1.04}),
    ("qwen3", 3000, {"skew": True}),          # several workgroups, ragged tail
    ("qwen3", 700, {"mask_mode": "zero"}),    # every slot active
    ("qwen3", 300, {"mask_bias": -8.0}),      # every slot masked
])
def test_stats_match_oracle(shape, T, kw):
    need_gpu()
    L = layer(shape, T, seed=2300 + T, **kw)
    sh = synth.SHAPES[shape]
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], sh.K)
    lay(L["x"])
    C = B.RoutingStats(sh.E, sh.K, "cuda")
    lay.stats(C)
    torch.cuda.synchronize()
    O = _oracle_stats(lay.routing, sh.E)
    np.testing.assert_array_equal(C.rank_masked.cpu().numpy(), O["rank_masked"])
    np.testing.assert_array_equal(C.active_hist.cpu().numpy(), O["active_hist"])
    np.testing.assert_array_equal(C.expert_load.cpu().numpy(), O["expert_load"])
    np.testing.assert_array_equal(C.expert_load.cpu().numpy(),
                                  lay.routing["expert_counts"].cpu().numpy())


def test_stats_accumulate_over_calls():
    need_gpu()
    sh = synth.SHAPES["qwen3"]
    C = B.RoutingStats(sh.E, sh.K, "cuda")
    want = {k: 0 for k in ("rank_masked", "active_hist", "expert_load")}
    for i, T in enumerate((64, 1, 333)):
        L = layer("qwen3", T, seed=2400 + i, mask_bias=-0.5)
        lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], sh.K)
        lay(L["x"])
        lay.stats(C)
        O = _oracle_stats(lay.routing, sh.E)
        for k in want:
            want[k] = want[k] + O[k]
    torch.cuda.synchronize()
    for k in want:
        np.testing.assert_array_equal(getattr(C, k).cpu().numpy(), want[k], err_msg=k)


def test_stats_null_outputs_skipped():
    import ctypes
    need_gpu()
    sh = synth.SHAPES["qwen3"]
    L = layer("qwen3", 100, seed=2500, mask_bias=-0.5)
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], sh.K)
    lay(L["x"])
    hist = torch.zeros(sh.K + 1, dtype=torch.int64, device="cuda")
    r = B.Routing(*[0] * 13)
    r.mask = lay.routing["mask"].data_ptr()
    r.masked_ids = lay.routing["masked_ids"].data_ptr()
    rc = B.lib().beam_moe_stats(ctypes.byref(lay.desc), ctypes.byref(r), None, hist.data_ptr(),
                                None, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    O = _oracle_stats(lay.routing, sh.E)
    np.testing.assert_array_equal(hist.cpu().numpy(), O["active_hist"])
