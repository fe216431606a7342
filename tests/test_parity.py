"""GPU parity: the HIP layer (through the C-ABI) against the fp64 oracle.

Bars: router logits within 1e-3 (max-abs relative to the largest logit and
relative L2); every discrete routing output (ids, mask bits, -1 ids, counts,
offsets, sorted lists, block map, active list) bit-exact against the oracle
run on the GPU's own float32 logits; y within relative L2 1e-2 (bf16 layer)
or 1e-5 (float32 layer) of the oracle's Eq. 8 on the same routing; tokens
with every slot masked exactly 0.  The y bound holds for the checked rows
together and for each row alone; unless a test names a sample, every row is
checked.
"""
import numpy as np
import pytest
import torch

import oracle
import dynamic_expert_sparsity_amd as B
from dynamic_expert_sparsity_amd import synth
from beamtest import (check_logits, check_routing_exact, check_y, gpu_routing_host, host, layer,
                      mode_record, need_gpu, run, sample_tokens)

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 1e-2}


def _full_check(L, K, tokens=None, block_m=0, flags=0, tau=0.0):
    need_gpu()
    y, R, lay = run(L, K, block_m=block_m, flags=flags, tau=tau)
    G = gpu_routing_host(R)
    check_logits(G, L)
    O = check_routing_exact(G, K, lay.sizes["block_m"], tau if tau else 0.5)
    err = check_y(y, L, K, O, TOL[L["x"].dtype], tokens)
    return y, G, O, err


# ---- tiny float32 layer: d=64, E=8, K=2, I=128, T=16 -----------------------
@pytest.mark.parametrize("mode,b", [("bias", 0.0), ("zero", 0.0), ("bias", -8.0)])
def test_tiny_fp32(mode, b):
    L = layer("tiny", 16, seed=100, mask_mode=mode, mask_bias=b)
    y, G, O, _ = _full_check(L, 2)
    if mode == "zero":
        assert G["mask"].min() == 1
    if b == -8.0:
        assert G["num_active"][0] == 0 and np.all(y == 0.0)


# ---- small bf16 layers: several tiles and a ragged tail ---------------------
SMALL = synth.LayerShape(128, 8, 2, 64, torch.bfloat16)


@pytest.mark.parametrize("T", [1, 5, 16, 63, 64, 65, 100, 300])
def test_small_bf16_tokens(T):
    L = layer(SMALL, T, seed=200 + T, mask_bias=0.0)
    _full_check(L, 2)


# Grouping at the batch sizes where its launches change: one routing
# workgroup up to 64 tokens, then the pair-scatter workgroups making their own
# tile bases up to 32 tiles (2048 tokens), then compact_bases first.  Shared
# experts ride along (the tile words of experts E..E+S-1 are full).
MID = synth.LayerShape(256, 48, 6, 128, torch.bfloat16)


@pytest.mark.parametrize("T", [64, 65, 128, 1024, 1025, 2048, 2049, 2113])
def test_grouping_launch_boundaries(T):
    need_gpu()
    L = layer(MID, T, seed=230 + T, mask_bias=-0.3, n_shared=1)
    lay = B.MoELayer(L["W_gate"], L["W_mask"], torch.cat([L["W_gu"], L["Ws_gu"]]).contiguous(),
                     torch.cat([L["W_dt"], L["Ws_dt"]]).contiguous(), 6)
    y, R = lay(L["x"])
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    G = gpu_routing_host({k: v.cpu() for k, v in R.items()})
    check_logits(G, L)
    O = check_routing_exact(G, 6, lay.sizes["block_m"], 0.5, n_shared=1)
    assert np.all(G["counts"][48:] == T)
    check_y(y, L, 6, O, TOL[torch.bfloat16], sample_tokens(T, 64, seed=T))


@pytest.mark.parametrize("E,K", [(8, 1), (8, 8), (60, 4), (64, 6), (256, 8), (130, 3)])
def test_expert_counts_and_topk(E, K):
    shape = synth.LayerShape(256, E, K, 64, torch.bfloat16)
    L = layer(shape, 77, seed=300 + E + K, mask_bias=-0.3)
    _full_check(L, K)


# streaming kernels whose k length ends in a short chunk (d % 256, I % 256 != 0)
@pytest.mark.parametrize("d,I,T", [(384, 192, 70), (640, 320, 33), (128, 1408, 40)])
def test_short_last_chunk(d, I, T):
    shape = synth.LayerShape(d, 16, 4, I, torch.bfloat16)
    L = layer(shape, T, seed=450 + d + I, mask_bias=0.0)
    _full_check(L, 4)


@pytest.mark.parametrize("bm", [16, 32, 64, 128])
def test_block_sizes(bm):
    L = layer(SMALL, 200, seed=400 + bm, mask_bias=0.2)
    _full_check(L, 2, block_m=bm)


@pytest.mark.parametrize("tau", [0.1, 0.3, 0.7, 0.9])
def test_threshold_variants(tau):
    L = layer(SMALL, 128, seed=500, mask_bias=0.0)
    y, G, O, _ = _full_check(L, 2, tau=tau)


# ---- Qwen3-30B-A3B-shaped layer (d=2048, E=128, K=8, I=768), decode --------
@pytest.mark.parametrize("T", [1, 8, 32, 128, 256])
@pytest.mark.parametrize("mode", ["bias", "zero"])
def test_qwen3_decode(T, mode):
    L = layer("qwen3", T, seed=600 + T, mask_bias=-1.04, mask_mode=mode)
    _full_check(L, 8)


# Small decode batches whose tokens have very different numbers of active
# slots (skewed recipe: per-token mask biases +1 / -2 / -8, so some tokens
# keep most slots and some none): the down kernel deals its workgroups to the
# tokens in proportion to their slot counts.
@pytest.mark.parametrize("T", [2, 3, 5, 8])
def test_qwen3_small_batch_uneven_slots(T):
    L = layer("qwen3", T, seed=650 + T, skew=True)
    _, G, O, _ = _full_check(L, 8)
    per_token = (np.asarray(O["masked_ids"]).reshape(T, 8) >= 0).sum(axis=1)
    if T >= 5:
        assert per_token.max() >= 4 and per_token.min() == 0, per_token


@pytest.mark.parametrize("b", [-1.04, 8.0])
def test_qwen3_prefill_2048(b):
    L = layer("qwen3", 2048, seed=700, mask_bias=b)
    _full_check(L, 8, tokens=sample_tokens(2048, 32, seed=1))


def test_zero_tokens():
    need_gpu()
    L = layer(SMALL, 0, seed=1)
    import dynamic_expert_sparsity_amd as B
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], 2)
    y, R = lay(L["x"])
    torch.cuda.synchronize()
    assert y.shape == (0, 128)


# ---- the tiled (prefill) path: grouped MFMA GEMMs over 128-position blocks
# (tiles of 128 rows, or 256 rows = two blocks of one expert) -----------------
GEMM_SMALL = synth.LayerShape(256, 8, 2, 128, torch.bfloat16)


@pytest.mark.parametrize("T", [1, 50, 300, 700])
def test_prefill_path_small(T):
    import dynamic_expert_sparsity_amd as B
    L = layer(GEMM_SMALL, T, seed=1000 + T, mask_bias=-0.2)
    y, G, O, _ = _full_check(L, 2, flags=B.BEAM_FORCE_PREFILL)


def test_prefill_and_decode_paths_agree():
    import dynamic_expert_sparsity_amd as B
    need_gpu()
    L = layer("qwen3", 600, seed=1100, mask_bias=0.0)
    yd, Rd, _ = run(L, 8, flags=B.BEAM_FORCE_DECODE)
    yp, Rp, lay = run(L, 8, flags=B.BEAM_FORCE_PREFILL)
    assert lay.sizes["path"] == 1 and lay.sizes["block_m"] == 128
    np.testing.assert_array_equal(Rd["masked_ids"].numpy(), Rp["masked_ids"].numpy())
    err = np.linalg.norm(yd - yp) / np.linalg.norm(yp)
    assert err < 5e-3


# ---- default above 512 tokens: the device picks, per call, the tiled kernels
# (blocks of <= 32 positions number >= 1.25 x the active experts, or one
# expert above 512 pairs) or the streaming kernels; skewed routing at E=16
# lands on the tiled side, at E=96 on the streaming side
def _expects_tiled(counts):
    act = counts[counts > 0]
    blocks = ((act + 31) // 32).sum()
    return 4 * blocks >= 5 * len(act) or counts.max() > 512


@pytest.mark.parametrize("E,tiled", [(16, True), (96, False)])
def test_per_call_kernel_choice(E, tiled):
    import dynamic_expert_sparsity_amd as B
    shape = synth.LayerShape(256, E, 2, 128, torch.bfloat16)
    L = layer(shape, 900, seed=1500, skew=True)
    y, G, O, _ = _full_check(L, 2)
    assert _expects_tiled(G["counts"]) == tiled
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], 2)
    lay(L["x"])
    assert lay.sizes["path"] == 1 and lay.sizes["block_m"] == 128


def _expected_family(counts, forced):
    act = counts[counts > 0]
    tiled = forced or 4 * ((act + 31) // 32).sum() >= 5 * len(act) or counts.max() > 512
    if not tiled:
        return 0
    n128 = ((act + 127) // 128).sum()
    n256 = ((act + 255) // 256).sum()
    return 1 if 10 * n128 < 13 * n256 else 2


# ---- the three kernel families: streaming, 128-row tiles, 256-row tiles
# (including 256-row tiles whose second half lies past the expert's segment)
@pytest.mark.parametrize("T,forced,b,family", [
    (300, True, 0.0, 1),      # ~37 pairs per expert: one 128-row tile each
    (1000, False, -0.3, 1),   # ~95 pairs per expert: tiled by the block rule, 128-row tiles
    (4096, False, 8.0, 2),    # ~1024 pairs per expert: 256-row tiles (half tiles at odd counts)
    (900, False, -1.5, 0),    # ~16 pairs per expert: streaming
])
def test_kernel_family_choice(T, forced, b, family):
    import dynamic_expert_sparsity_amd as B
    shape = synth.LayerShape(256, 16, 4, 128, torch.bfloat16)
    flags = B.BEAM_FORCE_PREFILL if forced else 0
    L = layer(shape, T, seed=1400 + T, mask_bias=b)
    y, G, O, _ = _full_check(L, 4, flags=flags)
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], 4, flags=flags)
    lay(L["x"])
    torch.cuda.synchronize()
    rec = mode_record(lay)
    counts = G["counts"]
    assert rec[0] == _expected_family(counts, forced)
    assert rec[0] == family, "the inputs did not land on the intended family"
    if family == 2:
        assert rec[2] == ((counts[counts > 0] + 255) // 256).sum()


# ---- the streaming kernels on the tiled path (above 512 tokens, where the
# device may still pick them), in both layouts: one column group per unit
# (~3 routed pairs per block of <= 32 positions at T = 700, b = -1.5) and two
# (~20 pairs per block at b = -0.1, whose ranges may begin or end with half a
# unit); the down projection's k length I = 384 ends in a short chunk (128
# of 256; the tiled path needs d % 256 == 0, so the up projection has none)
@pytest.mark.parametrize("T,b,wide", [(700, -1.5, 0), (700, -0.1, 1), (1500, -1.5, None)])
def test_streaming_on_tiled_path_short_chunks(T, b, wide):
    import dynamic_expert_sparsity_amd as B
    shape = synth.LayerShape(512, 64, 4, 384, torch.bfloat16)
    L = layer(shape, T, seed=1600 + T, mask_bias=b)
    y, G, O, _ = _full_check(L, 4)
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], 4)
    lay(L["x"])
    torch.cuda.synchronize()
    assert lay.sizes["path"] == 1
    rec = mode_record(lay)
    counts = G["counts"]
    assert rec[0] == _expected_family(counts, False) == 0
    blocks = ((counts[counts > 0] + 31) // 32).sum()
    assert rec[3] == (1 if counts.sum() >= 6 * blocks else 0)
    if wide is not None:
        assert rec[3] == wide, "the inputs did not land on the intended layout"


# ---- the streaming kernels' layout, chosen per call on the device: two
# column groups per unit once the routed pairs number >= 6 per block of <= 32
# positions (T = 500 keep ~0.5: ~16 pairs per expert), else one (keep ~0.15:
# ~5); on the streaming path (T <= 512) and forced decode above it
@pytest.mark.parametrize("T,b,flags,wide", [(500, 0.0, 0, 1), (500, -1.04, 0, 0),
                                            (1200, 0.0, 1, 1), (200, 8.0, 0, 1)])
def test_streaming_layout_choice(T, b, flags, wide):
    import dynamic_expert_sparsity_amd as B
    L = layer("qwen3", T, seed=1700 + T, mask_bias=b)
    y, G, O, _ = _full_check(L, 8, flags=flags)
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], 8, flags=flags)
    lay(L["x"])
    torch.cuda.synchronize()
    assert lay.sizes["path"] == 0
    counts = G["counts"]
    blocks = ((counts[counts > 0] + 31) // 32).sum()
    rec = mode_record(lay)
    assert rec[0] == 0 and rec[2] == blocks
    assert rec[3] == (1 if counts.sum() >= 6 * blocks else 0) == wide


# ---- both streaming layouts with short last k-chunks in both projections
# (d = 384 and I = 320 end in 128 and 64 of a 256-chunk)
@pytest.mark.parametrize("T,b,wide", [(300, 8.0, 1), (300, -1.5, 0), (37, 8.0, 1)])
def test_streaming_layouts_short_chunks(T, b, wide):
    import dynamic_expert_sparsity_amd as B
    shape = synth.LayerShape(384, 16, 4, 320, torch.bfloat16)
    L = layer(shape, T, seed=1800 + T, mask_bias=b)
    y, G, O, _ = _full_check(L, 4)
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], 4)
    lay(L["x"])
    torch.cuda.synchronize()
    assert lay.sizes["path"] == 0
    counts = G["counts"]
    blocks = ((counts[counts > 0] + 31) // 32).sum()
    assert mode_record(lay)[3] == (1 if counts.sum() >= 6 * blocks else 0) == wide


@pytest.mark.parametrize("b", [0.0, 8.0])
def test_qwen3_prefill_8192(b):
    L = layer("qwen3", 8192, seed=1200, mask_bias=b)
    _full_check(L, 8, tokens=sample_tokens(8192, 32, seed=2))


# the router-logit tilings of large batches with d % 256 != 0 (four waves
# split d): 32-token tiles of four column blocks (T <= 2048), 64-token tiles
# above; ragged last tiles and 2E = 16 columns (three of four blocks idle)
@pytest.mark.parametrize("T", [1500, 3001])
def test_router_tiles_large_batch(T):
    L = layer(SMALL, T, seed=1240 + T, mask_bias=0.0)
    _full_check(L, 2)


# above 4096 tokens the router's 64-token tiles take single-chunk LDS rings
# (two workgroups per CU): last tiles holding 1 and 44 tokens (every logit
# and route is checked); d = 128 gives two 64-wide k-chunks for four waves
@pytest.mark.parametrize("T", [4097, 8300])
def test_router_pair_tiles_ragged(T):
    L = layer(SMALL, T, seed=1250 + T, mask_bias=0.0)
    _full_check(L, 2)


# (T = 1024 at keep 0.15: the streaming kernels on the tiled path; T = 4096:
# the tiled kernels)
@pytest.mark.parametrize("T,b", [(1, -1.04), (64, 0.0), (1024, -1.04), (4096, -1.04)])
def test_large_layer(T, b):
    L = layer("large", T, seed=1300 + T, mask_bias=b)
    _full_check(L, 8)
