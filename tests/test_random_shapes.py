"""Parity of the HIP layer with the fp64 oracle over a fixed, seeded draw of
layer shapes, batch sizes, thresholds, shared-expert counts and path flags
(a spread of the cases the targeted tests pin one at a time): every routing
output bit-exact against the oracle's decisions on the GPU's logits, y to
the bf16 (1e-2) or float32 (1e-5) bound on sampled tokens.
"""
import numpy as np
import pytest
import torch

import dynamic_expert_sparsity_amd as B
from dynamic_expert_sparsity_amd import synth
from beamtest import check_routing_exact, check_y, gpu_routing_host, need_gpu, sample_tokens

pytestmark = pytest.mark.gpu


def _draw_cases(n, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        fp32 = rng.random() < 0.15
        d = int(rng.choice([64, 96, 160]) if fp32 else rng.choice([128, 256, 384, 512, 640]))
        E = int(rng.integers(2, 201))
        K = int(rng.integers(1, min(16, E) + 1))
        I = int(rng.choice([32, 48, 96] if fp32 else [64, 128, 192, 256, 320, 512]))
        S = int(rng.choice([0, 0, 0, 1, 2, 4]))
        if E + S > 256:
            continue
        T = int(rng.choice([1, 3, 17, 63, 64, 65, 129, 700, 1500, 3000]))
        tau = float(rng.choice([0.0, 0.0, 0.3, 0.8]))
        bias = float(rng.choice([-1.0, 0.0, 0.5]))
        tiled_ok = not fp32 and d % 256 == 0 and I % 128 == 0
        flags = int(rng.choice([0, 0, B.BEAM_FORCE_DECODE] +
                               ([B.BEAM_FORCE_PREFILL] if tiled_ok else [])))
        cases.append((d, E, K, I, S, T, tau, bias, flags, fp32))
    return cases


CASES = _draw_cases(24)


@pytest.mark.parametrize("d,E,K,I,S,T,tau,bias,flags,fp32", CASES,
                         ids=[f"d{c[0]}-E{c[1]}-K{c[2]}-I{c[3]}-S{c[4]}-T{c[5]}-tau{c[6]}"
                              f"-b{c[7]}-f{c[8]}{'-fp32' if c[9] else ''}" for c in CASES])
def test_random_shape(d, E, K, I, S, T, tau, bias, flags, fp32):
    need_gpu()
    shape = synth.LayerShape(d, E, K, I, torch.float32 if fp32 else torch.bfloat16)
    seed = 3000 + d + 7 * E + 13 * K + I + 17 * S + T
    L = synth.make_layer(shape, T, seed=seed, n_shared=S, mask_bias=bias, device="cuda")
    W_gu, W_dt = L["W_gu"], L["W_dt"]
    if S:
        W_gu = torch.cat([W_gu, L["Ws_gu"]]).contiguous()
        W_dt = torch.cat([W_dt, L["Ws_dt"]]).contiguous()
    lay = B.MoELayer(L["W_gate"], L["W_mask"], W_gu, W_dt, K, flags=flags, tau=tau)
    y, R = lay(L["x"])
    torch.cuda.synchronize()
    G = gpu_routing_host({k: v.cpu() for k, v in R.items()})
    O = check_routing_exact(G, K, lay.sizes["block_m"], tau if tau else 0.5, n_shared=S)
    if S:
        assert np.all(G["counts"][E:] == T)
    check_y(y.float().cpu().numpy(), L, K, O, 1e-5 if fp32 else 1e-2,
            tokens=sample_tokens(T, 24, seed=seed))


# Small decode batches (T <= 8 tokens, bf16): the three-launch path, whose
# every workgroup routes the batch itself (select over 1-16 experts per lane,
# E not a multiple of 16, shared experts) and whose down kernel deals its
# workgroups to the tokens by their slot counts (uniform or per-token mask
# biases).
def _draw_small_cases(n, seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        d = int(rng.choice([128, 256, 384, 640, 2048]))
        E = int(rng.integers(2, 257))
        K = int(rng.integers(1, min(16, E) + 1))
        S = int(rng.choice([0, 0, 1, 2, 4]))
        I = int(rng.choice([64, 128, 192, 320, 768]))
        T = int(rng.integers(1, 9))
        if E + S > 256 or (K + S) * I * 2 > 48 * 1024:
            continue
        skew = bool(rng.random() < 0.4) and d >= 2
        bias = float(rng.choice([-1.0, 0.0, 0.5]))
        cases.append((d, E, K, I, S, T, bias, skew))
    return cases


SMALL_CASES = _draw_small_cases(16)


@pytest.mark.parametrize("d,E,K,I,S,T,bias,skew", SMALL_CASES,
                         ids=[f"d{c[0]}-E{c[1]}-K{c[2]}-I{c[3]}-S{c[4]}-T{c[5]}-b{c[6]}"
                              f"{'-skew' if c[7] else ''}" for c in SMALL_CASES])
def test_random_small_batch(d, E, K, I, S, T, bias, skew):
    need_gpu()
    shape = synth.LayerShape(d, E, K, I, torch.bfloat16)
    seed = 5000 + d + 7 * E + 13 * K + I + 17 * S + T
    kw = {"skew": True} if skew else {"mask_bias": bias}
    L = synth.make_layer(shape, T, seed=seed, n_shared=S, device="cuda", **kw)
    W_gu, W_dt = L["W_gu"], L["W_dt"]
    if S:
        W_gu = torch.cat([W_gu, L["Ws_gu"]]).contiguous()
        W_dt = torch.cat([W_dt, L["Ws_dt"]]).contiguous()
    lay = B.MoELayer(L["W_gate"], L["W_mask"], W_gu, W_dt, K)
    y, R = lay(L["x"])
    torch.cuda.synchronize()
    G = gpu_routing_host({k: v.cpu() for k, v in R.items()})
    O = check_routing_exact(G, K, lay.sizes["block_m"], 0.5, n_shared=S)
    check_y(y.float().cpu().numpy(), L, K, O, 1e-2)
