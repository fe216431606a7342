"""GPU parity at the full Qwen3-30B-A3B-shaped layer (d=2048, E=128, K=8,
I=768, bf16), one batch per kernel family the device picks, EVERY output row
checked against the fp64 oracle:

  * streaming kernels: decode, T = 256, mask bias b = -1.04 (keep ~0.15);
  * 128-row tiles: prefill, T = 2048, b = 0 (keep 0.5, ~64 pairs per expert);
  * 256-row tiles: prefill, T = 8192, b = +8 (keep 1.0, ~512 pairs per expert);
  * the skewed load: T = 16384, Zipf expert popularity, per-token mask biases.

For each: router logits within 1e-3 of the float64 logits (paper section 3.2
Eq. 4-5); every discrete routing output bit-exact against the oracle on the
GPU's own logits (Eq. 4-7, the grouping of the news article's section 5); y
within relative L2 1e-2 for the whole batch and for every row alone (Eq. 3,
Eq. 8); and the routing from scratch (the oracle on float64 logits) agreeing
on every token whose decision margins exceed 1e-4 of the largest logit.

The keep rate: with x_0 = 1 and x_1.. ~ N(0, 1), a mask logit is exactly
Gaussian, z = b + N(0, s_e^2) with s_e the norm of expert e's mask row past
channel 0, so over all (token, expert) pairs P(z >= 0) = mean_e Phi(b / s_e),
and over the Top-K candidates (chosen by an independent router) ~ Phi(b).
"""
import math

import numpy as np
import pytest

from beamtest import (check_logits, check_route_from_scratch, check_routing_exact, check_y,
                      gpu_routing_host, host, keep_rate_bound, layer, mode_record, need_gpu, run)

pytestmark = pytest.mark.gpu

K = 8


@pytest.mark.parametrize("T,b,skew,family", [
    (256, -1.04, False, 0),
    (2048, 0.0, False, 1),
    (8192, 8.0, False, 2),
    (16384, None, True, None),
])
def test_full_size_every_row(T, b, skew, family):
    need_gpu()
    kw = {"skew": True} if skew else {"mask_bias": b}
    L = layer("qwen3", T, seed=3000 + T, **kw)
    y, R, lay = run(L, K)
    G = gpu_routing_host(R)
    check_logits(G, L)
    O = check_routing_exact(G, K, lay.sizes["block_m"])
    rec = mode_record(lay)
    print(f"[full size] T={T} {'skew' if skew else f'b={b:+g}'}: kernel family {rec[0]}, "
          f"layout {rec[3]}, active pairs {int(G['num_active'][0])}")
    if family is not None:
        assert rec[0] == family, "the inputs did not land on the intended kernel family"
    else:
        assert rec[0] in (1, 2)
    check_y(y, L, K, O, 1e-2)
    n_near = check_route_from_scratch(G, L, K)
    assert n_near <= T // 10 + 2  # ~4% of tokens on random logits


def _phi(v):
    return 0.5 * (1.0 + math.erf(v / math.sqrt(2.0)))


@pytest.mark.parametrize("b", [-1.04, 0.0])
def test_keep_rate_matches_phi(b):
    need_gpu()
    T = 8192
    L = layer("qwen3", T, seed=3100, mask_bias=b)
    y, R, lay = run(L, K)
    G = gpu_routing_host(R)
    check_routing_exact(G, K, lay.sizes["block_m"])
    Wm = host(L["W_mask"]).astype(np.float64)
    bb = Wm[:, 0]                       # the bias as stored (bf16-rounded)
    s = np.linalg.norm(Wm[:, 1:], axis=1)
    # over the candidate slots (the pages' statistic): ~ Phi(b)
    p = float(np.mean([_phi(v) for v in bb]))
    keep = float(G["mask"].mean())
    tol = keep_rate_bound(p, T * K)
    print(f"[keep rate] b={b:+g}: candidates {keep:.4f} vs Phi(b) {p:.4f} (tolerance {tol:.4f})")
    assert abs(keep - p) <= tol
    # over all (token, expert) pairs: the exact closed form mean_e Phi(b_e / s_e)
    p_all = float(np.mean([_phi(u / v) for u, v in zip(bb, s)]))
    keep_all = float((G["mask_logits"] >= 0).mean())
    tol_all = keep_rate_bound(p_all, T * Wm.shape[0])
    print(f"[keep rate] b={b:+g}: all pairs {keep_all:.4f} vs closed form {p_all:.4f}")
    assert abs(keep_all - p_all) <= tol_all
    # the count the grouping schedules is the mask's count
    assert int(G["num_active"][0]) == int(G["mask"].sum())
