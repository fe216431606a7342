"""Shared helpers for the GPU parity tests: run the HIP layer through the
C-ABI binding, and compare with the fp64 oracle."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import dynamic_expert_sparsity_amd as B
from dynamic_expert_sparsity_amd import synth

ROUTE_KEYS_EXACT = ["topk_ids", "mask", "masked_ids", "counts", "offsets", "active_experts",
                    "num_active"]


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")


class ExpertView:
    """Lazy per-expert float32 host copies of a device weight tensor."""

    def __init__(self, W):
        self.W = W

    def __getitem__(self, e):
        return self.W[e].float().cpu().numpy()


def host(t):
    return t.float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) else t.cpu().numpy()


def run(L, K, block_m=0, flags=0, tau=0.0, x=None):
    layer = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], K, block_m=block_m,
                       flags=flags, tau=tau)
    y, R = layer(L["x"] if x is None else x)
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in R.items()}
    return y.float().cpu().numpy(), out, layer


def gpu_routing_host(R):
    n = R["num_active"].numpy()
    return {
        "gate_logits": R["gate_logits"].numpy(), "mask_logits": R["mask_logits"].numpy(),
        "topk_ids": R["topk_ids"].numpy(), "topk_weights": R["topk_weights"].numpy(),
        "mask": R["mask"].numpy(), "g_hat": R["g_hat"].numpy(),
        "masked_ids": R["masked_ids"].numpy(), "counts": R["expert_counts"].numpy(),
        "offsets": R["expert_offsets"].numpy(),
        "sorted_pairs": R["sorted_pairs"].numpy()[:n[1]],
        "block_expert": R["block_expert"].numpy()[:n[3]],
        "active_experts": R["active_experts"].numpy()[:n[2]], "num_active": n,
    }


def check_routing_exact(G, K, block_m, tau=0.5, n_shared=0):
    """Every discrete routing output must equal the oracle's decisions on the
    GPU's own float32 logits, bit for bit; g and g_hat to float32 rounding."""
    O = oracle.route_from_logits(G["gate_logits"], G["mask_logits"], K, block_m, tau, n_shared)
    for k in ROUTE_KEYS_EXACT:
        if k == "num_active":
            want = np.array([O["num_active"][0], O["num_active"][1], len(O["active_experts"]),
                             len(O["block_expert"])])
        else:
            want = O[k]
        np.testing.assert_array_equal(G[k], want, err_msg=k)
    np.testing.assert_array_equal(G["sorted_pairs"], O["sorted_pairs"], err_msg="sorted_pairs")
    np.testing.assert_array_equal(G["block_expert"], O["block_expert"], err_msg="block_expert")
    np.testing.assert_allclose(G["topk_weights"], O["topk_weights"], rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(G["g_hat"], O["g_hat"], rtol=2e-6, atol=1e-7)
    return O


def check_logits(G, L, rel=1e-3):
    r, z = oracle.router_logits(host(L["x"]), host(L["W_gate"]), host(L["W_mask"]))
    for name, got, ref in (("gate", G["gate_logits"], r), ("mask", G["mask_logits"], z)):
        scale = max(np.abs(ref).max(), 1e-30)
        assert np.abs(got - ref).max() <= rel * scale, f"{name} logits max abs err"
        assert np.linalg.norm(got - ref) <= rel * max(np.linalg.norm(ref), 1e-30), f"{name} rel-L2"
    return r, z


def rel_l2(a, b):
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def check_y(y, L, K, O, tol, tokens=None):
    """y against the oracle's Eq. 8 on the same routing decisions (plus the
    shared experts when L has them).  The bound holds for the checked rows
    together (relative L2) and for every one of them alone; rows whose
    reference is exactly zero (no active slot, no shared expert) must be
    exactly zero."""
    rows = np.arange(y.shape[0]) if tokens is None else np.asarray(tokens)
    shared = None
    if "Ws_gu" in L and L["Ws_gu"].shape[0] > 0:
        n = L["Ws_gu"].shape[0]
        shared = ([L["Ws_gu"][s].float().cpu().numpy() for s in range(n)],
                  [L["Ws_dt"][s].float().cpu().numpy() for s in range(n)])
    ref = oracle.forward(host(L["x"]), None, None, ExpertView(L["W_gu"]), ExpertView(L["W_dt"]),
                         K, routing=O, tokens=rows, shared=shared)
    got = y[rows].astype(np.float64)
    err = rel_l2(got, ref)
    assert err <= tol, f"y rel-L2 {err:.3e} > {tol}"
    rn = np.linalg.norm(ref, axis=1)
    en = np.linalg.norm(got - ref, axis=1)
    live = rn > 0
    assert np.all(got[~live] == 0.0), "rows with a zero reference are not exactly zero"
    if live.any():
        per_row = en[live] / rn[live]
        worst = int(np.argmax(per_row))
        assert per_row[worst] <= tol, (f"row {int(rows[live][worst])}: rel-L2 "
                                       f"{per_row[worst]:.3e} > {tol}")
    if shared is None:
        # tokens with no active slot are exactly zero
        dead = rows[np.asarray(O["mask"])[rows].sum(axis=1) == 0]
        assert np.all(y[dead] == 0.0)
    return err


def decision_margins(r, z, K, thr=0.0):
    """Per token, the smallest gap between consecutive logits among the K + 1
    largest r (the Top-K set and its order are decided there, Eq. 4) and the
    smallest distance of a candidate's mask logit from the threshold (Eq. 6),
    both from float64 logits."""
    r = np.asarray(r, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    T, E = r.shape
    srt = -np.sort(-r, axis=1)[:, :min(K + 1, E)]
    gap = np.diff(-srt, axis=1).min(axis=1) if srt.shape[1] > 1 else np.full(T, np.inf)
    ids = np.argsort(-r, axis=1, kind="stable")[:, :K]
    zk = np.take_along_axis(z, ids, axis=1)
    zm = np.abs(zk - thr).min(axis=1)
    return gap, zm


def check_route_from_scratch(G, L, K, tau=0.5, margin=1e-4):
    """The GPU's decisions against routing from scratch (the oracle on float64
    logits of the exact inputs): ids and mask bits must agree on every token
    whose decision margins exceed margin * max|r| and margin * max|z|.
    Returns the number of tokens inside the margins (not compared)."""
    O = oracle.route(host(L["x"]), host(L["W_gate"]), host(L["W_mask"]), K, tau=tau)
    thr = oracle.mask_threshold_logit(tau)
    gap, zm = decision_margins(O["gate_logits"], O["mask_logits"], K, thr)
    near = (gap <= margin * np.abs(O["gate_logits"]).max()) | \
           (zm <= margin * np.abs(O["mask_logits"]).max())
    far = ~near
    np.testing.assert_array_equal(G["topk_ids"][far], O["topk_ids"][far], err_msg="topk_ids")
    np.testing.assert_array_equal(G["mask"][far], O["mask"][far], err_msg="mask")
    n_near = int(near.sum())
    print(f"[from-scratch routing] {int(far.sum())} tokens agree, {n_near} inside the "
          f"{margin:g} margins")
    return n_near


def keep_rate_bound(p, n):
    """Tolerance of a measured keep rate over n candidate slots around p."""
    return 4.0 * math.sqrt(p * (1.0 - p) / n) + 0.005


def mode_record(lay):
    """The call's kernel-family record {family, max count, records, layout} from
    the workspace (layout: tile token sets, tile bases, per-expert counts,
    pair positions, then the record, each piece rounded up to 256 bytes)."""
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731
    T, E2, K, S = lay.desc.T, lay.desc.E + lay.desc.n_shared, lay.desc.K, lay.desc.n_shared
    n_tiles = (T + 63) // 64
    off = al(n_tiles * E2 * 8) + al(n_tiles * E2 * 4) + al(E2 * 4) + al(T * (K + S) * 4)
    return lay.ws[off:off + 16].view(torch.int32).cpu().numpy()


def sample_tokens(T, n, seed=0):
    if T <= n:
        return np.arange(T)
    return np.sort(np.random.default_rng(seed).choice(T, n, replace=False))


def layer(shape, T, **kw):
    return synth.make_layer(shape, T, device="cuda", **kw)
