"""fp64 CPU oracle for the BEAM masked-MoE layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library; it receives plain arrays and returns plain
arrays.

Source of truth: "BEAM: Binary Expert Activation Masking for Dynamic Routing
in MoE" (arXiv 2605.14438), section 3.1 (Eq. 1-3) and section 3.2 (Eq. 4-8),
and the news article on the same paper, section 5 ("from theory to practice"),
which describes the two modified kernels (masked expert ids become -1; the
expert/token grouping leaves -1 out of its counts).

Everything here is plain, slow and obviously correct:
  * all floating point is float64 on the exact input values (bf16 and fp32
    inputs upcast exactly);
  * one library primitive per step (a matmul, a lexsort), no blocking, no
    fusion, no reordering beyond what the equations state.

Readings of points the pages leave open:
  R1  no router biases: r = x W_gate^T, z = x W_mask^T (weights stored
      [E, d], one row per expert, i.e. the transpose of the paper's
      W_m in R^{d_h x N});
  R2  the GLU activation of Eq. 3 is SiLU (SwiGLU);
  R4  Top-K selects on the logits r, then the softmax runs over the K kept
      values (Eq. 4: the other entries are -inf, so they get weight 0);
  R5  Top-K order and ties: slots are in descending logit order, equal logits
      go to the lower expert index first;
  R6  the binary mask of Eq. 6 (sigmoid(z) >= 0.5) is evaluated exactly as
      z >= 0 (sigmoid is strictly increasing with sigmoid(0) = 1/2); z = -0.0
      counts as >= 0;
  R7  no renormalisation after the mask (Eq. 7);
  R8  no minimum number of active experts: a token whose K slots are all
      masked gets y = 0 (the residual path, outside this layer, carries it);
  R9  z is computed for all N experts, the mask is applied only at the K
      candidates;
  R12 compaction order is unique: per expert, flat pair ids t*K+k ascending;
      per-expert segments padded with the value T*K to a multiple of block_m.
  T1  (threshold variants, the ablation over tau in the news article section
      8) tau != 0.5 is evaluated as z >= ln(tau / (1 - tau)), the exact
      preimage of sigmoid >= tau.
  B1  (training, paper section 3.3 and news article section 4) the
      binarisation m = [m_hat >= 0.5] is passed by the straight-through
      estimator: dL/dm_hat = dL/dm; the sparsity term is
      L_sp = beta * sum_t sum_k m_hat[t, id_k] over the K candidates of every
      token (a plain sum; any normalisation is folded into beta); dL/dm
      follows from Eq. 7-8 as g_k * dL/dg_hat_k.
  S1  (shared experts, news article sections 5 and 6: models with always-on
      shared experts keep running them for a token whose routed slots are
      all masked) a shared expert is a SwiGLU expert of the routed experts'
      shape, applied to every token with weight 1 and no mask, and added to
      the routed sum of Eq. 8.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "router_logits",
    "topk_select",
    "topk_softmax",
    "binary_mask",
    "mask_threshold_logit",
    "aggregate",
    "compact",
    "route",
    "route_from_logits",
    "swiglu_expert",
    "forward",
    "routing_stats",
    "mask_backward",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Step 1 / Step 2 logits (Eq. 4 r = R(x); Eq. 5 the argument of sigmoid)
# ---------------------------------------------------------------------------
def router_logits(x, W_gate, W_mask):
    """Main-router logits r and mask-router logits z, both [T, E] float64.

    Paper section 3.1: r = R(x), a linear router; Eq. 5: m_hat = sigmoid(x W_m).
    Weights are stored one row per expert ([E, d]); r[t, e] = <x_t, W_gate[e]>.
    """
    x64 = _f64(x)
    r = x64 @ _f64(W_gate).T
    z = x64 @ _f64(W_mask).T
    return r, z


# ---------------------------------------------------------------------------
# Top-K (Eq. 1 / Eq. 4)
# ---------------------------------------------------------------------------
def topk_select(r, K: int) -> np.ndarray:
    """Indices of the K largest logits per token, [T, K] int64.

    Eq. 4 keeps the K largest entries of r.  Order key (reading R5): value
    descending, then expert index ascending.  np.lexsort sorts by its last key
    first, so keys are (index, -value).
    """
    r = _f64(r)
    T, E = r.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    idx = np.arange(E)
    out = np.empty((T, K), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((idx, -r[t]))
        out[t] = order[:K]
    return out


def topk_softmax(r, ids) -> np.ndarray:
    """Routing weights g over the K kept experts, [T, K] float64.

    Eq. 4: g = Softmax(Top-K(r)); the dropped entries are -inf so only the K
    kept logits enter the normaliser.  Shifted by the largest kept logit for
    range safety (exact in real arithmetic).
    """
    r = _f64(r)
    kept = np.take_along_axis(r, np.asarray(ids), axis=1)
    shift = kept.max(axis=1, keepdims=True)
    w = np.exp(kept - shift)
    return w / w.sum(axis=1, keepdims=True)


def mask_threshold_logit(tau: float = 0.5) -> float:
    """Logit threshold equivalent to sigmoid(z) >= tau (Eq. 6 uses tau = 0.5)."""
    if not 0.0 < tau < 1.0:
        raise ValueError("tau must lie in (0, 1)")
    if tau == 0.5:
        return 0.0
    return math.log(tau / (1.0 - tau))


def binary_mask(z, ids, tau: float = 0.5) -> np.ndarray:
    """Binary mask m at the K candidates, [T, K] uint8.

    Eq. 6: m_i = 1 iff sigmoid(z_i) >= tau (tau = 0.5).  Evaluated exactly on
    the logit (reading R6): z >= logit(tau), which is z >= 0 at tau = 0.5.
    Eq. 7 only uses m at the Top-K candidates (reading R9).
    """
    zk = np.take_along_axis(_f64(z), np.asarray(ids), axis=1)
    return (zk >= mask_threshold_logit(tau)).astype(np.uint8)


def aggregate(g, m) -> np.ndarray:
    """Eq. 7: g_hat = g * m, with no renormalisation (reading R7)."""
    return _f64(g) * np.asarray(m, dtype=np.float64)


# ---------------------------------------------------------------------------
# Grouping of (token, expert) pairs (news article, section 5: ids of masked
# experts become -1 and are left out of the per-expert counts)
# ---------------------------------------------------------------------------
def compact(masked_ids, E: int, block_m: int, n_shared: int = 0) -> dict:
    """Per-expert counts, block-padded offsets and sorted pair lists.

    masked_ids: [T, K] with -1 for masked slots.  A routed pair is
    p = t*K + k.  With n_shared = S always-on shared experts (the pages'
    DeepSeek and Qwen1.5-MoE models; reading S1), expert E + s also receives
    every token t as the pair p = T*K + t*S + s.
    Returns int64 arrays over the E + S experts:
      counts[E+S]        pairs routed to each expert (-1 excluded)
      offsets[E+S+1]     exclusive prefix sum of counts rounded up to block_m
      sorted_pairs[num_padded]  per expert, its pair ids ascending, then the
                         pad value T*(K+S) up to the next multiple of block_m
      block_expert[num_padded // block_m]   expert owning each block
      active_experts[n]  experts with count >= 1, ascending
      num_active         (P, num_padded), P = all scheduled pairs
    """
    mi = np.asarray(masked_ids)
    T, K = mi.shape
    S = int(n_shared)
    E2 = E + S
    pad = T * (K + S)
    flat = mi.reshape(-1)
    counts = np.zeros(E2, dtype=np.int64)
    lists = [[] for _ in range(E2)]
    for p in range(T * K):          # ascending pair id -> lists come out sorted
        e = int(flat[p])
        if e < 0:
            continue
        counts[e] += 1
        lists[e].append(p)
    for t in range(T):              # shared pairs, ascending in t for each s
        for s in range(S):
            counts[E + s] += 1
            lists[E + s].append(T * K + t * S + s)
    offsets = np.zeros(E2 + 1, dtype=np.int64)
    for e in range(E2):
        padded = -(-int(counts[e]) // block_m) * block_m
        offsets[e + 1] = offsets[e] + padded
    num_padded = int(offsets[E2])
    sorted_pairs = np.full(num_padded, pad, dtype=np.int64)
    block_expert = np.empty(num_padded // block_m, dtype=np.int64)
    for e in range(E2):
        o = int(offsets[e])
        sorted_pairs[o:o + len(lists[e])] = lists[e]
        block_expert[o // block_m:int(offsets[e + 1]) // block_m] = e
    active = np.array([e for e in range(E2) if counts[e] > 0], dtype=np.int64)
    return {
        "counts": counts,
        "offsets": offsets,
        "sorted_pairs": sorted_pairs,
        "block_expert": block_expert,
        "active_experts": active,
        "num_active": np.array([int(counts.sum()), num_padded], dtype=np.int64),
    }


def route_from_logits(r, z, K: int, block_m: int = 16, tau: float = 0.5,
                      n_shared: int = 0) -> dict:
    """Steps 1-4 of section 3.2 plus the grouping, starting from given logits.

    Used with the GPU's float32 logits so that every discrete output (ids,
    mask, masked ids, counts, lists) must agree bit for bit: the float32
    values are upcast exactly and compared exactly.
    """
    r = _f64(r)
    z = _f64(z)
    E = r.shape[1]
    ids = topk_select(r, K)
    g = topk_softmax(r, ids)
    m = binary_mask(z, ids, tau)
    g_hat = aggregate(g, m)
    masked_ids = np.where(m == 1, ids, -1)
    out = {
        "gate_logits": r,
        "mask_logits": z,
        "topk_ids": ids,
        "topk_weights": g,
        "mask": m,
        "g_hat": g_hat,
        "masked_ids": masked_ids,
    }
    out.update(compact(masked_ids, E, block_m, n_shared))
    return out


def route(x, W_gate, W_mask, K: int, block_m: int = 16, tau: float = 0.5,
          n_shared: int = 0) -> dict:
    """Routing from scratch: Eq. 4-7 on fp64 logits, then the grouping."""
    r, z = router_logits(x, W_gate, W_mask)
    return route_from_logits(r, z, K, block_m, tau, n_shared)


# ---------------------------------------------------------------------------
# Routing statistics (the paper's analyses of the learned mask: how often the
# slot of each rank is masked, how many experts a token keeps, the load of
# each expert; news article section 7)
# ---------------------------------------------------------------------------
def routing_stats(mask, masked_ids, E: int) -> dict:
    """Counts over one routing, by plain loops over the tokens.

    mask [T, K] in {0, 1}; slot k holds the expert of the k-th largest router
    logit (reading R5), so "rank k" is slot k.  Returns int64 arrays:
      rank_masked[K]   tokens whose rank-k slot is masked
      active_hist[K+1] tokens with exactly j active slots, j = 0..K
      expert_load[E]   active pairs of each expert (masked ids -1 excluded,
                       as in the grouping)
    The mask probability of rank k is rank_masked[k] / T; the mean number of
    active experts per token is sum_j j * active_hist[j] / T.
    """
    m = np.asarray(mask)
    mi = np.asarray(masked_ids)
    T, K = m.shape
    rank_masked = np.zeros(K, dtype=np.int64)
    active_hist = np.zeros(K + 1, dtype=np.int64)
    expert_load = np.zeros(E, dtype=np.int64)
    for t in range(T):
        n_active = 0
        for k in range(K):
            if m[t, k]:
                n_active += 1
                expert_load[int(mi[t, k])] += 1
            else:
                rank_masked[k] += 1
        active_hist[n_active] += 1
    return {"rank_masked": rank_masked, "active_hist": active_hist,
            "expert_load": expert_load}


# ---------------------------------------------------------------------------
# Experts (Eq. 3) and the masked weighted sum (Eq. 8)
# ---------------------------------------------------------------------------
def _silu(a):
    # SiLU(a) = a * sigmoid(a) (reading R2); written as a / (1 + exp(-a)).
    return a / (1.0 + np.exp(-a))


def swiglu_expert(xs, Wg, Wu, Wd):
    """Eq. 3: E(x) = (SiLU(x W_gate) * (x W_up)) W_down, for rows xs [n, d].

    Storage: Wg, Wu [I, d] (one row per intermediate unit), Wd [d, I]
    (one row per output channel), so x W_gate = xs @ Wg^T.
    """
    xs = _f64(xs)
    a = xs @ _f64(Wg).T
    u = xs @ _f64(Wu).T
    h = _silu(a) * u
    return h @ _f64(Wd).T


def forward(x, W_gate, W_mask, W_gu, W_dt, K: int, routing: dict | None = None,
            tokens=None, tau: float = 0.5, shared=None):
    """Masked-MoE layer output y, [T or len(tokens), d] float64 (Eq. 8).

    x        [T, d]
    W_gate   [E, d], W_mask [E, d]
    W_gu     indexable by expert: W_gu[e] is [2I, d]; rows 0..I-1 are the
             gate projection, rows I..2I-1 the up projection (Eq. 3)
    W_dt     indexable by expert: W_dt[e] is [d, I] (down projection)
    routing  optional dict with "topk_ids", "mask" and "g_hat" (e.g. from
             route_from_logits on the GPU's logits); computed from scratch
             with route() when None.
    tokens   optional subset of token indices; y is returned for those rows
             only (the layer is per token, Eq. 8).
    shared   optional (Ws_gu, Ws_dt), each indexable by shared expert s like
             W_gu / W_dt: always-on experts added with weight 1 and never
             masked (reading S1), so a token whose K slots are all masked
             still gets their output.

    y_t = sum_k g_hat[t,k] * E_{ids[t,k]}(x_t) over the slots with m = 1, in
    slot order, after the shared experts' sum (if any); without shared
    experts y_t = 0 when no slot survives (reading R8).  Experts are
    visited one at a time and only for the tokens routed to them; each
    expert's weights are upcast to float64 when it is visited.
    """
    x64 = _f64(x)
    T, d = x64.shape
    if routing is None:
        routing = route(x, W_gate, W_mask, K, tau=tau)
    ids = np.asarray(routing["topk_ids"])
    m = np.asarray(routing["mask"])
    g_hat = _f64(routing["g_hat"])
    rows = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)

    # expert e -> list of (row in output, token, slot) with an active mask bit
    work: dict[int, list[tuple[int, int, int]]] = {}
    for i, t in enumerate(rows):
        for k in range(ids.shape[1]):
            if m[t, k]:
                work.setdefault(int(ids[t, k]), []).append((i, int(t), k))

    # per-slot outputs, then the slot-ordered sum of Eq. 8
    contrib = np.zeros((len(rows), ids.shape[1], d), dtype=np.float64)
    for e in sorted(work):
        items = work[e]
        gu = _f64(W_gu[e])
        I = gu.shape[0] // 2
        o = swiglu_expert(x64[[t for _, t, _ in items]], gu[:I], gu[I:], W_dt[e])
        for j, (i, t, k) in enumerate(items):
            contrib[i, k] = g_hat[t, k] * o[j]
    y = np.zeros((len(rows), d), dtype=np.float64)
    if shared is not None:
        Ws_gu, Ws_dt = shared
        for s in range(len(Ws_gu)):
            gu = _f64(Ws_gu[s])
            I = gu.shape[0] // 2
            y += swiglu_expert(x64[rows], gu[:I], gu[I:], Ws_dt[s])
    for k in range(ids.shape[1]):
        y += contrib[:, k]
    return y


# ---------------------------------------------------------------------------
# Mask-router backward: straight-through estimator and sparsity gradient
# (paper section 3.3, "straight-through estimation"; news article section 4)
# ---------------------------------------------------------------------------
def mask_backward(x, W_mask, ids, g, m, z, slot_grad, beta: float) -> dict:
    """Gradients of the mask router for one layer call (reading B1).

    x [T, d], W_mask [E, d]; ids, g, m [T, K]: the forward's Top-K ids, the
    softmax weights g and the hard mask m; z [T, E]: mask logits;
    slot_grad [T, K]: dL/dg_hat (for y = sum_k g_hat_k E_k(x), this is
    <dL/dy, E_{id_k}(x)>, also for masked slots).  Returns float64:
      dz [T, E]        dL/dz: (g_k * slot_grad_k + beta) * s (1 - s) at each
                       candidate id_k, s = sigmoid(z); 0 elsewhere
      dW_mask [E, d]   dz^T x
      dx [T, d]        dz W_mask (the mask router's share of dL/dx)
      d_gate [T, E]    dL/dr through the softmax over the kept logits (Eq. 4)
                       with dL/dg_k = m_k * slot_grad_k; 0 off the Top-K
    """
    x = _f64(x)
    W = _f64(W_mask)
    ids = np.asarray(ids)
    g = _f64(g)
    m = _f64(m)
    z = _f64(z)
    sg = _f64(slot_grad)
    T, K = ids.shape
    E = W.shape[0]
    dz = np.zeros((T, E))
    d_gate = np.zeros((T, E))
    for t in range(T):
        dg = m[t] * sg[t]                       # dL/dg_k through g_hat = g * m
        inner = float(np.dot(g[t], dg))
        for k in range(K):
            e = int(ids[t, k])
            s = 1.0 / (1.0 + math.exp(-z[t, e]))
            dm_hat = g[t, k] * sg[t, k] + beta  # STE: dL/dm_hat = dL/dm, plus L_sp
            dz[t, e] += dm_hat * s * (1.0 - s)
            d_gate[t, e] += g[t, k] * (dg[k] - inner)   # softmax Jacobian
    return {"dz": dz, "dW_mask": dz.T @ x, "dx": dz @ W, "d_gate": d_gate}
