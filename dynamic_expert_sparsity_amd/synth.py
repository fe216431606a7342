"""Seeded synthetic inputs for the BEAM masked-MoE layer.

This module only draws random tensors in a fixed recipe.  It holds none of the
layer's arithmetic (no routing, masking, activation or sum), and both the GPU
path's tests and the fp64 oracle receive the tensors it returns.

Recipe (the same for every shape; the paper evaluates Qwen3-30B-A3B-shaped
layers, E=128 experts, top-8, no shared experts, at learned keep rates; these
draws stand in for the trained weights, the SFT data and the serving trace,
none of which are used):

  x       [T, d]    N(0, 1), channel 0 fixed at 1.0 (carries per-expert biases)
  W_gate  [E, d]    N(0, 1/d)
  W_mask  [E, d]    N(0, 1/d), column 0 (input channel 0) set to the mask bias b;
                    mask_mode="zero" gives the all-zero mask router of the
                    paper's initialisation (every mask bit 1)
  W_gu    [E, 2I, d] N(0, 1/d); rows 0..I-1 gate projection, I..2I-1 up
  W_dt    [E, d, I]  N(0, 1/I)  (down projection, one row per output channel)

Skewed load ("skew=True"): W_gate[:, 0] = 0.5 * ln p_rank(e) with
p_r = r^-1.1 / sum_{j<=E} j^-1.1 and rank(e) a seeded permutation of 1..E;
W_mask[:, 0] = 0; input channel 1 carries a per-token mask bias b_t
(W_mask[:, 1] = 1, W_gate[:, 1] = 0): +1 for 50% of the tokens, -2 for 40%,
-8 for 10%, assigned by a seeded permutation.

Shared experts (n_shared > 0) are drawn like routed experts, from their own
streams.

Every tensor comes from its own torch.Generator seeded from
(seed, layer, tensor id, expert), drawn in float32 in storage order and then
rounded to the storage dtype (bfloat16: round to nearest even).  Draws on
"cuda" and on "cpu" use different generators and give different values; every
consumer receives the tensors themselves, never a regenerated copy.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

__all__ = ["LayerShape", "SHAPES", "N_SHARED", "make_layer", "make_router", "make_tokens", "with_mask_bias",
           "workload_name"]


@dataclass(frozen=True)
class LayerShape:
    d: int
    E: int
    K: int
    I: int
    dtype: torch.dtype


SHAPES = {
    # tiny correctness shape, float32 throughout
    "tiny": LayerShape(64, 8, 2, 128, torch.float32),
    # Qwen3-30B-A3B-shaped layer: d=2048, 128 experts, top-8, intermediate 768
    "qwen3": LayerShape(2048, 128, 8, 768, torch.bfloat16),
    # larger layer: d=4096, 128 experts, top-8, intermediate 1536
    "large": LayerShape(4096, 128, 8, 1536, torch.bfloat16),
    # DeepSeekV2-Lite-shaped layer: 64 routed experts, top-6, 2 shared experts
    "dsv2lite": LayerShape(2048, 64, 6, 1408, torch.bfloat16),
    # Qwen1.5-MoE-A2.7B-shaped layer: 60 routed experts, top-4, 4 shared experts
    "qwen15": LayerShape(2048, 60, 4, 1408, torch.bfloat16),
}

# shared (always-on) experts of each shape
N_SHARED = {"tiny": 0, "qwen3": 0, "large": 0, "dsv2lite": 2, "qwen15": 4}

_TID = {"x": 1, "W_gate": 2, "W_mask": 3, "W_gu": 4, "W_dt": 5, "perm": 6,
        "tokperm": 7, "Ws_gu": 8, "Ws_dt": 9}


def _gen(device, seed: int, layer: int, tid: int, expert: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    s = (((seed * 1_000_003 + layer) * 1_009 + tid) * 4_099 + expert) % (2**62)
    g.manual_seed(s)
    return g


def _randn(shape, std, dtype, device, gen) -> torch.Tensor:
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def make_router(shape: LayerShape | str, T: int, *, seed: int = 0, layer: int = 0,
                mask_bias: float = 0.0, mask_mode: str = "bias", skew: bool = False,
                device="cpu") -> dict:
    """Return dict(x, W_gate, W_mask): make_layer's tokens and routers alone
    (the same values make_layer gives for the same arguments)."""
    if isinstance(shape, str):
        shape = SHAPES[shape]
    d, E, dt = shape.d, shape.E, shape.dtype
    dev = torch.device(device)

    x = _randn((T, d), 1.0, torch.float32, dev, _gen(dev, seed, layer, _TID["x"]))
    if T > 0:
        x[:, 0] = 1.0
    W_gate = _randn((E, d), 1.0 / math.sqrt(d), torch.float32, dev,
                    _gen(dev, seed, layer, _TID["W_gate"]))
    if mask_mode == "zero":
        W_mask = torch.zeros((E, d), dtype=torch.float32, device=dev)
    elif mask_mode == "bias":
        W_mask = _randn((E, d), 1.0 / math.sqrt(d), torch.float32, dev,
                        _gen(dev, seed, layer, _TID["W_mask"]))
        W_mask[:, 0] = float(mask_bias)
    else:
        raise ValueError(f"unknown mask_mode {mask_mode!r}")

    if skew:
        if d < 2:
            raise ValueError("skewed recipe needs d >= 2")
        cpu = torch.device("cpu")
        ranks = torch.randperm(E, generator=_gen(cpu, seed, layer, _TID["perm"])) + 1
        w = torch.arange(1, E + 1, dtype=torch.float64) ** -1.1
        p = w / w.sum()
        W_gate[:, 0] = (0.5 * torch.log(p[ranks - 1])).to(torch.float32).to(dev)
        W_gate[:, 1] = 0.0
        if mask_mode == "bias":
            W_mask[:, 0] = 0.0
            W_mask[:, 1] = 1.0
        n_pos = (T * 5) // 10
        n_fun = (T * 4) // 10
        bt = torch.full((T,), -8.0, dtype=torch.float32)
        perm = torch.randperm(T, generator=_gen(cpu, seed, layer, _TID["tokperm"]))
        bt[perm[:n_pos]] = 1.0
        bt[perm[n_pos:n_pos + n_fun]] = -2.0
        if T > 0:
            x[:, 1] = bt.to(dev)
    return {"x": x.to(dt), "W_gate": W_gate.to(dt), "W_mask": W_mask.to(dt)}


def make_layer(shape: LayerShape | str, T: int, *, seed: int = 0, layer: int = 0,
               mask_bias: float = 0.0, mask_mode: str = "bias", skew: bool = False,
               n_shared: int = 0, device="cpu") -> dict:
    """Return dict(x, W_gate, W_mask, W_gu, W_dt[, Ws_gu, Ws_dt]) of torch tensors.

    mask_mode: "bias" (column 0 of W_mask = mask_bias) or "zero" (W_mask = 0).
    """
    if isinstance(shape, str):
        shape = SHAPES[shape]
    d, E, I, dt = shape.d, shape.E, shape.I, shape.dtype
    dev = torch.device(device)
    out = make_router(shape, T, seed=seed, layer=layer, mask_bias=mask_bias,
                      mask_mode=mask_mode, skew=skew, device=dev)

    W_gu = torch.empty((E, 2 * I, d), dtype=dt, device=dev)
    W_dt = torch.empty((E, d, I), dtype=dt, device=dev)
    for e in range(E):
        W_gu[e] = _randn((2 * I, d), 1.0 / math.sqrt(d), dt, dev,
                         _gen(dev, seed, layer, _TID["W_gu"], e))
        W_dt[e] = _randn((d, I), 1.0 / math.sqrt(I), dt, dev,
                         _gen(dev, seed, layer, _TID["W_dt"], e))
    out["W_gu"] = W_gu
    out["W_dt"] = W_dt
    if n_shared > 0:
        Ws_gu = torch.empty((n_shared, 2 * I, d), dtype=dt, device=dev)
        Ws_dt = torch.empty((n_shared, d, I), dtype=dt, device=dev)
        for s in range(n_shared):
            Ws_gu[s] = _randn((2 * I, d), 1.0 / math.sqrt(d), dt, dev,
                              _gen(dev, seed, layer, _TID["Ws_gu"], s))
            Ws_dt[s] = _randn((d, I), 1.0 / math.sqrt(I), dt, dev,
                              _gen(dev, seed, layer, _TID["Ws_dt"], s))
        out["Ws_gu"] = Ws_gu
        out["Ws_dt"] = Ws_dt
    return out


def make_tokens(shape: LayerShape | str, T: int, *, seed: int = 0, layer: int = 0,
                device="cpu") -> torch.Tensor:
    """x [T, d] of make_layer's recipe (N(0,1), channel 0 = 1) on its own stream."""
    if isinstance(shape, str):
        shape = SHAPES[shape]
    dev = torch.device(device)
    x = _randn((T, shape.d), 1.0, torch.float32, dev, _gen(dev, seed, layer, _TID["x"], 1))
    if T > 0:
        x[:, 0] = 1.0
    return x.to(shape.dtype)


def with_mask_bias(W_mask: torch.Tensor, b: float) -> torch.Tensor:
    """A copy of W_mask with its input-channel-0 column set to the bias b."""
    out = W_mask.clone()
    out[:, 0] = float(b)
    return out


def workload_name(shape_name: str, T: int, *, mask_bias=None, mask_mode="bias",
                  skew=False) -> str:
    s = SHAPES[shape_name]
    dt = "f32" if s.dtype == torch.float32 else "bf16"
    if skew:
        m = "skew"
    elif mask_mode == "zero":
        m = "allones"
    else:
        m = f"b{mask_bias:+g}"
    return f"d{s.d}-E{s.E}-K{s.K}-I{s.I}-{dt}-T{T}-{m}"
