"""A stack of layers captured once in a HIP graph and replayed.

The layer needs no host round trip between its kernels (the kernel family,
the number of active experts and every list length are read on the device),
so a whole stack of layer calls can be captured and replayed.  Each replay
must give, bit for bit, what the same calls give eagerly; eager calls of the
same layers between replays (which overwrite the same buffers) must not
disturb the next replay; and the outputs must match the fp64 oracle's Eq. 8
on the GPU's routing decisions.
"""
import numpy as np
import pytest
import torch

import dynamic_expert_sparsity_amd as B
from dynamic_expert_sparsity_amd import synth
from beamtest import check_routing_exact, check_y, gpu_routing_host, need_gpu, sample_tokens

pytestmark = pytest.mark.gpu


def _stack(shape, Ts, seed):
    """Distinct layers; layer i gets Ts[i] tokens of the skewed recipe."""
    out = []
    for i, T in enumerate(Ts):
        L = synth.make_layer(shape, T, seed=seed, layer=i, skew=True, device="cuda")
        lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], shape.K)
        lay.prepare(T)
        out.append((lay, L))
    return out


def _snapshot(stack):
    res = []
    for lay, _ in stack:
        n = lay.routing["num_active"].clone()
        res.append((lay.y.clone(), lay.routing["masked_ids"].clone(),
                    lay.routing["g_hat"].clone(), n))
    return res


def _same(a, b):
    return all(torch.equal(x, y) for p, q in zip(a, b) for x, y in zip(p, q))


@pytest.mark.parametrize("shape,Ts", [
    # small layers: ring kernels (d, I multiples of 256), decode, a batch
    # large enough for the per-call choice between the kernel families, and
    # one of more than 16 select tiles (grouping with separate pair scatter)
    (synth.LayerShape(512, 32, 4, 256, torch.bfloat16), [1, 64, 64, 700, 33, 3000]),
    # the Qwen3-shaped layer at decode sizes
    ("qwen3", [64, 64, 256]),
])
def test_graph_replay_matches_eager(shape, Ts):
    need_gpu()
    if isinstance(shape, str):
        shape = synth.SHAPES[shape]
    stack = _stack(shape, Ts, seed=2100 + len(Ts))

    def step():
        for lay, L in stack:
            lay(L["x"])

    step()
    torch.cuda.synchronize()
    eager = _snapshot(stack)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert _same(_snapshot(stack), eager), f"replay {rep} differs from the eager step"
        # eager work on the same buffers between replays: another batch
        lay0, L0 = stack[0]
        x_other = synth.make_tokens(shape, Ts[0], seed=77, layer=rep, device="cuda")
        lay0(x_other)
        torch.cuda.synchronize()

    # the replayed outputs against the oracle, on the GPU's routing decisions
    g.replay()
    torch.cuda.synchronize()
    for (lay, L), T in zip(stack, Ts):
        G = gpu_routing_host({k: v.cpu() for k, v in lay.routing.items()})
        O = check_routing_exact(G, shape.K, lay.sizes["block_m"])
        y = lay.y.float().cpu().numpy()
        check_y(y, L, shape.K, O, 1e-2, tokens=sample_tokens(T, 48, seed=T))
    del g


def test_graph_replay_with_new_inputs():
    """Inputs copied into the captured buffers before a replay are routed
    afresh: the replay equals an eager call on the new tokens."""
    need_gpu()
    shape = synth.SHAPES["qwen3"]
    T = 32
    L = synth.make_layer(shape, T, seed=2200, mask_bias=-1.04, device="cuda")
    lay = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], shape.K)
    x_buf = L["x"].clone()
    lay(x_buf)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lay(x_buf)
    ref = B.MoELayer(L["W_gate"], L["W_mask"], L["W_gu"], L["W_dt"], shape.K)
    for rep in range(3):
        x_new = synth.make_tokens(shape, T, seed=2201, layer=rep, device="cuda")
        x_buf.copy_(x_new)
        g.replay()
        y_ref, R_ref = ref(x_new)
        torch.cuda.synchronize()
        assert torch.equal(lay.y, y_ref), f"replay {rep}"
        assert torch.equal(lay.routing["masked_ids"], R_ref["masked_ids"])
        counts = np.asarray(lay.routing["expert_counts"].cpu())
        assert counts.sum() == int(lay.routing["num_active"][0].item())
    del g
