#!/usr/bin/env python3
"""Benchmark of the BEAM masked-MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one call of the whole layer (router logits, Top-K/softmax/mask,
compaction, expert up and down projections on the active pairs, combine) on
one batch of T tokens, with the inputs already resident in HBM.  The headline
workload is the Qwen3-30B-A3B-shaped layer (d=2048, E=128 experts, top-8,
I=768, bf16) at decode, T=256 tokens, mask bias b=-1.04 (expected keep rate
Phi(-1.04) = 0.149, the paper's ~85% FLOP cut).  Steps rotate over several
independently drawn weight sets (as the layers of a model would) so that the
256 MB infinity cache cannot serve repeated weights.

Printed on one JSON line: tokens/s (value), ms per step, per-call HIP-event
durations (median, p10, p90), the HBM roofline of the dominant kernel
(per-stage HIP events recorded on the launch stream inside the timed steps),
the whole-layer HBM fraction, this GPU's measured copy/read bandwidth and
bf16 MFMA rate, the same kernels with the mask forced all-ones (W_mask = 0,
plain Top-K), a sweep over the decode batch sizes, the prefill runs (keep
0.15 / 0.3 / 0.5 / 1.0 at T = 2048 and 8192, and the skewed T = 16384 load),
the vendor GEMM (hipBLASLt through torch) on the same expert GEMM shapes as
context for the prefill MFMA figures, a stack of 48 distinct layers at T = 64 under the skewed load (eager and as
one replayed HIP graph; also at T = 1 and 8), a DeepSeekV2-Lite-shaped layer with two always-on
shared experts (decode, masked and all-ones), the mask-router backward
(straight-through estimator + sparsity term), the d=4096/I=1536 layer (decode T = 1 and 64,
prefill T = 4096, keep 0.15 and 0.5), and the fp64 oracle timed on this
host's cores on a bounded sample of the headline workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, vendor figure
# untimed calls before the warm-up steps of each measured configuration
SETTLE_S = 0.3
METRIC = "masked-MoE layer tok/s + HBM GB/s (decode) / MFMA % (prefill), E128 K8"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--T", type=int, default=256, help="tokens per step (decode batch)")
    ap.add_argument("--mask-bias", type=float, default=-1.04)
    ap.add_argument("--sets", type=int, default=0, help="weight sets to rotate (0 = auto)")
    ap.add_argument("--sweep", default="1,8,32,128,256",
                    help="decode batch sizes for the sweep ('' to skip)")
    ap.add_argument("--sweep-steps", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--prefill", default="2048,8192",
                    help="prefill batch sizes measured at mask biases -1.04/-0.52/0/+8 ('' to skip)")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--prefill-biases", default="-1.04,-0.52,0,8",
                    help="mask biases of the prefill runs (keep rate Phi(b))")
    ap.add_argument("--prefill-flags", type=int, default=0,
                    help="descriptor flags of the prefill runs (1 forces the streaming path, "
                         "2 the tiled path; 0 lets the library choose)")
    ap.add_argument("--only-prefill", action="store_true",
                    help="measure the prefill runs only (no decode headline, sweep or CPU baseline)")
    ap.add_argument("--skew", action="store_true", default=True,
                    help="also measure the skewed-load workload (T=16384)")
    ap.add_argument("--no-skew", dest="skew", action="store_false")
    ap.add_argument("--only-headline", action="store_true",
                    help="measure the headline workload only (no all-ones run, no sweep)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured copy/read/MFMA peaks")
    ap.add_argument("--stack", action="store_true", default=True,
                    help="also time the 48-layer stack at T=64 under the skewed load")
    ap.add_argument("--no-stack", dest="stack", action="store_false")
    ap.add_argument("--stack-T", type=int, default=64)
    ap.add_argument("--stack-steps", type=int, default=20)
    ap.add_argument("--stack-small", default="1,8",
                    help="comma list of small T for the same stack (launch-bound decode), '' for none")
    ap.add_argument("--backward", action="store_true", default=True,
                    help="also time the mask-router backward at T = 256, 2048, 8192")
    ap.add_argument("--no-backward", dest="backward", action="store_false")
    ap.add_argument("--only-backward", action="store_true",
                    help="time the mask-router backward only (no decode headline, sweep, prefill "
                         "or CPU baseline)")
    ap.add_argument("--shared", action="store_true", default=True,
                    help="also measure the DeepSeekV2-Lite-shaped layer with 2 shared experts")
    ap.add_argument("--no-shared", dest="shared", action="store_false")
    ap.add_argument("--vendor-gemm", action="store_true", default=True,
                    help="also time the vendor GEMM (torch.bmm / matmul, hipBLASLt) on the "
                         "expert GEMM shapes of the T=8192 keep-1.0 prefill layer")
    ap.add_argument("--no-vendor-gemm", dest="vendor_gemm", action="store_false")
    ap.add_argument("--large", action="store_true", default=True,
                    help="also measure the d=4096/I=1536 layer (decode T=1, 64; prefill 4096)")
    ap.add_argument("--no-large", dest="large", action="store_false")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (torch) three times, so that "
                         "hardware byte counters can be scaled by a copy of known size")
    return ap.parse_args()


# ---------------------------------------------------------------------------
HERE = os.path.dirname(os.path.abspath(__file__))
COUNTERS = os.path.join(HERE, "profiles", "decode_d2048_E128_K8_I768_T256_hbm_counters.md")


def counted_traffic():
    """Calibrated HBM bytes per launch of the dominant decode kernel, from the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary of the headline
    workload; None when that summary is missing or any of the kernel's
    source files (a comma list, hashed in order) has changed since the
    counters were taken."""
    import hashlib
    try:
        kv = {}
        for line in open(COUNTERS):
            line = line.strip()
            if line.startswith("traffic_") and ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        h = hashlib.sha256()
        for name in kv["traffic_source"].split(","):
            h.update(open(os.path.join(HERE, name.strip()), "rb").read())
        if h.hexdigest() != kv["traffic_source_sha256"]:
            return None
        return {"kernel": kv["traffic_kernel"], "bytes": int(kv["traffic_bytes_per_launch"])}
    except (OSError, KeyError, ValueError):
        return None


def algorithmic(n_act, P, T, d, E, I):
    """Algorithmic HBM bytes and FLOPs of one layer call and of its stages.

    Unit of work: one active expert (count >= 1) = 3*d*I bf16 weights read
    once (2*d*I gate/up rows, d*I down rows); one active pair = 6*d*I FLOPs;
    the router reads 2*E*d bf16 weights and does 4*d*E FLOPs per token.
    """
    b = 2  # bf16
    up = n_act * 2 * I * d * b + T * d * b + P * I * b
    down = n_act * d * I * b + P * I * b + P * d * b
    layer = n_act * 3 * d * I * b + 2 * E * d * b + 2 * T * d * b
    flops = 6.0 * d * I * P + 4.0 * d * E * T
    return {"up": up, "down": down, "layer": layer, "flops": flops}


def pct(vals, q):
    """The q-quantile (0..1) of vals, linear between order statistics."""
    v = sorted(vals)
    if not v:
        return None
    x = q * (len(v) - 1)
    i = int(math.floor(x))
    j = min(i + 1, len(v) - 1)
    return v[i] + (v[j] - v[i]) * (x - i)


def dist(vals):
    return {"median_ms": round(pct(vals, 0.5), 5), "p10_ms": round(pct(vals, 0.1), 5),
            "p90_ms": round(pct(vals, 0.9), 5), "n": len(vals)}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the layer has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import dynamic_expert_sparsity_amd as B
    from dynamic_expert_sparsity_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.lib()

    peaks = None
    if not args.no_peaks:
        from dynamic_expert_sparsity_amd import peak
        peaks = peak.measure(dev)
        log(f"measured peaks: copy {peaks['copy_GBps']} GB/s, read {peaks['read_GBps']} GB/s, "
            f"MFMA bf16 {peaks['mfma_bf16_TFLOPs']} TFLOP/s")

    shape = synth.SHAPES["qwen3"]
    d, E, K, I = shape.d, shape.E, shape.K, shape.I
    sweep = [int(v) for v in args.sweep.split(",") if v.strip()] if args.sweep else []
    if args.only_headline:
        sweep = []
    T_max = max([args.T] + sweep)

    # weight sets: enough that the bytes touched between two uses of one set
    # exceed the 256 MB infinity cache by a wide margin (48 also gives the
    # 48-layer stack distinct weights per layer)
    per_set_bytes = E * 3 * d * I * 2
    if args.sets:
        n_sets = args.sets
    else:
        n_sets = 4 if args.only_headline else 48
    free, total = torch.cuda.mem_get_info()
    n_sets = max(1, min(n_sets, int(0.6 * free // per_set_bytes)))
    log(f"drawing {n_sets} weight sets ({n_sets * per_set_bytes / 1e9:.1f} GB) on {dev}")
    t0 = time.time()
    sets = [synth.make_layer(shape, T_max, seed=0, layer=s, mask_bias=args.mask_bias, device=dev)
            for s in range(n_sets)]
    zeros_mask = torch.zeros_like(sets[0]["W_mask"])
    torch.cuda.synchronize()
    log(f"drawn in {time.time() - t0:.1f}s")

    def make_layers(T, allones=False):
        Ls = []
        for S in sets:
            Ls.append((B.MoELayer(S["W_gate"], zeros_mask if allones else S["W_mask"], S["W_gu"],
                                  S["W_dt"], K), S["x"][:T].contiguous()))
        return Ls

    def settle(Ls, seconds):
        """Untimed layer calls for `seconds` of wall time: the GPU's clocks
        drop while it waits on host work (buffer allocation, weight draws),
        and 20 steps started from an idle GPU run ~10% slower than the same
        steps in a continuous run (measured: 215 / 200 us per call for the
        first two 20-step runs after 1 s idle, 192 us in a steady run); a
        decode loop keeps the GPU busy, so the timing starts from that state."""
        ns = len(Ls)
        t_end = time.perf_counter() + seconds
        i = 0
        while time.perf_counter() < t_end:
            for _ in range(8):
                lay, x = Ls[i % ns]
                lay(x)
                i += 1
            torch.cuda.synchronize()

    def timed(Ls, steps, warmup, events=None, settle_s=0.0):
        """Time `steps` calls (wall clock, synchronised on both sides).

        events=None: no events (the clean timing).  events="stages": one event
        between every two stages (diagnostic: each record adds a few us).
        events="call": two events bracketing each whole call (per-call
        durations).  events=<stage name>: two events bracketing that stage
        only, on the launch stream (the kernel's launch duration).
        Returns (ms per step, dict of per-stage ms per step or None, list of
        per-step ms of the bracketed span or None)."""
        ns = len(Ls)
        for lay, x in Ls:  # buffers of every layer allocated before any timing
            lay.prepare(x.shape[0])
        if settle_s > 0:
            settle(Ls, settle_s)
        for i in range(warmup):
            lay, x = Ls[i % ns]
            lay(x)
        n_ev = len(B.STAGES) + 1
        ev = B.HipEvents(n_ev * steps) if events else None
        slots = None
        if events == "call":
            slots = (0, n_ev - 1)
        elif events and events != "stages":
            j = B.STAGES.index(events)
            slots = (j, j + 1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            lay, x = Ls[i % ns]
            if ev is None:
                lay(x)
            else:
                hs = ev.handles[i * n_ev:(i + 1) * n_ev]
                if slots:
                    hs = [h if q in slots else None for q, h in enumerate(hs)]
                lay(x, events=hs)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        stages, per = None, None
        if ev is not None:
            stages = {}
            if slots:
                per = [ev.elapsed_ms(i * n_ev + slots[0], i * n_ev + slots[1])
                       for i in range(steps)]
                stages[events] = sum(per) / steps
            else:
                for j, name in enumerate(B.STAGES):
                    stages[name] = sum(ev.elapsed_ms(i * n_ev + j, i * n_ev + j + 1)
                                       for i in range(steps)) / steps
                stages["gpu_total"] = sum(ev.elapsed_ms(i * n_ev, i * n_ev + n_ev - 1)
                                          for i in range(steps)) / steps
            ev.close()
        return ms, stages, per

    def counts(Ls):
        """Active pairs and active experts per entry (from one call each)."""
        out = []
        for lay, x in Ls:
            lay(x)
            torch.cuda.synchronize()
            na = lay.routing["num_active"].cpu().tolist()
            out.append((na[0], na[2]))
        return out

    def measure(Ls, T, steps, warmup, dims=(d, E, K, I), kernels=()):
        d_, E_, K_, I_ = dims
        ms, _, _ = timed(Ls, steps, warmup, settle_s=SETTLE_S)
        _, _, per = timed(Ls, steps, 5, events="call")
        _, stages, _ = timed(Ls, max(20, steps // 4), 5, events="stages")
        kern = {k: timed(Ls, steps, 5, events=k)[1][k] for k in kernels}
        cs = counts(Ls)
        P = sum(c[0] for c in cs) / len(cs)
        n_act = sum(c[1] for c in cs) / len(cs)
        alg = algorithmic(n_act, P, T, d_, E_, I_)
        r = {"T": T, "ms_per_step": ms, "tok_per_s": T / (ms * 1e-3),
             "per_call": dist(per),
             "active_pairs": P, "active_experts": n_act, "keep_rate": P / (T * K_),
             "layer_bytes": alg["layer"], "layer_GBps": alg["layer"] / (ms * 1e-3) / 1e9}
        r["layer_hbm_frac"] = r["layer_GBps"] / HBM_PEAK_GBPS
        r["stages_ms_evented"] = stages
        r["kernel_ms"] = kern
        r["_alg"] = alg
        return r

    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 copies of 1 GiB (1073741824 bytes read and written each)")
        del src, dst

    # ---- prefill: tiled grouped-GEMM path, MFMA utilisation ---------------
    def prefill_entry(Ls, T, b, skew, steps, dims=(d, E, K, I)):
        d_, E_, K_, I_ = dims
        ms, _, _ = timed(Ls, steps, 3, settle_s=SETTLE_S)
        _, _, per = timed(Ls, steps, 2, events="call")
        kern = {k: timed(Ls, steps, 2, events=k)[1][k] for k in ("router", "up", "down")}
        cs = counts(Ls)
        P = sum(c[0] for c in cs) / len(cs)
        n_act = sum(c[1] for c in cs) / len(cs)
        alg = algorithmic(n_act, P, T, d_, E_, I_)
        fl_up = 4.0 * d_ * I_ * P
        fl_dn = 2.0 * d_ * I_ * P
        out = {"T": T, "mask_bias": None if skew else b, "skew": skew,
               "keep_rate": round(P / (T * K_), 4), "active_pairs": P,
               "ms_per_step": round(ms, 5), "tok_per_s": round(T / (ms * 1e-3), 1),
               "per_call": dist(per),
               "mfma_frac_layer": round(alg["flops"] / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
               "hbm_frac_layer": round(alg["layer"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
               "kernel_ms": {k: round(v, 5) for k, v in kern.items()},
               "mfma_frac_up": round(fl_up / (kern["up"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
               "mfma_frac_down": round(fl_dn / (kern["down"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
               # the larger of the two floors: weight bytes at peak HBM, FLOPs at peak MFMA
               "roofline_ms": round(max(alg["layer"] / (HBM_PEAK_GBPS * 1e9),
                                        alg["flops"] / (BF16_PEAK_TFLOPS * 1e12)) * 1e3, 5)}
        out["roofline_frac"] = round(out["roofline_ms"] / ms, 4)
        return out

    def measure_prefill(T, b, skew=False, steps=args.prefill_steps):
        n = min(2, n_sets)
        Ls = []
        for s in range(n):
            S = sets[s]
            if skew:
                Sk = synth.make_layer(shape, T, seed=1, layer=100 + s, skew=True, device=dev)
                Ls.append((B.MoELayer(Sk["W_gate"], Sk["W_mask"], Sk["W_gu"], Sk["W_dt"], K,
                                      flags=args.prefill_flags), Sk["x"]))
            else:
                x = synth.make_tokens(shape, T, seed=0, layer=s, device=dev)
                Ls.append((B.MoELayer(S["W_gate"], synth.with_mask_bias(S["W_mask"], b),
                                      S["W_gu"], S["W_dt"], K, flags=args.prefill_flags), x))
        out = prefill_entry(Ls, T, b, skew, steps)
        del Ls
        return out

    def run_prefill():
        prefill_out = []
        for T in [int(v) for v in args.prefill.split(",") if v.strip()]:
            for b in [float(v) for v in args.prefill_biases.split(",") if v.strip()]:
                r = measure_prefill(T, b)
                prefill_out.append(r)
                log(f"prefill T={T} b={b:+g}: {r['ms_per_step']*1e3:.1f} us, keep {r['keep_rate']}, "
                    f"MFMA {r['mfma_frac_layer']:.3f}, roofline {r['roofline_frac']:.3f}")
        if args.skew:
            r = measure_prefill(16384, None, skew=True, steps=max(5, args.prefill_steps // 2))
            prefill_out.append(r)
            log(f"skew T=16384: {r['ms_per_step']*1e3:.1f} us, keep {r['keep_rate']}, "
                f"MFMA {r['mfma_frac_layer']:.3f}, roofline {r['roofline_frac']:.3f}")
        return prefill_out

    if args.only_backward:
        print(json.dumps({"metric": METRIC, "unit": "tok/s", "n_gpus": 1, "dtype": "bf16",
                          "data": "synthetic",
                          "mask_backward": run_backward(B, sets, shape, dev)}), flush=True)
        return

    if args.only_prefill:
        prefill_out = run_prefill()
        print(json.dumps({"metric": METRIC, "unit": "tok/s", "n_gpus": 1, "dtype": "bf16",
                          "data": "synthetic", "prefill": prefill_out}), flush=True)
        return

    # ---- headline --------------------------------------------------------
    log(f"headline: T={args.T}, {args.steps} steps after {args.warmup} warm-up")
    Ls = make_layers(args.T)
    head = measure(Ls, args.T, args.steps, args.warmup, kernels=("up", "down"))
    del Ls
    ones = None
    if not args.only_headline:
        Ls = make_layers(args.T, allones=True)
        ones = measure(Ls, args.T, args.steps, args.warmup, kernels=("up", "down"))
        del Ls
    km = head["kernel_ms"]
    dom = max(km, key=km.get)
    alg = head["_alg"]
    achieved = alg[dom] / (km[dom] * 1e-3) / 1e9
    # counted bytes apply to the headline workload and the up kernel they were taken on
    tr = counted_traffic() if (dom == "up" and args.T == 256 and args.mask_bias == -1.04) else None
    roofline = {"bound": "hbm", "kernel": f"expert_{dom}", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": tr["bytes"] if tr else None,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                "copy-calibrated)" if tr else None,
                "alg_bytes_per_launch": alg[dom],
                "avg_launch_ms": round(km[dom], 5),
                "measured_peak": peaks["read_GBps"] if peaks else None,
                "frac_of_measured_peak": round(achieved / peaks["read_GBps"], 4) if peaks else None,
                "other": {k: {"avg_launch_ms": round(v, 5),
                              "GBps": round(alg[k] / (v * 1e-3) / 1e9, 1)}
                          for k, v in km.items() if k != dom}}

    # ---- sweep -------------------------------------------------------------
    sweep_out = []
    for T in sweep:
        Ls = make_layers(T)
        m = measure(Ls, T, args.sweep_steps, 10)
        Ls = make_layers(T, allones=True)
        o = measure(Ls, T, args.sweep_steps, 10)
        del Ls
        sweep_out.append({
            "T": T,
            "masked": {k: _r(v) for k, v in m.items() if not k.startswith("_")},
            "allones": {k: _r(v) for k, v in o.items() if not k.startswith("_")},
            "speedup_vs_allones": round(o["ms_per_step"] / m["ms_per_step"], 3),
            "byte_ratio_allones": round(o["layer_bytes"] / m["layer_bytes"], 3),
        })
        log(f"sweep T={T}: masked {m['ms_per_step']*1e3:.1f} us, "
            f"all-ones {o['ms_per_step']*1e3:.1f} us")

    # ---- 48-layer stack at T = 64, skewed load ------------------------------
    stack = None
    if args.stack and not args.only_headline:
        stack = run_stack(B, synth, sets, shape, dev, args.stack_T, args.stack_steps,
                          dims=(d, E, K, I))
        log(f"stack: {stack['layers']} layers at T={stack['T']}: eager "
            f"{stack['eager']['ms_per_step']:.3f} ms, graph {stack['graph']['ms_per_step']:.3f} ms "
            f"per step")
    # the same stack at a few tokens, where kernel launches dominate
    stack_small = []
    if args.stack and not args.only_headline and args.stack_small:
        for Ts in (int(v) for v in args.stack_small.split(",") if v):
            st = run_stack(B, synth, sets, shape, dev, Ts, args.stack_steps, dims=(d, E, K, I))
            stack_small.append(st)
            log(f"stack: {st['layers']} layers at T={Ts}: eager "
                f"{st['eager']['ms_per_step']:.3f} ms, graph {st['graph']['ms_per_step']:.3f} ms "
                f"per step")

    # ---- shared experts: DeepSeekV2-Lite-shaped layer ------------------------
    shared = None
    if args.shared and not args.only_headline:
        shared = run_shared(B, synth, dev, measure, args)

    # ---- mask-router backward (STE + sparsity term) ------------------------
    backward = None
    if args.backward and not args.only_headline:
        backward = run_backward(B, sets, shape, dev)

    prefill_out = [] if args.only_headline else run_prefill()
    vendor = None
    if args.vendor_gemm and not args.only_headline:
        vendor = run_vendor_gemm(dev, shape)

    # ---- CPU baseline: the fp64 oracle on this host's cores ---------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(sets, args.T, K, args.cpu_seconds)

    # ---- the larger layer: d=4096, I=1536 -----------------------------------
    large = None
    if args.large and not args.only_headline:
        del sets
        torch.cuda.empty_cache()
        large = run_large(B, synth, dev, measure, prefill_entry, args)

    out = {
        "metric": METRIC,
        "value": round(head["tok_per_s"], 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": synth.workload_name("qwen3", args.T, mask_bias=args.mask_bias),
                   "phase": "decode", "T": args.T, "d": d, "E": E, "K": K, "I": I,
                   "mask_bias": args.mask_bias, "weight_sets": n_sets,
                   "keep_rate": round(head["keep_rate"], 4),
                   "active_experts": head["active_experts"], "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "per_call": head["per_call"],
        "layer_hbm": {"bytes": head["layer_bytes"], "GBps": round(head["layer_GBps"], 1),
                      "frac": round(head["layer_hbm_frac"], 4)},
        "measured_peaks": peaks,
        "stages_ms_evented": _r(head["stages_ms_evented"]),
        "allones": None if ones is None else {
            "ms_per_step": round(ones["ms_per_step"], 5),
            "tok_per_s": round(ones["tok_per_s"], 1),
            "per_call": ones["per_call"],
            "active_experts": ones["active_experts"],
            "layer_bytes": ones["layer_bytes"],
            "kernel_ms": _r(ones["kernel_ms"]),
            "speedup_masked_vs_allones": round(ones["ms_per_step"] / head["ms_per_step"], 3)},
        "sweep": sweep_out,
        "prefill": prefill_out,
        "vendor_gemm": vendor,
        "stack": stack,
        "stack_small": stack_small,
        "shared": shared,
        "mask_backward": backward,
        "large": large,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def run_stack(B, synth, sets, shape, dev, T, steps, dims):
    """A stack of distinct layers called back to back on one stream, T tokens
    each, under the skewed load (Zipf expert popularity, per-token mask bias):
    eagerly, then as one captured HIP graph replayed per step."""
    import torch

    d, E, K, I = dims
    Ls = []
    for l, S in enumerate(sets):
        R = synth.make_router(shape, T, seed=4, layer=200 + l, skew=True, device=dev)
        Ls.append((B.MoELayer(R["W_gate"], R["W_mask"], S["W_gu"], S["W_dt"], K), R["x"]))
    for lay, x in Ls:
        lay.prepare(T)

    def step():
        for lay, x in Ls:
            lay(x)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    # routing statistics and eager outputs of one step
    pairs, acts, ys = [], [], []
    for lay, x in Ls:
        y, R = lay(x)
        torch.cuda.synchronize()
        na = R["num_active"].cpu().tolist()
        pairs.append(na[0])
        acts.append(na[2])
        ys.append(y.clone())
    byts = sum(algorithmic(a, p, T, d, E, I)["layer"] for a, p in zip(acts, pairs))

    def time_steps(run):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for a, b in evs:
            a.record()
            run()
            b.record()
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3 / steps
        per = [a.elapsed_time(b) for a, b in evs]
        return {"ms_per_step": round(wall, 5), "tok_per_s": round(T / (wall * 1e-3), 1),
                "per_step": dist(per), "ms_per_layer": round(wall / len(Ls), 5),
                "layer_hbm_frac": round(byts / (wall * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}

    eager = time_steps(step)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # one eager pass on the capture stream first
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(lay.y, y0) for (lay, _), y0 in zip(Ls, ys))
    graph = time_steps(g.replay)
    graph["replay_equals_eager"] = same
    n = len(Ls)
    out = {"workload": f"{n} layers d{d}-E{E}-K{K}-I{I}-bf16-T{T}-skew", "layers": n, "T": T,
           "keep_rate": round(sum(pairs) / (n * T * K), 4),
           "active_experts_per_layer": round(sum(acts) / n, 2),
           "bytes_per_step": byts, "eager": eager, "graph": graph}
    del g, Ls
    return out


def run_vendor_gemm(dev, shape, reps=20):
    """Context for the prefill MFMA figures: the vendor library's bf16 GEMM
    (torch.bmm / torch.matmul, hipBLASLt) on the expert GEMMs of the T=8192
    keep-1.0 layer (E experts x 8192 K / E rows each, up [rows, d] x [d, 2I],
    down [rows, I] x [I, d]), as one batched call and as one dense GEMM over
    all rows, plus a square 8192^3 GEMM.  Operands are random and contiguous
    (no transposed views)."""
    import torch

    E, d, I = shape.E, shape.d, shape.I
    M = 8192 * shape.K // E
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    bf = torch.bfloat16
    rnd = lambda *sz: torch.randn(*sz, generator=g, device=dev, dtype=torch.float32).to(bf)  # noqa: E731

    def timeit(f, flops):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            f()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        tf = flops / (ms * 1e-3) / 1e12
        return {"us": round(ms * 1e3, 1), "TFLOPs": round(tf, 1),
                "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}

    out = {"library": "torch.bmm / torch.matmul (hipBLASLt), bf16", "rows_per_expert": M}
    A = rnd(E, M, d)
    Wu = rnd(E, d, 2 * I)
    out["bmm_up"] = timeit(lambda: torch.bmm(A, Wu), 2.0 * E * M * d * 2 * I)
    W1 = Wu[0].contiguous()
    A2 = A.reshape(E * M, d)
    out["dense_up"] = timeit(lambda: A2 @ W1, 2.0 * E * M * d * 2 * I)
    del Wu, W1, A, A2
    H = rnd(E, M, I)
    Wd = rnd(E, I, d)
    out["bmm_down"] = timeit(lambda: torch.bmm(H, Wd), 2.0 * E * M * I * d)
    W2 = Wd[0].contiguous()
    H2 = H.reshape(E * M, I)
    out["dense_down"] = timeit(lambda: H2 @ W2, 2.0 * E * M * I * d)
    del H, Wd, W2, H2
    X, Y = rnd(8192, 8192), rnd(8192, 8192)
    out["square_8192"] = timeit(lambda: X @ Y, 2.0 * 8192 ** 3)
    del X, Y
    torch.cuda.empty_cache()
    log("vendor GEMM: " + ", ".join(f"{k} {v['us']} us ({v['mfma_frac']:.3f})"
                                    for k, v in out.items() if isinstance(v, dict)))
    return out


def run_backward(B, sets, shape, dev, steps=20, batch=10):
    """beam_moe_mask_backward after a forward of the headline layer, T = 256,
    2048 and 8192 tokens (slot gradients drawn once per T).  Each sample
    times `batch` calls enqueued back to back between two events and counts
    their mean: the device time of a call, without the binding's per-call
    host work (four output allocations and the ctypes call, some 15 us,
    which the device otherwise spends idle).  Algorithmic bytes: x read
    (T d bf16), dx and the two [T, E] float32 logit gradients written,
    dW_mask written; FLOPs of the dW contraction 2 T E d."""
    import torch

    d, E, K = shape.d, shape.E, shape.K
    out = []
    for T in (256, 2048, 8192):
        S = sets[0]
        x = S["x"][:T].contiguous() if S["x"].shape[0] >= T else None
        if x is None:
            from dynamic_expert_sparsity_amd import synth
            x = synth.make_tokens(shape, T, seed=0, layer=0, device=dev)
        lay = B.MoELayer(S["W_gate"], S["W_mask"], S["W_gu"], S["W_dt"], K)
        lay(x)
        gen = torch.Generator(device=dev)
        gen.manual_seed(T)
        sg = torch.randn((T, K), generator=gen, device=dev, dtype=torch.float32)
        for _ in range(3):
            lay.mask_backward(x, sg, 0.01)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for a, b in evs:
            a.record()
            for _ in range(batch):
                lay.mask_backward(x, sg, 0.01)
            b.record()
        torch.cuda.synchronize()
        per = [a.elapsed_time(b) / batch for a, b in evs]
        ms = pct(per, 0.5)
        byts = T * d * 2 + T * d * 4 + 2 * T * E * 4 + E * d * 4
        flops = 2.0 * T * E * d
        out.append({"T": T, "per_call": dist(per), "alg_bytes": byts,
                    "GBps": round(byts / (ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                    "dW_TFLOPs": round(flops / (ms * 1e-3) / 1e12, 2)})
        log(f"mask backward T={T}: {ms * 1e3:.1f} us")
        del lay
    return {"workload": f"d{d}-E{E}-K{K}-bf16 mask router backward, beta 0.01",
            "timing": f"mean of {batch} calls enqueued back to back per sample", "runs": out}


def run_shared(B, synth, dev, measure, args):
    """The DeepSeekV2-Lite-shaped layer (d=2048, 64 routed experts, top-6,
    I=1408, 2 always-on shared experts): decode T = 1, 32, 256 at mask bias
    -1.04 and with the all-ones mask (the shared experts run in both)."""
    import torch

    shp = synth.SHAPES["dsv2lite"]
    S = synth.N_SHARED["dsv2lite"]
    d, E, K, I = shp.d, shp.E, shp.K, shp.I
    per_set = (E + S) * 3 * d * I * 2
    free, _ = torch.cuda.mem_get_info()
    n = max(1, min(24, int(0.4 * free // per_set)))
    log(f"shared-expert layer: drawing {n} weight sets ({n * per_set / 1e9:.1f} GB)")
    sets = []
    for s in range(n):
        L = synth.make_layer(shp, 256, seed=0, layer=400 + s, mask_bias=-1.04, n_shared=S,
                             device=dev)
        L["W_gu"] = torch.cat([L.pop("W_gu"), L.pop("Ws_gu")]).contiguous()
        L["W_dt"] = torch.cat([L.pop("W_dt"), L.pop("Ws_dt")]).contiguous()
        sets.append(L)
    zeros = torch.zeros_like(sets[0]["W_mask"])
    out = []
    for T in (1, 32, 256):
        row = {"T": T}
        for kind in ("masked", "allones"):
            Ls = [(B.MoELayer(L["W_gate"], zeros if kind == "allones" else L["W_mask"],
                              L["W_gu"], L["W_dt"], K), L["x"][:T].contiguous()) for L in sets]
            m = measure(Ls, T, args.sweep_steps, 10, dims=(d, E, K, I))
            row[kind] = {k: _r(v) for k, v in m.items() if not k.startswith("_")}
            del Ls
        row["speedup_vs_allones"] = round(row["allones"]["ms_per_step"] /
                                          row["masked"]["ms_per_step"], 3)
        out.append(row)
        log(f"shared-expert layer T={T}: masked {row['masked']['ms_per_step']*1e3:.1f} us, "
            f"all-ones {row['allones']['ms_per_step']*1e3:.1f} us")
    del sets
    return {"workload": f"d{d}-E{E}+{S}shared-K{K}-I{I}-bf16", "weight_sets": n, "runs": out}


def run_large(B, synth, dev, measure, prefill_entry, args):
    """The d=4096, E=128, K=8, I=1536 layer: decode T = 1 and 64, prefill
    T = 4096, each at mask biases -1.04 and 0 (keep 0.15 and 0.5)."""
    import torch

    shp = synth.SHAPES["large"]
    d, E, K, I = shp.d, shp.E, shp.K, shp.I
    per_set = E * 3 * d * I * 2
    free, _ = torch.cuda.mem_get_info()
    n = max(1, min(4, int(0.5 * free // per_set)))
    log(f"large layer: drawing {n} weight sets ({n * per_set / 1e9:.1f} GB)")
    sets = [synth.make_layer(shp, 64, seed=0, layer=300 + s, mask_bias=0.0, device=dev)
            for s in range(n)]
    out = []
    for b in (-1.04, 0.0):
        masks = [synth.with_mask_bias(S["W_mask"], b) for S in sets]
        lays = [B.MoELayer(S["W_gate"], m, S["W_gu"], S["W_dt"], K) for S, m in zip(sets, masks)]
        for T in (1, 64):
            if T == 1:
                # distinct single tokens, so repeated calls do not find their
                # experts in the infinity cache
                Ls = [(lays[j % n], sets[j % n]["x"][j // n:j // n + 1].contiguous())
                      for j in range(64)]
            else:
                Ls = [(lays[s], sets[s]["x"]) for s in range(n)]
            m = measure(Ls, T, args.sweep_steps, 10, dims=(d, E, K, I))
            out.append({"phase": "decode", "mask_bias": b,
                        **{k: _r(v) for k, v in m.items() if not k.startswith("_")}})
            log(f"large decode T={T} b={b:+g}: {m['ms_per_step']*1e3:.1f} us, "
                f"HBM {m['layer_hbm_frac']:.3f}")
        xs = [synth.make_tokens(shp, 4096, seed=0, layer=300 + s, device=dev)
              for s in range(min(n, 2))]
        pl = [B.MoELayer(S["W_gate"], m, S["W_gu"], S["W_dt"], K)
              for S, m in zip(sets[:len(xs)], masks)]
        r = prefill_entry(list(zip(pl, xs)), 4096, b, False, args.prefill_steps,
                          dims=(d, E, K, I))
        out.append({"phase": "prefill", **r})
        log(f"large prefill T=4096 b={b:+g}: {r['ms_per_step']*1e3:.1f} us, "
            f"MFMA {r['mfma_frac_layer']:.3f}, roofline {r['roofline_frac']:.3f}")
        del lays, pl, xs, masks
    del sets
    return {"workload": f"d{d}-E{E}-K{K}-I{I}-bf16", "weight_sets": n, "runs": out}


def _r(v):
    if isinstance(v, float):
        return round(v, 5)
    if isinstance(v, dict):
        return {k: _r(x) for k, x in v.items()}
    return v


def cpu_baseline(sets, T, K, budget_s):
    """Time the fp64 oracle (route from scratch + Eq. 8) on this host."""
    import numpy as np
    import torch

    import oracle

    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = None
    cores = len(os.sched_getaffinity(0))
    total_t = 0.0
    total_tok = 0
    calls = 0
    for s, S in enumerate(sets):
        x = S["x"][:T].float().cpu().numpy()
        Wg = S["W_gate"].float().cpu().numpy()
        Wm = S["W_mask"].float().cpu().numpy()
        # host float32 copies of the experts this batch uses (not timed)
        R0 = oracle.route(x, Wg, Wm, K)
        used = sorted(set(int(e) for e in np.asarray(R0["masked_ids"]).ravel() if e >= 0))
        Wgu = {e: S["W_gu"][e].float().cpu().numpy() for e in used}
        Wdt = {e: S["W_dt"][e].float().cpu().numpy() for e in used}
        t0 = time.perf_counter()
        R = oracle.route(x, Wg, Wm, K)
        oracle.forward(x, Wg, Wm, Wgu, Wdt, K, routing=R)
        total_t += time.perf_counter() - t0
        total_tok += T
        calls += 1
        del Wgu, Wdt
        if total_t >= budget_s or calls >= 32:
            break
    log(f"cpu baseline: {calls} layer calls of T={T} in {total_t:.1f}s")
    return {"value": round(total_tok / total_t, 2), "unit": "tok/s", "cores": cores,
            "blas_threads": blas, "kind": "oracle",
            "sample": f"{calls} layer calls x {T} tokens (distinct weight sets), fp64 route + Eq. 8, "
                      f"{total_t:.1f} s"}


if __name__ == "__main__":
    main()
