#!/usr/bin/env python3
"""Benchmark of the routed-MoE layer forward on one MI355X.

Workload (default): GLM-5.2-like MoE layers (h=6144, 256 routed experts of
int4 gs64 weights, I=2048, top-8, 1 shared expert, routed_scaling_factor 2.5),
8 independent layers resident in HBM (43.7 GB of experts), decode T=1 token
per layer call.  One step = one forward of each of the 8 layers, each on its
own seeded hidden state (a pool of distinct inputs rotates, so routed experts
change from call to call and the 256 MB Infinity Cache cannot serve them).

Prints one JSON line: MoE-layer tokens/s (value), expert-weight HBM GB/s, the
roofline of the dominant kernel (per-launch algorithmic bytes over its mean
HIP-event duration, measured on the library's stream), and the CPU oracle
timed on a bounded sample of the same workload (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--tokens T] [--layers L]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--tokens", type=int, default=1, help="tokens per layer call (decode batch)")
    ap.add_argument("--layers", type=int, default=8, help="resident layers cycled by a step")
    ap.add_argument("--pool", type=int, default=32, help="distinct inputs per layer")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: this build has no multi-GPU path "
              "(--gpus must be 1; see the sharding notes of the design).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import routed_expert_ffn_f32_amd as cm
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cm.load_library()  # fails loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    shape = synth.GLM
    T, L, K, W = args.tokens, args.layers, args.steps, args.warmup
    h, I, E, k = shape.hidden, shape.inter, shape.n_experts, shape.top_k

    # ---- resident layers -------------------------------------------------
    t0 = time.time()
    layers, keep = [], []
    for l in range(L):
        wr, b = synth.router(shape, args.seed, l)
        routed = synth.routed_tables(shape, args.seed, l)
        shared = synth.shared_tables(shape, args.seed, l)
        tensors = {"router_w": torch.from_numpy(wr).to(dev), "sel_bias": torch.from_numpy(b).to(dev)}
        tensors.update({n: torch.from_numpy(v).to(dev) for n, v in routed.items()})
        tensors.update({"sh_" + n: torch.from_numpy(v).to(dev) for n, v in shared.items()})
        del routed, shared
        cfg = cm.make_config(hidden=h, n_experts=E, top_k=k, inter=I, n_shared=shape.n_shared,
                             routed_scaling_factor=shape.rsf, max_tokens=max(T, 1))
        layers.append(cm.MoELayer(cfg, tensors))
        keep.append(tensors)
        log(f"layer {l} resident ({time.time() - t0:.1f} s)")
    xs = [[torch.from_numpy(synth.hidden(shape, args.seed, T, layer=l, batch=i)).to(dev)
           for i in range(args.pool)] for l in range(L)]
    outs = [torch.empty((T, h), dtype=torch.float32, device=dev) for _ in range(L)]
    torch.cuda.synchronize()

    # distinct experts per (layer, input): read back from the library's own
    # dispatch (n_active) once, outside any timed region
    n_active = np.zeros((L, args.pool), np.int64)
    for l in range(L):
        for i in range(args.pool):
            layers[l](xs[l][i], outs[l])
            _, r = layers[l].last_routing()
            n_active[l, i] = int(r["n_active"].item())

    def step(s):
        for l in range(L):
            layers[l](xs[l][(s * L + l) % args.pool], outs[l])

    for s in range(W):
        step(s)
    torch.cuda.synchronize()

    # ---- timed region ------------------------------------------------------
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for s in range(K):
        step(W + s)
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / K
    calls = [(l, (W + s) * L + l) for s in range(K) for l in range(L)]
    tok_per_s = T * L * K / (total_ms / 1e3)
    eb = shape.expert_bytes
    experts_read = sum(int(n_active[l, c % args.pool]) + shape.n_shared for l, c in calls)
    expert_gbps = experts_read * eb / (total_ms / 1e3) / 1e9

    # ---- per-kernel HIP-event timing over a second timed region -------------
    for lay in layers:
        cm.coli_moe_profile_begin(lay.handle, K)
    torch.cuda.synchronize()
    for s in range(K):
        step(W + s)
    torch.cuda.synchronize()
    kern = {}
    for lay in layers:
        _, d = cm.coli_moe_profile_end(lay.handle)
        for name, (ms, n) in d.items():
            a = kern.setdefault(name, [0.0, 0])
            a[0] += ms
            a[1] += n
    kern_us = {n: round(1e3 * ms / c, 3) for n, (ms, c) in kern.items() if c}

    # dominant kernel: gate/up GEMV; algorithmic bytes per launch = the
    # selected experts' gate and up codes + scales, the token rows read and
    # the intermediate rows written
    gate_up_w = 2 * (I * h // 2 + 4 * I * h // 64)
    mean_experts = float(np.mean([n_active[l, c % args.pool] for l, c in calls])) + shape.n_shared
    gu_bytes = mean_experts * gate_up_w + T * h * 4 + (T * k + T * shape.n_shared) * I * 4
    gu_ms, gu_n = kern.get("expert_gemv_gate_up", (0.0, 0))
    gu_avg_s = gu_ms / gu_n / 1e3 if gu_n else float("nan")
    achieved = gu_bytes / gu_avg_s / 1e9

    result = {
        "metric": "MoE-layer tokens/s + expert-weight HBM GB/s (int4 gs64, decode T=1)",
        "value": round(tok_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,0.02) weights quantised to int4 gs64, N(0,1) hidden states)",
        "config": {"workload": f"GLM-5.2-like MoE layer decode T={T}, {L} layers resident in HBM",
                   "hidden": h, "n_experts": E, "top_k": k, "inter": I, "n_shared": shape.n_shared,
                   "tokens_per_call": T, "layers": L, "input_pool": args.pool, "seed": args.seed},
        "expert_weight_GBps": round(expert_gbps, 1),
        "expert_weight_frac_of_hbm_peak": round(expert_gbps / HBM_PEAK_GBPS, 4),
        "us_per_layer_call": round(1e3 * total_ms / (K * L), 3),
        "kernel_avg_us": kern_us,
        "roofline": {"kernel": "expert_gemv_gate_up", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None, "bytes_per_launch": int(gu_bytes)},
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, shape, layers, xs, outs, dev)

    print(json.dumps(result), flush=True)


def cpu_baseline(args, shape, layers, xs, outs, dev):
    """The oracle, as it stands, on a bounded sample of the same workload:
    single decode tokens of layer 0 from its input pool, until the time
    budget is spent.  The GPU's outputs for the same tokens are compared on
    the way (max relative error, floored at the row RMS)."""
    import numpy as np
    import torch

    import oracle
    import synth

    wr, b = synth.router(shape, args.seed, 0)
    shared = synth.shared_tables(shape, args.seed, 0)
    done, spent, worst = 0, 0.0, 0.0
    cache = {}
    while spent < args.cpu_seconds and done < args.pool:
        x = xs[0][done].cpu().numpy()
        idx, _ = oracle.route(shape, wr, b, x)
        for e in np.unique(idx):
            if int(e) not in cache:
                cache[int(e)] = synth.expert(shape, args.seed, int(e), 0)
        routed = [cache.get(e) for e in range(shape.n_experts)]
        t0 = time.perf_counter()
        ref, _, _ = oracle.forward(shape, wr, b, routed, shared, x)
        spent += time.perf_counter() - t0
        layers[0](xs[0][done], outs[0])
        torch.cuda.synchronize()
        got = outs[0].cpu().numpy().astype(np.float64)
        r = ref.astype(np.float64)
        rms = np.sqrt((r ** 2).mean(axis=-1, keepdims=True))
        worst = max(worst, float((np.abs(got - r) / np.maximum(np.abs(r), rms)).max()))
        done += 1
    T = xs[0][0].shape[0]
    return {"value": round(done * T / spent, 4), "unit": "tokens/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"{done} decode calls of T={T} on layer 0 (routing + 8 routed + shared expert "
                      f"FFNs in float64), {spent:.1f} s",
            "gpu_max_rel_err_on_sample": worst}


if __name__ == "__main__":
    main()
