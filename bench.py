#!/usr/bin/env python3
"""Benchmark of the routed-MoE layer forward on one MI355X.

Headline workload: GLM-5.2-like MoE layers (h=6144, 256 routed experts of
int4 gs64 weights, I=2048, top-8, 1 shared expert, routed_scaling_factor 2.5),
8 independent layers resident in HBM (43.7 GB of experts), decode T=1 token
per layer call.  One step = one forward of each of the 8 layers, each on its
own seeded hidden state (a pool of distinct inputs rotates, so routed experts
change from call to call and the 256 MB Infinity Cache cannot serve them).

Also measured in the same run (extra fields of the JSON line):
  decode_batches  the same 8-layer stack at T = 2, 4 and 64 tokens per call;
  routing_limits_decode_T1  the stack at T = 1 with the lossy routing
                  overrides (adaptive expert top-p, explicit smaller k);
  prefill         T = 4096 tokens on the GLM-like layer with Zipf-skewed
                  expert load (fp16 MFMA path): tokens/s and the grouped-GEMM
                  kernels' FLOP rate against the fp16 dense peak and against
                  the rate this GPU sustains on varied fp16 operands;
  small_configs   the tiny layer (T = 4) and the OLMoE-like layer (T = 16,
                  8 weight copies in turn so that HBM serves every call);
  int8_mtp_layer  the GLM-like layer with int8 tables (the MTP head's
                  format) at T = 1..4;
  expert_cache    the GLM-like layer served from pinned host memory through
                  an HBM expert cache, and the router look-ahead prefetch.

Prints one JSON line: MoE-layer tokens/s (value), expert-weight HBM GB/s, the
roofline of the dominant kernel (per-launch algorithmic bytes over its mean
HIP-event duration, measured on the library's stream; HBM traffic from the
committed rocprofv3 counter summary when it matches the kernel source), and
the CPU oracle timed on a bounded sample of the same workload (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]
    python bench.py --copy-calibration   # plain 1 GiB device copy (counter scale)
    python bench.py --prefill-only       # the prefill layer alone (for counter runs)
    python bench.py --int8-only          # the int8 (MTP-head format) layer alone
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E, published
F16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 / bf16 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_expert_gemv_gate_up.txt")
TRAFFIC_FILE_DOWN = os.path.join(ROOT, "profiles", "traffic_expert_gemv_down.txt")
# sources of the dominant kernel: a counter summary taken on other sources
# describes other code
TRAFFIC_SOURCES = ["routed_expert_ffn_f32_amd/csrc/expert_gemv.hip", "routed_expert_ffn_f32_amd/csrc/wave.h",
                   "routed_expert_ffn_f32_amd/csrc/select.h", "routed_expert_ffn_f32_amd/csrc/small_route.h",
                   "routed_expert_ffn_f32_amd/csrc/internal.h"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8, help="resident layers cycled by a step")
    ap.add_argument("--pool", type=int, default=32, help="distinct inputs per layer")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="headline decode T=1 only")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device-to-device copy 5 times and exit")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill layer (T=4096, Zipf load): print its JSON object and exit")
    ap.add_argument("--no-cache", action="store_true", help="skip the expert-cache rows")
    ap.add_argument("--cache-only", action="store_true",
                    help="only the expert-cache rows (host-backed GLM-like layer): print their JSON object and exit")
    ap.add_argument("--int8-only", action="store_true",
                    help="only the int8-table layer (the MTP head's format): print its JSON object and exit")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def sources_digest() -> str:
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(path=None):
    """HBM bytes per launch of a decode kernel (default: the dominant one) from
    its committed counter summary, or None when it is absent or was taken on
    other sources."""
    try:
        kv = {}
        with open(path or TRAFFIC_FILE) as f:
            for line in f:
                line = line.strip()
                if line and not line.startswith("#") and "=" in line:
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != sources_digest():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_calibration():
    import torch
    dev = torch.device("cuda:0")
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 5}), flush=True)


def time_calls(torch, fn, n):
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(n):
        fn(i)
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1)


def kernel_profile(cm, handles, run, n_calls):
    """Mean HIP-event duration per launch of each library kernel over n_calls
    forwards of each handle (events recorded by the library on its stream)."""
    for hd in handles:
        cm.coli_moe_profile_begin(hd, n_calls)
    run()
    import torch
    torch.cuda.synchronize()
    kern = {}
    for hd in handles:
        _, d = cm.coli_moe_profile_end(hd)
        for name, (ms, n) in d.items():
            a = kern.setdefault(name, [0.0, 0])
            a[0] += ms
            a[1] += n
    return {n: (ms, c) for n, (ms, c) in kern.items() if c}


def measured_peaks(cm, torch, dev):
    """This GPU's own rates, measured in the same run with the library's
    probes, beside the published peaks: the HBM read rate over an 8 GiB
    buffer (every byte read once), the back-to-back bf16 MFMA rate on
    all-ones operands and the fp16 rate on operands that vary from one MFMA
    to the next (one wave per SIMD on every CU; the clock falls with the
    power that varied data draws); each the best of five launches timed with
    HIP events, each probe's result checked."""
    stream = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def best_ms(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return min(out)

    nbytes = 8 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    hbm_ms = best_ms(lambda: cm.coli_moe_probe_stream(buf.data_ptr(), nbytes, sink.data_ptr(), stream))
    del buf
    blocks, iters = 256, 40000
    sink.zero_()
    mfma_ms = best_ms(lambda: cm.coli_moe_probe_mfma(iters, blocks, sink.data_ptr(), stream))
    torch.cuda.synchronize()
    waves_ok = int(sink.item())
    flops = blocks * 4 * iters * cm.MFMA_PROBE_MFMAS_PER_ROUND * 32768
    iters16 = iters // 2
    sink.zero_()
    f16_ms = best_ms(lambda: cm.coli_moe_probe_mfma_f16(iters16, blocks, 12345, sink.data_ptr(), stream))
    torch.cuda.synchronize()
    waves16 = int(sink.item())
    flops16 = blocks * 4 * iters16 * cm.MFMA_F16_PROBE_MFMAS_PER_ROUND * 32768
    return {"hbm_read_GBps": round(nbytes / (hbm_ms / 1e3) / 1e9, 1), "hbm_buffer_bytes": nbytes,
            "mfma_bf16_ones_TFLOPs": round(flops / (mfma_ms / 1e3) / 1e12, 1),
            "mfma_probe_waves_checked": f"{waves_ok} of {6 * blocks * 4}",
            "mfma_f16_varied_TFLOPs": round(flops16 / (f16_ms / 1e3) / 1e12, 1),
            "mfma_f16_probe_waves_finite": f"{waves16} of {6 * blocks * 4}",
            "published": {"hbm_GBps": HBM_PEAK_GBPS, "f16_bf16_dense_TFLOPs": F16_PEAK_TFLOPS}}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: the library has no multi-GPU path "
              "(--gpus must be 1; see the sharding notes of the design).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    import routed_expert_ffn_f32_amd as cm
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cm.load_library()  # fails loudly if the HIP library is not built
    dev = torch.device("cuda:0")
    if args.prefill_only:
        print(json.dumps(prefill(args, cm, torch, np, synth, dev)), flush=True)
        return
    if args.cache_only:
        print(json.dumps(cache_rows(args, cm, torch, np, synth, dev)), flush=True)
        return
    if args.int8_only:
        print(json.dumps(int8_rows(args, cm, torch, np, synth, dev)), flush=True)
        return
    shape = synth.GLM
    L, K, W = args.layers, args.steps, args.warmup
    h, I, E, k = shape.hidden, shape.inter, shape.n_experts, shape.top_k
    batches = [] if args.no_extra else [2, 4, 64]
    max_t = max([1] + batches)

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
                             routed_scaling_factor=shape.rsf, max_tokens=max_t)
        layers.append(cm.MoELayer(cfg, tensors))
        keep.append(tensors)
        log(f"layer {l} resident ({time.time() - t0:.1f} s)")
    eb = shape.expert_bytes

    def make_pool(T, n):
        xs = [[torch.from_numpy(synth.hidden(shape, args.seed, T, layer=l, batch=1000 * T + i)).to(dev)
               for i in range(n)] for l in range(L)]
        outs = [torch.empty((T, h), dtype=torch.float32, device=dev) for _ in range(L)]
        # distinct experts per (layer, input) from the library's own dispatch,
        # read back once outside any timed region
        na = np.zeros((L, n), np.int64)
        ex = [[None] * n for _ in range(L)]  # the experts each call reads: active routed ones, then -1 (shared)
        for l in range(L):
            for i in range(n):
                layers[l](xs[l][i], outs[l])
                _, r = layers[l].last_routing()
                na[l, i] = int(r["n_active"].item())
                act = r["active"][:na[l, i]].cpu().tolist() + ([-1] if shape.n_shared else [])
                ex[l][i] = torch.tensor(act, dtype=torch.int32, device=dev)
        make_pool.experts = ex
        return xs, outs, na

    def run_stack(xs, outs, s0, steps):
        n = len(xs[0])
        for s in range(s0, s0 + steps):
            for l in range(L):
                layers[l](xs[l][(s * L + l) % n], outs[l])

    # ---- headline: decode T=1 ---------------------------------------------
    T = 1
    xs, outs, n_active = make_pool(T, args.pool)
    run_stack(xs, outs, 0, W)
    torch.cuda.synchronize()
    total_ms = time_calls(torch, lambda s: run_stack(xs, outs, W + s, 1), K)
    ms_per_step = total_ms / K
    calls = [(l, (W + s) * L + l) for s in range(K) for l in range(L)]
    tok_per_s = T * L * K / (total_ms / 1e3)
    experts_read = sum(int(n_active[l, c % args.pool]) + shape.n_shared for l, c in calls)
    expert_gbps = experts_read * eb / (total_ms / 1e3) / 1e9

    # per-kernel HIP-event timing over a second timed region
    kern = kernel_profile(cm, [lay.handle for lay in layers], lambda: run_stack(xs, outs, W, K), K)
    kern_us = {n: round(1e3 * ms / c, 3) for n, (ms, c) in kern.items()}

    # dominant kernel: gate/up GEMV; algorithmic bytes per launch = the
    # selected experts' gate and up codes + scales, the token rows read and
    # the intermediate rows written
    gate_up_w = 2 * (I * h // 2 + 4 * I * h // 64)
    mean_experts = float(np.mean([n_active[l, c % args.pool] for l, c in calls])) + shape.n_shared
    dom_name = "expert_gemv_gate_up"
    dom_bytes = mean_experts * gate_up_w + T * h * 4 + (T * k + T * shape.n_shared) * I * 4
    dom_ms, dom_n = kern.get(dom_name, (0.0, 0))
    dom_avg_s = dom_ms / dom_n / 1e3 if dom_n else float("nan")
    achieved = dom_bytes / dom_avg_s / 1e9
    traffic = read_traffic()

    # read ceiling of the same access pattern: a pure-load launch of the
    # same calls' gate and up rows (same grid, nothing computed)
    stream = torch.cuda.current_stream().cuda_stream

    def probe_us_per_call(probe, exs, pool, s0, n):
        """Mean time of one probe launch per layer call over the calls
        s0 .. s0+n-1 of the stack (the experts those calls read)."""
        def run(a, steps):
            for st in range(a, a + steps):
                for l in range(L):
                    e = exs[l][(st * L + l) % pool]
                    probe(layers[l].handle, e.data_ptr(), e.numel(), stream)
        run(0, s0)
        return 1e3 * time_calls(torch, lambda st: run(s0 + st, 1), n) / (n * L)

    probe_us = probe_us_per_call(cm.coli_moe_probe_read, make_pool.experts, args.pool, W, K)
    probe_bytes = mean_experts * gate_up_w
    # the same for the down + combine launch: its experts' down rows, its
    # grid and row split, loads only
    probe_down_us = probe_us_per_call(cm.coli_moe_probe_read_down, make_pool.experts, args.pool, W, K)

    # every decode kernel's algorithmic bytes and rate: the router (f32 table
    # and the token row, the digit planes written), gate/up (above), down with
    # the combine (the experts' down codes and scales, the intermediate rows,
    # the output row)
    down_w = h * (I // 2 + 4 * I // 64)
    per_kernel_bytes = {
        "router_logits": E * h * 4 + T * h * 4 + T * (6 * h // 8 + h // 32) * 4,
        dom_name: dom_bytes,
        "expert_gemv_down": mean_experts * down_w + (T * k + T * shape.n_shared) * I * 4 + T * h * 4,
    }
    kernel_rates = {}
    for name, nbytes in per_kernel_bytes.items():
        ms, n = kern.get(name, (0.0, 0))
        if n:
            us = 1e3 * ms / n
            kernel_rates[name] = {"bytes": int(nbytes), "us": round(us, 3), "GBps": round(nbytes / us / 1e3, 1)}
    # HBM traffic per launch from the committed counter summaries (null when
    # the kernel's sources changed since the counters were taken)
    for name, path in ((dom_name, TRAFFIC_FILE), ("expert_gemv_down", TRAFFIC_FILE_DOWN)):
        if name in kernel_rates:
            tr = read_traffic(path)
            kernel_rates[name]["traffic"] = None if tr is None else round(tr)

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
        "kernel_rates": kernel_rates,
        "roofline": {"kernel": dom_name, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "bytes_per_launch": int(dom_bytes)},
        "read_ceiling": {"kernel": "read probe: the same calls' gate and up rows, loads only, same grid",
                         "us_per_launch": round(probe_us, 3), "GBps": round(probe_bytes / probe_us / 1e3, 1),
                         "dominant_kernel_time_over_probe": round(1e6 * dom_avg_s / probe_us, 4)},
        "read_ceiling_down": {"kernel": "read probe: the same calls' down rows, loads only, the down + combine "
                                        "launch's grid and row split",
                              "us_per_launch": round(probe_down_us, 3),
                              "GBps": round(mean_experts * down_w / probe_down_us / 1e3, 1),
                              "down_kernel_time_over_probe": (round(kernel_rates["expert_gemv_down"]["us"] /
                                                                    probe_down_us, 4)
                                                              if "expert_gemv_down" in kernel_rates else None)},
    }
    # per-step times of the same stack (a separate loop, one event per step)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    evs[0].record()
    for s in range(K):
        run_stack(xs, outs, W + s, 1)
        evs[s + 1].record()
    torch.cuda.synchronize()
    st = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(K))
    result["step_ms_percentiles"] = {"p10": round(st[K // 10], 5), "p50": round(st[K // 2], 5),
                                     "p90": round(st[min(K - 1, (9 * K) // 10)], 5)}
    del xs, outs

    # ---- this GPU's own peak rates --------------------------------------------
    peaks = measured_peaks(cm, torch, dev)
    peaks["dominant_kernel_frac_of_measured_hbm"] = round(achieved / peaks["hbm_read_GBps"], 4)
    result["measured_peaks"] = peaks

    # ---- decode batches on the same stack ----------------------------------
    if batches:
        res = {}
        for Tb in batches:
            pool = 8
            xb, ob, na = make_pool(Tb, pool)
            steps = max(10, K // (4 * Tb)) if Tb < 64 else 10
            run_stack(xb, ob, 0, 3)
            ms = time_calls(torch, lambda s: run_stack(xb, ob, 3 + s, 1), steps)
            n_calls = steps * L
            reads = sum(int(na[l, ((3 + s) * L + l) % pool]) + shape.n_shared for s in range(steps) for l in range(L))
            res[str(Tb)] = {"tokens_per_s": round(Tb * n_calls / (ms / 1e3), 1),
                            "us_per_layer_call": round(1e3 * ms / n_calls, 2),
                            "expert_weight_GBps": round(reads * eb / (ms / 1e3) / 1e9, 1),
                            "mean_distinct_experts": round(float(na.mean()), 1)}
            if Tb <= 4:
                # the small-batch launches stream the batch's distinct experts
                # over the grids of the two read probes: their sum is the
                # floor of the call's expert reads
                fl = sum(probe_us_per_call(pr, make_pool.experts, pool, 3, steps)
                         for pr in (cm.coli_moe_probe_read, cm.coli_moe_probe_read_down))
                res[str(Tb)]["read_probe_floor_us"] = round(fl, 2)
                res[str(Tb)]["call_over_read_floor"] = round(1e3 * ms / n_calls / fl, 3)
            del xb, ob
            log(f"decode T={Tb}: {res[str(Tb)]}")
        result["decode_batches"] = res

    # ---- run-time routing limits (lossy), decode T=1 on the same stack ------
    if not args.no_extra:
        import warnings
        res = {}
        for k_use, top_p in ((k, 0.7), (k, 0.5), (6, 1.0), (4, 1.0)):
            with warnings.catch_warnings():
                warnings.simplefilter("ignore")
                for lay in layers:
                    lay.set_routing(k_use, top_p)
            pool = 16
            xb, ob, na = make_pool(1, pool)
            steps = max(20, K // 2)
            run_stack(xb, ob, 0, 5)
            ms = time_calls(torch, lambda s: run_stack(xb, ob, 5 + s, 1), steps)
            n_calls = steps * L
            reads = sum(int(na[l, ((5 + s) * L + l) % pool]) + shape.n_shared for s in range(steps) for l in range(L))
            res[f"k{k_use}_p{top_p}"] = {"k_use": k_use, "top_p": top_p,
                                         "tokens_per_s": round(n_calls / (ms / 1e3), 1),
                                         "us_per_layer_call": round(1e3 * ms / n_calls, 2),
                                         "mean_routed_experts_per_token": round(float(na.mean()), 2),
                                         "expert_bytes_vs_plain": round((float(na.mean()) + shape.n_shared) / (k + shape.n_shared), 4),
                                         "expert_weight_GBps": round(reads * eb / (ms / 1e3) / 1e9, 1)}
            del xb, ob
            log(f"routing limits {res[f'k{k_use}_p{top_p}']}")
        for lay in layers:
            lay.set_routing()
        result["routing_limits_decode_T1"] = {
            "note": "lossy overrides (explicit smaller k, adaptive expert top-p); the synthetic router's scores are "
                    "nearly flat, so top-p keeps more experts here than a trained router's peaked scores would",
            **res}

    # ---- prefill on its own layer ------------------------------------------
    if not args.no_extra:
        result["prefill"] = prefill(args, cm, torch, np, synth, dev)
        result["prefill"]["mfma_gemm_frac_of_measured_f16_varied"] = round(
            result["prefill"]["mfma_gemm_tflops"] / peaks["mfma_f16_varied_TFLOPs"], 4)

    if not args.no_extra:
        result["small_configs"] = small_config_rows(args, cm, torch, np, synth, dev)
        result["int8_mtp_layer"] = int8_rows(args, cm, torch, np, synth, dev)

    if not args.no_extra and not args.no_cache:
        result["expert_cache"] = cache_rows(args, cm, torch, np, synth, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, shape, layers, dev)

    print(json.dumps(result), flush=True)


def prefill(args, cm, torch, np, synth, dev):
    """T = 4096 on the GLM-like layer with Zipf-skewed expert load."""
    shape = synth.GLM_PREFILL
    T = 4096
    h, I, k = shape.hidden, shape.inter, shape.top_k
    wr, b = synth.router(shape, args.seed, 0)
    tensors = {"router_w": torch.from_numpy(wr).to(dev), "sel_bias": torch.from_numpy(b).to(dev)}
    tensors.update({n: torch.from_numpy(v).to(dev) for n, v in synth.routed_tables(shape, args.seed, 0).items()})
    tensors.update({"sh_" + n: torch.from_numpy(v).to(dev) for n, v in synth.shared_tables(shape, args.seed, 0).items()})
    cfg = cm.make_config(hidden=h, n_experts=shape.n_experts, top_k=k, inter=I, n_shared=shape.n_shared,
                         routed_scaling_factor=shape.rsf, max_tokens=T)
    lay = cm.MoELayer(cfg, tensors)
    x = torch.from_numpy(synth.hidden(shape, args.seed, T)).to(dev)
    out = torch.empty_like(x)
    for _ in range(2):
        lay(x, out)
    n = 10
    ms = time_calls(torch, lambda i: lay(x, out), n)
    _, r = lay.last_routing()
    n_active = int(r["n_active"].item())
    kern = kernel_profile(cm, [lay.handle], lambda: [lay(x, out) for _ in range(n)], n)
    flops_gu = 2 * 2 * h * I * (T * k + T * shape.n_shared)
    flops_dn = 2 * h * I * (T * k + T * shape.n_shared)
    gu = kern.get("expert_mfma_gate_up", (0.0, 1))
    dn = kern.get("expert_mfma_down", (0.0, 1))
    gu_us, dn_us = 1e3 * gu[0] / gu[1], 1e3 * dn[0] / dn[1]
    mfma_tflops = (flops_gu + flops_dn) / ((gu_us + dn_us) * 1e-6) / 1e12
    res = {"workload": f"GLM-5.2-like layer prefill T={T}, Zipf(1.1)-skewed expert load, fp16 MFMA path",
           "tokens_per_s": round(T * n / (ms / 1e3), 1),
           "ms_per_layer_call": round(ms / n, 3),
           "distinct_experts": n_active,
           "ffn_tflop_per_call": round((flops_gu + flops_dn) / 1e12, 4),
           "kernel_avg_us": {nm: round(1e3 * t / c, 2) for nm, (t, c) in kern.items()},
           "mfma_gemm_tflops": round(mfma_tflops, 1),
           "mfma_gemm_frac_of_f16_peak": round(mfma_tflops / F16_PEAK_TFLOPS, 4)}
    lay.close()
    del tensors
    log(f"prefill: {res}")
    return res


def small_config_rows(args, cm, torch, np, synth, dev):
    """The two small configurations: the tiny layer at T = 4 (launch-latency
    bound: microseconds per forward) and the OLMoE-like layer at T = 16
    (HBM-bound).  The OLMoE-like layer's 226 MB would sit in the 256 MB
    Infinity Cache, so 8 independent copies (8 seeded layers, 1.8 GB) are
    called in turn: each call's experts come from HBM.  Each layer's output
    is checked against the oracle once, outside the timed region."""
    import oracle
    res = {}
    for name, shape, T, n_layers in (("tiny", synth.TINY, 4, 1), ("olmoe_like", synth.OLMOE, 16, 8)):
        h, E, k = shape.hidden, shape.n_experts, shape.top_k
        lays, keep = [], []
        for l in range(n_layers):
            wr, b = synth.router(shape, args.seed, l)
            t = {"router_w": torch.from_numpy(wr).to(dev), "sel_bias": torch.from_numpy(b).to(dev)}
            routed = synth.routed_tables(shape, args.seed, l)
            t.update({n: torch.from_numpy(v).to(dev) for n, v in routed.items()})
            shared = synth.shared_tables(shape, args.seed, l)
            if shared is not None:
                t.update({"sh_" + n: torch.from_numpy(v).to(dev) for n, v in shared.items()})
            cfg = cm.make_config(hidden=h, n_experts=E, top_k=k, inter=shape.inter, n_shared=shape.n_shared,
                                 routed_scaling_factor=shape.rsf, max_tokens=T)
            lays.append(cm.MoELayer(cfg, t))
            keep.append(t)
            if l == 0:  # parity of the timed configuration, once
                x0 = synth.hidden(shape, args.seed, T, layer=l, batch=77)
                got = lays[0](torch.from_numpy(x0).to(dev)).cpu().numpy()
                ref, _, _ = oracle.forward(shape, wr, b, routed, shared, x0)
                den = np.maximum(np.abs(ref), np.sqrt((ref.astype(np.float64) ** 2).mean(axis=1, keepdims=True)))
                parity = float((np.abs(got - ref) / den).max())
            del routed, shared
        pool = 16
        xs = [[torch.from_numpy(synth.hidden(shape, args.seed, T, layer=l, batch=500 + i)).to(dev) for i in range(pool)]
              for l in range(n_layers)]
        out = torch.empty((T, h), dtype=torch.float32, device=dev)
        na = np.zeros((n_layers, pool), np.int64)
        for l in range(n_layers):
            for i in range(pool):
                lays[l](xs[l][i], out)
                _, r = lays[l].last_routing()
                na[l, i] = int(r["n_active"].item())
        n = max(200, args.steps)
        call = lambda c: lays[c % n_layers](xs[c % n_layers][(c // n_layers) % pool], out)
        for c in range(10):
            call(c)
        ms = time_calls(torch, call, n)
        reads = sum(int(na[c % n_layers, (c // n_layers) % pool]) + shape.n_shared for c in range(n))
        nbytes = reads * shape.expert_bytes + n * (h * E * 4)
        res[name] = {"workload": f"{name} layer h={h} E={E} k={k} I={shape.inter} shared={shape.n_shared}, T={T}"
                                 + (f", {n_layers} weight copies called in turn" if n_layers > 1 else ""),
                     "tokens_per_s": round(T * n / (ms / 1e3), 1), "us_per_call": round(1e3 * ms / n, 3),
                     "mean_distinct_experts": round(float(na.mean()), 2),
                     "weights_GBps": round(nbytes / (ms / 1e3) / 1e9, 1),
                     "weights_frac_of_hbm_peak": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "max_rel_err_vs_oracle": parity}
        log(f"{name}: {res[name]}")
        for lay in lays:
            lay.close()
        del lays, keep, xs
    return res


def int8_rows(args, cm, torch, np, synth, dev):
    """The GLM-like layer with int8 tables (one scale per row, the multi-token
    prediction head's format), resident: draft (T = 1) and verify (T = 2..4)
    calls on a pool of fresh inputs; tokens/s, expert-weight GB/s, and the
    gate/up launch's algorithmic bytes over its HIP-event time."""
    shape = synth.GLM_MTP_I8
    h, I, E, k = shape.hidden, shape.inter, shape.n_experts, shape.top_k
    t0 = time.time()
    wr, b = synth.router(shape, args.seed, 0)
    tensors = {"router_w": torch.from_numpy(wr).to(dev), "sel_bias": torch.from_numpy(b).to(dev)}
    tensors.update({n: torch.from_numpy(v).to(dev) for n, v in synth.routed_tables(shape, args.seed, 0).items()})
    tensors.update({"sh_" + n: torch.from_numpy(v).to(dev) for n, v in synth.shared_tables(shape, args.seed, 0).items()})
    cfg = cm.make_config(hidden=h, n_experts=E, top_k=k, inter=I, n_shared=shape.n_shared,
                         routed_scaling_factor=shape.rsf, max_tokens=4, weight_format=cm.COLI_MOE_WEIGHTS_INT8_ROW)
    lay = cm.MoELayer(cfg, tensors)
    log(f"int8 MTP layer resident ({time.time() - t0:.1f} s)")
    eb = shape.expert_bytes
    gate_up_w = 2 * (I * h + 4 * I)
    res = {"workload": f"GLM-5.2-like MoE layer with int8 tables (scale per row), h={h} E={E} k={k} I={I}, 1 layer resident",
           "expert_bytes": eb}
    pool = 32
    for T in (1, 2, 3, 4):
        xs = [torch.from_numpy(synth.hidden(shape, args.seed, T, batch=9000 + 100 * T + i)).to(dev) for i in range(pool)]
        out = torch.empty((T, h), dtype=torch.float32, device=dev)
        na = []
        for x in xs:
            lay(x, out)
            _, r = lay.last_routing()
            na.append(int(r["n_active"].item()))
        n = max(40, args.steps)
        for i in range(5):
            lay(xs[i % pool], out)
        ms = time_calls(torch, lambda i: lay(xs[i % pool], out), n)
        reads = sum(na[i % pool] + shape.n_shared for i in range(n))
        kern = kernel_profile(cm, [lay.handle], lambda: [lay(xs[i % pool], out) for i in range(n)], n)
        gu = kern.get("expert_gemv_gate_up", (0.0, 1))
        dn = kern.get("expert_gemv_down", (0.0, 1))
        gu_us, dn_us = 1e3 * gu[0] / gu[1], 1e3 * dn[0] / dn[1]
        mean_e = float(np.mean(na)) + shape.n_shared
        gu_bytes = mean_e * gate_up_w + T * (3 * h + h // 8) + (T * k + T * shape.n_shared) * I * 4
        row = {"tokens_per_s": round(T * n / (ms / 1e3), 1), "us_per_call": round(1e3 * ms / n, 2),
               "mean_distinct_experts": round(float(np.mean(na)), 2),
               "expert_weight_GBps": round(reads * eb / (ms / 1e3) / 1e9, 1),
               "kernel_avg_us": {nm: round(1e3 * t / c, 2) for nm, (t, c) in kern.items()},
               "gate_up_GBps": round(gu_bytes / gu_us / 1e3, 1),
               "gate_up_frac_of_hbm_peak": round(gu_bytes / gu_us / 1e3 / HBM_PEAK_GBPS, 4),
               "down_GBps": round((mean_e * h * (I + 4) + (T * k + T) * I * 4) / dn_us / 1e3, 1)}
        res[f"T{T}"] = row
        log(f"int8 MTP layer T={T}: {row}")
        del xs
    lay.close()
    del tensors
    return res


def cache_rows(args, cm, torch, np, synth, dev):
    """The GLM-like layer with its 256 routed experts in pinned host memory
    and an HBM expert cache of n slots, decode T = 1 on fresh N(0,1) inputs
    (uniform routing, the hardest case for a cache): tokens/s against the
    hit rate, and the host -> HBM copy rate.  Then router look-ahead prefetch
    on two such layers whose inputs are correlated like consecutive layers of
    a residual stream (x1 = x0 + 0.2 N(0,1)): the pair's tokens/s with and
    without it, and its recall."""
    shape = synth.GLM
    h, E, k, I = shape.hidden, shape.n_experts, shape.top_k, shape.inter
    eb = shape.expert_bytes

    def host_layer(layer):
        routed = synth.routed_tables(shape, args.seed, layer)
        host = {n: torch.from_numpy(v).pin_memory() for n, v in routed.items()}
        del routed
        wr, b = synth.router(shape, args.seed, layer)
        res = {"router_w": torch.from_numpy(wr).to(dev), "sel_bias": torch.from_numpy(b).to(dev)}
        res.update({"sh_" + n: torch.from_numpy(v).to(dev) for n, v in synth.shared_tables(shape, args.seed, layer).items()})
        return res, host

    cfg = cm.make_config(hidden=h, n_experts=E, top_k=k, inter=I, n_shared=shape.n_shared,
                         routed_scaling_factor=shape.rsf, max_tokens=1)
    t0 = time.time()
    res0, host0 = host_layer(0)
    log(f"cache bench: layer 0 in pinned host memory ({time.time() - t0:.1f} s)")
    xs = [torch.from_numpy(synth.hidden(shape, args.seed, 1, layer=0, batch=5000 + i)).to(dev) for i in range(64)]
    out = torch.empty((1, h), dtype=torch.float32, device=dev)
    rows = []
    for n_slots in (256, 128, 64, 32):
        C = cm.ExpertCache(cfg, res0, host0, n_slots)
        warm = 256 if n_slots == E else 32
        for i in range(warm):
            C(xs[i % 64], out)
        torch.cuda.synchronize()
        s0 = C.stats()
        n = 64
        t = time.perf_counter()
        for i in range(n):
            C(xs[(warm + i) % 64], out)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t
        s1 = C.stats()
        need = s1["needed"] - s0["needed"]
        hits = s1["hits"] - s0["hits"]
        copied = s1["bytes_copied"] - s0["bytes_copied"]
        rows.append({"n_slots": n_slots, "hbm_GB": round(n_slots * eb / 1e9, 2), "tokens_per_s": round(n / dt, 1),
                     "us_per_call": round(1e6 * dt / n, 1), "hit_rate": round(hits / need, 4),
                     "host_to_hbm_GBps": round(copied / dt / 1e9, 2)})
        log(f"cache {rows[-1]}")
        C.close()
        del C
    # PILOT on two correlated layers, 32 slots each
    res1, host1 = host_layer(1)
    rng = np.random.default_rng(args.seed)
    pairs = []
    for i in range(64):
        x0 = synth.hidden(shape, args.seed, 1, layer=0, batch=6000 + i)
        x1 = (x0 + 0.2 * rng.standard_normal(x0.shape)).astype(np.float32)
        pairs.append((torch.from_numpy(x0).to(dev), torch.from_numpy(x1).to(dev)))
    pilot = {}
    for use in (False, True):
        C0, C1 = cm.ExpertCache(cfg, res0, host0, 32), cm.ExpertCache(cfg, res1, host1, 32)

        def step(i):
            x0, x1 = pairs[i % 64]
            if use:
                C1.prefetch(x0, k)
            C0(x0, out)
            C1(x1, out)

        for i in range(16):
            step(i)
        torch.cuda.synchronize()
        a0, b0 = C1.stats(), C0.stats()
        n = 48
        t = time.perf_counter()
        for i in range(n):
            step(16 + i)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t
        a1 = C1.stats()
        key = "with_prefetch" if use else "without_prefetch"
        pilot[key] = {"tokens_per_s_two_layers": round(n / dt, 1), "us_per_token_two_layers": round(1e6 * dt / n, 1),
                      "layer1_hit_rate": round((a1["hits"] - a0["hits"]) / (a1["needed"] - a0["needed"]), 4)}
        if use:
            pilot[key]["layer1_prefetch_recall"] = round(
                (a1["prefetch_hits"] - a0["prefetch_hits"]) / (a1["needed"] - a0["needed"]), 4)
        log(f"pilot {key}: {pilot[key]}")
        C0.close()
        C1.close()
    del host0, host1
    return {"workload": "GLM-5.2-like layer, 256 routed experts (21.2 MB each) in pinned host memory, "
                        "decode T=1 on fresh N(0,1) inputs (uniform routing)",
            "expert_bytes": eb, "slots": rows,
            "router_lookahead_prefetch": dict(pilot, slots_per_layer=32,
                                              inputs="x1 = x0 + 0.2 N(0,1) (consecutive-layer correlation)")}


def host_cpu():
    """The host's CPU as lscpu and /proc/cpuinfo describe it: model string,
    sockets, physical cores, logical CPUs."""
    import subprocess
    info = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        kv = dict(ln.split(":", 1) for ln in out.splitlines() if ":" in ln)
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        info["model_name"] = kv.get("Model name", "")
        for key, name in (("Socket(s)", "sockets"), ("Core(s) per socket", "cores_per_socket"),
                          ("Thread(s) per core", "threads_per_core"), ("CPU(s)", "logical_cpus")):
            if kv.get(key, "").isdigit():
                info[name] = int(kv[key])
        if "sockets" in info and "cores_per_socket" in info:
            info["physical_cores"] = info["sockets"] * info["cores_per_socket"]
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    try:
        cores, fields = set(), {}
        phys = None
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ":" not in ln:
                    continue
                k, v = (x.strip() for x in ln.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping") and k not in fields:
                    fields[k] = v
                if k == "physical id":
                    phys = v
                if k == "core id":
                    cores.add((phys, v))
        info["cpuinfo"] = fields
        if cores and "physical_cores" not in info:
            info["physical_cores"] = len(cores)
    except OSError:
        pass
    info["affinity_cpus"] = len(os.sched_getaffinity(0))
    return info


def cpu_baseline(args, shape, layers, dev):
    """The oracle, as it stands, on a bounded sample of the same workload:
    single decode tokens of layer 0, until the time budget is spent.  The
    GPU's outputs for the same tokens are compared on the way (max relative
    error, floored at the row RMS)."""
    import numpy as np
    import torch

    import oracle
    import synth

    wr, b = synth.router(shape, args.seed, 0)
    shared = synth.shared_tables(shape, args.seed, 0)
    done, spent, worst = 0, 0.0, 0.0
    cache = {}
    out = torch.empty((1, shape.hidden), dtype=torch.float32, device=dev)
    while spent < args.cpu_seconds and done < 512:
        x = synth.hidden(shape, args.seed, 1, layer=0, batch=1000 + done)
        idx, _ = oracle.route(shape, wr, b, x)
        for e in np.unique(idx):
            if int(e) not in cache:
                cache[int(e)] = synth.expert(shape, args.seed, int(e), 0)
        routed = [cache.get(e) for e in range(shape.n_experts)]
        t0 = time.perf_counter()
        ref, _, _ = oracle.forward(shape, wr, b, routed, shared, x)
        spent += time.perf_counter() - t0
        layers[0](torch.from_numpy(x).to(dev), out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        r = ref.astype(np.float64)
        rms = np.sqrt((r ** 2).mean(axis=-1, keepdims=True))
        worst = max(worst, float((np.abs(got - r) / np.maximum(np.abs(r), rms)).max()))
        done += 1
    cpu = host_cpu()
    return {"value": round(done / spent, 4), "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "cores_meaning": "OpenMP threads the oracle ran on (one per logical CPU it may use)",
            "host_cpu": cpu,
            "sample": f"{done} decode calls of T=1 on layer 0 (routing + 8 routed + shared expert "
                      f"FFNs in float64), {spent:.1f} s",
            "gpu_max_rel_err_on_sample": worst}


if __name__ == "__main__":
    main()
