"""Benchmark: multi-adapter LoRA linear on one MI355X.

One step = the whole hot path over one decode batch of the 70B-shaped
projections: the q (8192 -> 8192) and v (8192 -> 1024) LoRA linear layers
of one attention layer, for 512 rows with 12 adapters of rank {4 x3, 16 x6,
64 x3} (alpha = 2r, Zipf 1.1 popularity, 10% rows without adapter), bf16
with fp32 accumulation.  Both projections share x and the per-row adapter
ids, so they run as one multi-slice call: plan, one base GEMM over the
stacked [9216, 8192] weight (256 x 144 tiles, each computed by two
workgroups over the two halves of k) that also computes the shrink
(t = x A^T for every adapter rank, folded into its tiles), one expand.  The shrink as its
own kernel (x read once for both slices) is timed in a second pass with the
folding turned off (kernels.separate_shrink_step, kernels.shrink_gbs).

Inputs are seeded synthetic tensors already resident in HBM.  The step
rotates over several independent buffer sets (x, W_q, W_v, adapter slots,
outputs; ~1.6 GB total), so weights are not served from the 256 MiB
Infinity Cache between steps.

Prints one JSON line (rank 0):
  value      = tokens/s through the (q + v) pair = 512 * steps / elapsed
  roofline   = base GEMM (the dominant kernel) MFMA TFLOP/s vs the bf16 peak,
               from per-launch HIP events recorded on the launch stream
               (with the shrink folded in, its flops count too)
  cpu_baseline = the fp64 oracle on a bounded row sample, on the host cores
  adapter_activation = host-to-device loading of the same adapters through
               the pool manager (GB/s against the PCIe 5.0 x16 link)
  merge      = lora_merge (W' = W + s B A) at the q and v shapes, HBM GB/s
  quantized_base = the same step over INT8 / INT4 base weights
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_c3_gemm.json")
GEMM_SOURCE = os.path.join(ROOT, "lora_row_adapter_amd", "csrc", "gemm.hip")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU reaches its steady clock only after some hundreds of steps
    # (measured: 20 warmup steps understate throughput by ~4%)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--sets", type=int, default=8, help="rotating buffer sets")
    ap.add_argument("--path", default="auto", choices=["auto", "gather", "sgmv"])
    ap.add_argument("--storage", default="slots", choices=["slots", "pool"],
                    help="adapter storage of the timed step: rank-padded slots, or a paged pool "
                         "of 2 MiB pages (unpadded A and B)")
    ap.add_argument("--settle-ms", type=float, default=1500.0,
                    help="untimed steps run for this long before the warmup, so the shader clock "
                         "has settled whatever --warmup is (0: none)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-activation", action="store_true",
                    help="skip the adapter-activation (host-to-device) measurement")
    ap.add_argument("--no-merge", action="store_true",
                    help="skip the merged-weight (lora_merge) measurement")
    ap.add_argument("--no-quant", action="store_true",
                    help="skip the INT8 / INT4 base-weight measurement")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the decode-4096, prefill and paged-pool workloads")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="write profiles/ summaries from a rocprofv3 run whose trace/, fetch/, "
                         "write/, cfetch/, cwrite/ output directories are under DIR, and exit")
    ap.add_argument("--profiled-command", default="python3 bench.py --no-cpu-baseline --steps 20",
                    help="the bench command the profiling run used (recorded in the summary)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-sized device buffer 5 times (scales the FETCH_SIZE / "
                         "WRITE_SIZE counters of a profiling run) and exit")
    return ap.parse_args()


def copy_calibration(mib):
    """A plain device-to-device copy of known size, for counter calibration."""
    n = int(mib) << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.summarize_profiles:
        from lora_row_adapter_amd import profile_tools
        res = profile_tools.summarize(args.summarize_profiles, os.path.join(ROOT, "profiles"),
                                      args.profiled_command, 256, GEMM_SOURCE,
                                      "c3_proj70b_bf16 q+v, 512 rows")
        print(json.dumps({k: v for k, v in res.items() if k != "kernel_trace"}, indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU (--gpus %d requested): the layer is row-independent, "
              "and a run over several GPUs is not provided."
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import lora_row_adapter_amd as lr
    from lora_row_adapter_amd import workloads as wl

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    lr.load_library()
    path = {"auto": lr.PATH_AUTO, "gather": lr.PATH_GATHER, "sgmv": lr.PATH_SGMV}[args.path]

    log("generating c3_proj70b_bf16")
    w = wl.c3_proj70b_bf16()
    M, k = w.M, w.k
    pq, pv = w.proj("q"), w.proj("v")
    ids = torch.from_numpy(w.ids).to(dev)
    scales = torch.from_numpy(w.scales).to(dev)
    ranks = torch.from_numpy(w.ranks).to(dev)

    def slot_adapters(p):
        A, B = wl.slots(w, p)
        return A.to(dev), B.to(dev)

    def pool_adapters(p, i):
        pool, table, _n = wl.pool(w, p, page_bytes=2 << 20, seed_offset=i)
        return pool.to(dev), table.to(dev)

    base = {"x": w.x.to(dev), "W": torch.cat([pq.W, pv.W], dim=0).contiguous().to(dev)}
    if args.storage == "slots":
        base["Aq"], base["Bq"] = slot_adapters(pq)
        base["Av"], base["Bv"] = slot_adapters(pv)
    else:
        base["Pq"], base["Tq"] = pool_adapters(pq, 0)
        base["Pv"], base["Tv"] = pool_adapters(pv, 1)
    sets = []
    for i in range(args.sets):
        s = {kk: (v if i == 0 else v.clone()) for kk, v in base.items()}
        if args.storage == "slots":
            s["slices"] = [lr.Slice(pq.d, lr.Adapters.slots(s["Aq"], s["Bq"], ranks), scales),
                           lr.Slice(pv.d, lr.Adapters.slots(s["Av"], s["Bv"], ranks), scales)]
        else:
            s["slices"] = [lr.Slice(pq.d, lr.Adapters.paged(s["Pq"], s["Tq"], ranks, 2 << 20,
                                                            w.max_rank), scales),
                           lr.Slice(pv.d, lr.Adapters.paged(s["Pv"], s["Tv"], ranks, 2 << 20,
                                                            w.max_rank), scales)]
        s["y"] = torch.empty(M, pq.d + pv.d, dtype=torch.bfloat16, device=dev)
        sets.append(s)
    set_bytes = sum(v.numel() * v.element_size() for kk, v in sets[0].items() if torch.is_tensor(v))
    ws = torch.zeros(lr.workspace_bytes_sliced(M, k, torch.bfloat16, sets[0]["slices"]),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log("%d buffer sets of %.0f MB" % (args.sets, set_bytes / 1e6))

    stream = torch.cuda.current_stream()

    def step(i, flags=0):
        s = sets[i % len(sets)]
        lr.lora_linear_sliced(s["x"], s["W"], s["slices"], ids, y=s["y"], workspace=ws, path=path,
                              flags=flags, stream=stream)

    def profiled(n, flags=0):
        """n steps under the library's per-launch events (library-side, on
        the launch stream); kernel class -> {ms, launches}, wall seconds."""
        with lr.Profiler():
            t1 = time.perf_counter()
            for i in range(n):
                step(i, flags)
            prof = lr.Profiler.read(reset=True)
            torch.cuda.synchronize()
            return prof, time.perf_counter() - t1

    # settle: untimed steps until the clock holds steady (measured: with 20
    # warmup steps and no settling the figure reads ~4% low)
    settle_steps = 0
    if args.settle_ms > 0:
        t_s = time.perf_counter()
        while (time.perf_counter() - t_s) * 1e3 < args.settle_ms:
            for i in range(50):
                step(settle_steps + i)
            settle_steps += 50
            torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = M * args.steps / elapsed
    y_timed = sets[(args.steps - 1) % len(sets)]["y"].clone()  # the last timed step's output
    device_errors = lr.lora_check(ws, stream=stream)
    log("timed: %.3f ms/step, %.3g tokens/s" % (ms_per_step, value))

    # the same steps again with per-launch events (library-side, on the
    # launch stream) for per-kernel durations
    # (at most 400 steps: the library's event ring holds 8192 launches)
    prof_steps = min(args.steps, 400)
    prof, ev_elapsed = profiled(prof_steps)
    per = {kname: prof[kname]["ms"] * 1e3 / max(prof[kname]["launches"], 1)
           for kname in lr.KERNEL_CLASSES}
    launches = {kname: prof[kname]["launches"] for kname in lr.KERNEL_CLASSES}
    log("per-launch us: " + json.dumps({k_: round(v, 2) for k_, v in per.items()}))
    # the same steps reusing the plan already in the workspace (same ids): the
    # base GEMM launch without the plan it otherwise carries
    rprof, _ = profiled(prof_steps, lr.FLAG_REUSE_PLAN)
    gemm_us_reused = rprof["gemm"]["ms"] * 1e3 / max(rprof["gemm"]["launches"], 1)
    log("gemm us with the plan reused: %.2f" % gemm_us_reused)

    # per-step GPU time from events between steps on the stream (rotating
    # buffer sets, as timed), and the same with one buffer set only (warm:
    # x, W and the adapters stay in the Infinity Cache, as for a layer whose
    # input was just written)
    def step_times(n, same_set):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        evs[0].record(stream)
        for i in range(n):
            step(0 if same_set else i)
            evs[i + 1].record(stream)
        evs[-1].synchronize()
        return np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n)])
    cold = step_times(prof_steps, False)
    warm = step_times(prof_steps, True)

    def dist(a):
        return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
                "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}
    step_us = {"rotating_sets": dist(cold), "warm_same_buffer": dist(warm),
               "tokens_per_s_at_median": round(M / (np.median(cold) * 1e-6), 1),
               "warm_tokens_per_s_at_median": round(M / (np.median(warm) * 1e-6), 1),
               "what": "GPU time per step between events on the launch stream; rotating_sets = the "
                       "timed configuration, warm_same_buffer = one buffer set reused (inputs resident "
                       "in the Infinity Cache)"}
    log("step us: " + json.dumps(step_us))

    bq = wl.algorithmic_bytes(w, pq)
    bv = wl.algorithmic_bytes(w, pv)
    # no shrink launch: the library folded the shrink into the base GEMM,
    # which then also does the shrink's algorithmic work
    folded = prof["shrink"]["launches"] + prof["sgmv_shrink"]["launches"] == 0
    gemm_flops = bq["gemm_flops"] + bv["gemm_flops"]
    gemm_alg_flops = gemm_flops + (bq["shrink_flops"] + bv["shrink_flops"] if folded else 0.0)
    gemm_us_step = prof["gemm"]["ms"] * 1e3 / prof_steps
    gemm_tflops = gemm_alg_flops / (gemm_us_step * 1e-6) / 1e12
    expand_us_step = (prof["expand"]["ms"] + prof["sgmv_expand"]["ms"]) * 1e3 / prof_steps
    expand_gbs = (bq["expand_bytes"] + bv["expand_bytes"]) / (expand_us_step * 1e-6) / 1e9
    kernel_us_step = sum(prof[kname]["ms"] for kname in lr.KERNEL_CLASSES) * 1e3 / prof_steps
    # the shrink as its own kernel: the same steps with the folding turned off
    # (the multi-slice shrink reads x once for both projections)
    x_bytes = bq["M_a"] * k * 2
    shrink_bytes = bq["shrink_bytes"] + bv["shrink_bytes"] - x_bytes
    for i in range(min(args.warmup, 500)):
        step(i, lr.FLAG_SEPARATE_SHRINK)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(prof_steps):
        step(i, lr.FLAG_SEPARATE_SHRINK)
    torch.cuda.synchronize()
    sep_ms = (time.perf_counter() - t2) * 1e3 / prof_steps
    sprof, _ = profiled(prof_steps, lr.FLAG_SEPARATE_SHRINK)
    shrink_us_step = (sprof["shrink"]["ms"] + sprof["sgmv_shrink"]["ms"]) * 1e3 / prof_steps
    shrink_gbs = shrink_bytes / (shrink_us_step * 1e-6) / 1e9
    separate = {
        "flags": "LORA_FLAG_SEPARATE_SHRINK",
        "ms_per_step": round(sep_ms, 4),
        "tokens_per_s": M / (sep_ms * 1e-3),
        "per_launch_us": {k_: round(sprof[k_]["ms"] * 1e3 / sprof[k_]["launches"], 3)
                          for k_ in lr.KERNEL_CLASSES if sprof[k_]["launches"]},
    }
    log("separate shrink: %.3f ms/step, per-launch us %s" % (sep_ms, json.dumps(separate["per_launch_us"])))

    traffic = None
    try:
        t = json.load(open(TRAFFIC_FILE))
        src_sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
        if t.get("source_sha256") == src_sha:
            traffic = t["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        traffic = None

    result = {
        "metric": "LoRA-linear tokens/s; shrink/expand HBM GB/s and base-GEMM TFLOP/s vs peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "c3_proj70b_bf16: q 8192->8192 and v 8192->1024 LoRA linear, 512 decode "
                        "rows, 12 adapters ranks 4x3/16x6/64x3 alpha=2r, Zipf(1.1), 10% none",
            "M": M, "k": k, "d_q": pq.d, "d_v": pv.d, "n_adapters": w.S, "max_rank": w.max_rank,
            "adapter_storage": args.storage, "path": args.path, "buffer_sets": args.sets,
            "call": "lora_linear_sliced (q and v slices, W stacked [9216, 8192])",
            "buffer_set_mb": round(set_bytes / 1e6, 1),
        },
        "roofline": {
            "kernel": ("k_gemm_bf16_split<144, true, 2> (base GEMM over the stacked q+v weight as split-K "
                       "workgroup pairs, shrink folded in; achieved counts the base GEMM's and the "
                       "shrink's algorithmic flops)"
                       if folded else "k_gemm_bf16_split<144, false, 2> (base GEMM over the stacked q+v "
                       "weight as split-K workgroup pairs)"),
            "bound": "mfma",
            "achieved": gemm_tflops,
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": gemm_tflops / BF16_PEAK_TFLOPS,
            "traffic": traffic,
        },
        "kernels": {
            "per_launch_us": {k_: round(v, 3) for k_, v in per.items() if launches[k_]},
            "launches_per_step": {k_: launches[k_] / prof_steps for k_ in launches if launches[k_]},
            "kernel_us_per_step": round(kernel_us_step, 3),
            "event_pass_ms_per_step": round(ev_elapsed * 1e3 / prof_steps, 4),
            "tokens_per_s_from_kernel_sum": M / (kernel_us_step * 1e-6),
            "gemm_tflops": round(gemm_tflops, 1),
            "gemm_us_plan_reused": round(gemm_us_reused, 2),
            "plan_in_gemm_us": round(per["gemm"] - gemm_us_reused, 2),
            "shrink_folded_into_gemm": folded,
            "shrink_gbs": round(shrink_gbs, 1),
            "shrink_frac_hbm": round(shrink_gbs / HBM_PEAK_GBS, 4),
            "shrink_measured_in": "separate-shrink pass (the shrink kernel alone)",
            "separate_shrink_step": separate,
            "expand_gbs": round(expand_gbs, 1),
            "expand_frac_hbm": round(expand_gbs / HBM_PEAK_GBS, 4),
            "algorithmic": {"q": bq, "v": bv, "fused_shrink_bytes": shrink_bytes},
        },
        "step_us": step_us,
        "device_errors": device_errors,
        "settle": {"steps": settle_steps, "ms": args.settle_ms},
    }
    if not args.no_others:
        result["gather_path"] = gather_path(lr, wl, w, sets, ids, ws, stream, step)

    if not args.no_activation:
        result["adapter_activation"] = adapter_activation(lr, w, pq, pv, stream)
    if not args.no_merge:
        result["merge"] = merge_rate(lr, w, pq, pv, sets, stream)
    if not args.no_quant:
        result["quantized_base"] = quantized_rate(lr, wl, w, sets, ids, ws, stream, args)
    if not args.no_others:
        result["other_configs"] = other_configs(lr, wl, stream)
    if not args.no_cpu_baseline:
        y_last = y_timed.double().cpu().numpy()
        result["cpu_baseline"], result["output_check"] = cpu_baseline(w, pq, pv, args.cpu_seconds,
                                                                      y_last)
        result["oracle_seconds"] = oracle_seconds(wl, w)
    print(json.dumps(result), flush=True)


def other_configs(lr, wl, stream, n_sets=4, steps=200, warmup=100):
    """The other seeded workloads, one lora_linear call per step, rotating x,
    W and y over n_sets buffer sets (adapters: one copy -- the c4 pool holds
    1024 adapters in 2 MiB pages):
      c1_decode_bf16   256 rows, d = k = 4096, 4 slots of rank 16
      c2_prefill_bf16  8 x 1024 rows, d = k = 4096, ranks 8..64 padded to 64,
                       one adapter per sequence (contiguous runs: 64-row SGMV items)
      c4_paged_bf16    2048 rows from 256 sequences, d = k = 5120, 1024 adapters
                       of rank 16 in a paged pool, ~131 present
    Per workload: tokens/s, event-timed launches, the base GEMM's TFLOP/s and
    the shrink / expand GB/s against the algorithmic bytes of the instance.
    The base GEMM's launch carries the layer's plan; its TFLOP/s is taken
    from a pass that reuses the plan already in the workspace (the launch
    without it), and plan_in_gemm_us is what carrying the plan adds."""
    dev = torch.device("cuda:0")
    out = {}
    for name, make, storage in (("c1_decode_bf16", wl.c1_decode_bf16, "slots"),
                                ("c2_prefill_bf16", wl.c2_prefill_bf16, "slots"),
                                ("c4_paged_bf16", wl.c4_paged_bf16, "pool")):
        w = make()
        p = w.projections[0]
        M = w.M
        ids = torch.from_numpy(w.ids).to(dev)
        scales = torch.from_numpy(w.scales).to(dev)
        ranks = torch.from_numpy(w.ranks).to(dev)
        if storage == "slots":
            A, B = wl.slots(w, p)
            ad = lr.Adapters.slots(A.to(dev), B.to(dev), ranks)
        else:
            pool, table, _ = wl.pool(w, p)
            ad = lr.Adapters.paged(pool.to(dev), table.to(dev), ranks, w.page_bytes, w.max_rank)
        x0, W0 = w.x.to(dev), p.W.to(dev)
        xs = [x0] + [x0.clone() for _ in range(n_sets - 1)]
        Ws = [W0] + [W0.clone() for _ in range(n_sets - 1)]
        ys = [torch.empty(M, p.d, dtype=w.dtype, device=dev) for _ in range(n_sets)]
        ws = lr.new_workspace(M, p.d, w.k, w.dtype, ad, device=dev)

        def step(i, flags=0):
            lr.lora_linear(xs[i % n_sets], Ws[i % n_sets], ad, ids, scales, y=ys[i % n_sets],
                           workspace=ws, flags=flags, stream=stream)
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0

        def profiled(flags=0):
            with lr.Profiler():
                for i in range(steps):
                    step(i, flags)
                prof = lr.Profiler.read(reset=True)
                torch.cuda.synchronize()
            return {kn: prof[kn]["ms"] * 1e3 / prof[kn]["launches"] for kn in lr.KERNEL_CLASSES
                    if prof[kn]["launches"]}
        per = profiled()
        # the same steps reusing the plan already in the workspace: the base
        # GEMM launch without the plan it otherwise carries
        per_reuse = profiled(lr.FLAG_REUSE_PLAN)
        alg = wl.algorithmic_bytes(w, p)
        shr = per.get("sgmv_shrink", per.get("shrink"))
        exp = per.get("sgmv_expand", per.get("expand"))
        gemm = per_reuse.get("gemm")
        out[name] = {
            "rows": M, "d": p.d, "k": w.k, "adapter_storage": storage, "n_present": alg["n_present"],
            "adapted_rows": alg["M_a"],
            "tokens_per_s": round(M * steps / el, 1), "ms_per_step": round(el * 1e3 / steps, 4),
            "per_launch_us": {kn: round(v, 2) for kn, v in per.items()},
            "gemm_us_plan_reused": round(gemm, 2) if gemm else None,
            "plan_in_gemm_us": round(per["gemm"] - gemm, 2) if gemm and "gemm" in per else None,
            "gemm_tflops": round(alg["gemm_flops"] / gemm / 1e6, 1) if gemm else None,
            "gemm_frac_bf16_peak": round(alg["gemm_flops"] / gemm / 1e6 / BF16_PEAK_TFLOPS, 4) if gemm else None,
            "shrink_gbs": round(alg["shrink_bytes"] / shr / 1e3, 1) if shr else None,
            "expand_gbs": round(alg["expand_bytes"] / exp / 1e3, 1) if exp else None,
        }
        log("%s: %s" % (name, json.dumps(out[name])))
        del xs, Ws, ys, ws, ad
        torch.cuda.empty_cache()
    return out


def quantized_rate(lr, wl, w, sets, ids, ws, stream, args):
    """The same q+v step over an INT8 (per-row scales) and an INT4 (per-row,
    per-128-k-group scales) stacked base weight: lora_linear_sliced_q with
    the buffer sets' x, adapters and outputs, each set with its own
    quantized weight copy; tokens/s and the base GEMM's event-timed launch."""
    out = {}
    M = w.M
    steps = max(100, args.steps // 2)
    for fmt, group in (("int8", 0), ("int4", 128)):
        q, s = wl.quantized_base(w, fmt, group=group or 128, names=["q", "v"])
        code = lr.W_INT8 if fmt == "int8" else lr.W_INT4
        qws = [lr.QWeight(code, q.cuda(), s.cuda(), w.k, group=group) for _ in range(len(sets))]

        def step(i):
            st_ = sets[i % len(sets)]
            lr.lora_linear_sliced_q(st_["x"], qws[i % len(qws)], st_["slices"], ids, y=st_["y"],
                                    workspace=ws, stream=stream)
        for i in range(max(200, args.warmup // 4)):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        with lr.Profiler():
            for i in range(200):
                step(i)
            prof = lr.Profiler.read(reset=True)
            torch.cuda.synchronize()
        gemm_us = prof["gemm"]["ms"] * 1e3 / max(prof["gemm"]["launches"], 1)
        flops = 2.0 * M * q.shape[0] * w.k
        wbytes = q.numel() + s.numel() * 4
        out[fmt] = {"tokens_per_s": round(M * steps / el, 1), "ms_per_step": round(el * 1e3 / steps, 4),
                    "gemm_us": round(gemm_us, 2), "gemm_tflops": round(flops / gemm_us / 1e6, 1),
                    "weight_bytes": int(wbytes), "group": group or None}
    log("quantized base: " + json.dumps(out))
    return out


def merge_rate(lr, w, pq, pv, sets, stream, reps=20):
    """lora_merge at the 70B shapes: W' = W + s B A for the q (8192 x 8192)
    and v (1024 x 8192) weights, adapters of rank 16 and 64, out of place,
    rotating over the buffer sets' weights; HBM bytes per launch = read W +
    write W' + A and B once."""
    out = {}
    Wq_all = [s_["W"][:pq.d] for s_ in sets]
    Wv_all = [s_["W"][pq.d:] for s_ in sets]
    for name, p, Ws, sl in (("q", pq, Wq_all, 0), ("v", pv, Wv_all, 1)):
        dsts = [torch.empty_like(Ws[0]) for _ in range(2)]
        for a in (3, 9):  # ranks 16 and 64
            r = int(w.ranks[a])

            def go(i):
                s_ = sets[i % len(sets)]
                lr.lora_merge(Ws[i % len(Ws)], s_["slices"][sl].adapters, a,
                              s_["slices"][sl].scales, out=dsts[i % 2], stream=stream)
            for i in range(4):
                go(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(reps):
                go(i)
            e1.record(stream)
            e1.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            nbytes = (2 * p.d * w.k + r * (w.k + p.d)) * 2
            gbs = nbytes / us / 1e3
            out["%s_r%d" % (name, r)] = {"us": round(us, 2), "gbs": round(gbs, 1),
                                         "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                                         "bytes": nbytes}
    log("merge: " + json.dumps(out))
    return out


def adapter_activation(lr, w, pq, pv, stream, page_bytes=65536, reps=20):
    """Host-to-device activation of the workload's 12 adapters (q and v
    weights) into two managed pools of 64 KiB pages, from pinned host memory.

    warm: one batch per pool, every adapter reloaded in place (rows kernel +
          copy kernel);
    cold: every adapter evicted, then one batch per pool (placement too);
    single_calls: warm, but one lora_pool_load call per adapter;
    copy: one plain pinned-to-device copy of the same number of bytes."""
    pools, host = [], []
    total = 0
    for p in (pq, pv):
        pages = [-(-int(r) * (w.k + p.d) * 2 // page_bytes) for r in w.ranks]
        pools.append(lr.AdapterPool(sum(pages), page_bytes, w.S, max(pages), w.max_rank, w.k, p.d,
                                    dtype=torch.bfloat16, device="cuda", stream=stream))
        host.append([(p.A[s].pin_memory(), p.B[s].pin_memory()) for s in range(w.S)])
        total += sum(int(r) * (w.k + p.d) * 2 for r in w.ranks)

    def load_all(evict_first, batch=True):
        for pool, hs in zip(pools, host):
            if evict_first:
                for s in range(w.S):
                    pool.evict(s, stream=stream)
            if batch:
                pool.load_batch([(s, A, B) for s, (A, B) in enumerate(hs)], stream=stream)
            else:
                for s, (A, B) in enumerate(hs):
                    pool.load(s, A, B, stream=stream)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        host_us = (time.perf_counter() - t0) * 1e6 / reps
        return e0.elapsed_time(e1) * 1e3 / reps, host_us

    warm_us, warm_host = timed(lambda: load_all(False))
    cold_us, cold_host = timed(lambda: load_all(True))
    single_us, single_host = timed(lambda: load_all(False, batch=False))
    src = torch.empty(total, dtype=torch.uint8).pin_memory()
    dst = torch.empty(total, dtype=torch.uint8, device="cuda")
    copy_us, _ = timed(lambda: dst.copy_(src, non_blocking=True))
    st = [pl.stats() for pl in pools]
    peak = 64.0  # PCIe 5.0 x16, one direction
    res = {
        "what": "H2D activation of the 12 q+v adapters (%.2f MB) into managed 64 KiB-page pools, "
                "pinned host source, %d reps" % (total / 1e6, reps),
        "bytes": total,
        "warm_us": round(warm_us, 2), "warm_gbs": round(total / warm_us / 1e3, 2),
        "cold_us": round(cold_us, 2), "cold_gbs": round(total / cold_us / 1e3, 2),
        "single_calls_us": round(single_us, 2),
        "single_calls_gbs": round(total / single_us / 1e3, 2),
        "plain_copy_us": round(copy_us, 2), "plain_copy_gbs": round(total / copy_us / 1e3, 2),
        "host_us_per_set": {"warm": round(warm_host, 1), "cold": round(cold_host, 1),
                            "single_calls": round(single_host, 1)},
        "link_peak_gbs": peak, "frac_link_warm": round(total / warm_us / 1e3 / peak, 4),
        "frac_of_plain_copy_warm": round(copy_us / warm_us, 4),
        "evictions": sum(x["evictions"] for x in st),
    }
    log("adapter activation: " + json.dumps(res))
    return res


def cpu_baseline(w, pq, pv, target_s, y_gpu):
    """The fp64 oracle, as it is, on a bounded sample of the same rows; the
    first full pass also checks the last timed step's output (y_gpu, both
    projections, every row) at the layer's bf16 bound."""
    import oracle
    threads = oracle.default_threads()
    used = oracle.threads_used(threads)
    rng = np.random.default_rng(0)
    order = rng.permutation(w.M)
    check = {}

    def run(rows):
        t0 = time.perf_counter()
        outs = []
        for p in (pq, pv):
            outs.append(oracle.lora_linear(w.x[torch.from_numpy(rows)], p.W, p.A, p.B,
                                           w.scales.astype(np.float64), w.ids[rows],
                                           max_rank=w.max_rank, n_threads=threads))
        el = time.perf_counter() - t0
        if len(rows) == w.M and not check:
            for name, ref, lo, hi in (("q", outs[0], 0, pq.d), ("v", outs[1], pq.d, pq.d + pv.d)):
                got = y_gpu[np.asarray(rows)][:, lo:hi]
                check["normwise_" + name] = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
            check["tol"] = 2e-2
            check["rows"] = int(len(rows))
            check["ok"] = all(check["normwise_" + n] <= 2e-2 for n in ("q", "v"))
        return el

    probe = np.sort(order[:used])
    t_probe = run(probe)
    n = int(min(w.M, max(used, round(target_s / max(t_probe, 1e-9) * len(probe)))))
    rows = np.sort(order[:n])
    t = run(rows) if n != len(probe) else t_probe
    passes = 1
    # the whole batch is quicker than the target: repeat full passes
    while n == w.M and t * (passes + 1) / passes < target_s * 1.05 and t / passes < target_s:
        t += run(rows)
        passes += 1
    log("cpu oracle: %d rows x %d passes in %.1f s on %d threads" % (n, passes, t, used))
    if not check:  # the sample stopped short of every row: check those it covered
        check = {"rows": 0, "ok": None, "note": "the oracle sample did not cover a full pass"}
    log("output check: " + json.dumps(check))
    return ({"value": n * passes / t, "unit": "tokens/s", "cores": used, "kind": "oracle",
             "sample": "%d of the 512 rows (seeded) x %d passes, q and v projections, fp64, %.1f s"
                       % (n, passes, t)}, check)


def oracle_seconds(wl, w3):
    """One full oracle pass of every workload on all host threads, and of
    the two small ones on one thread (fp64, seconds per pass)."""
    import oracle
    threads = oracle.default_threads()
    out = {"threads": oracle.threads_used(threads)}
    for name, make in (("c0_tiny_fp32", wl.c0_tiny_fp32), ("c1_decode_bf16", wl.c1_decode_bf16),
                       ("c2_prefill_bf16", wl.c2_prefill_bf16), ("c3_proj70b_bf16", None),
                       ("c4_paged_bf16", wl.c4_paged_bf16)):
        w = w3 if make is None else make()
        entry = {}
        for nt in ((threads, 1) if name in ("c0_tiny_fp32", "c1_decode_bf16") else (threads,)):
            t0 = time.perf_counter()
            for p in w.projections:
                oracle.lora_linear(w.x, p.W, p.A, p.B, w.scales.astype(np.float64), w.ids,
                                   max_rank=w.max_rank, n_threads=nt)
            entry["s_%d_threads" % oracle.threads_used(nt)] = round(time.perf_counter() - t0, 4)
        entry["rows"] = w.M
        out[name] = entry
        del w
    log("oracle seconds: " + json.dumps(out))
    return out


def gather_path(lr, wl, w3, sets, ids, ws, stream, step_fn, steps=200):
    """The VALU gather kernels (LDS-staged A tiles, wavefront reduction
    over k) at the 70B q+v step and at the decode-4096 workload: step time
    and their event-timed shrink / expand launches."""
    out = {}
    for name in ("c3_proj70b_bf16", "c1_decode_bf16"):
        if name == "c3_proj70b_bf16":
            def go(i):
                s_ = sets[i % len(sets)]
                lr.lora_linear_sliced(s_["x"], s_["W"], s_["slices"], ids, y=s_["y"], workspace=ws,
                                      path=lr.PATH_GATHER, stream=stream)
            M = w3.M
            alg = [wl.algorithmic_bytes(w3, w3.proj("q")), wl.algorithmic_bytes(w3, w3.proj("v"))]
        else:
            w = wl.c1_decode_bf16()
            p = w.projections[0]
            dev = torch.device("cuda:0")
            A, B = wl.slots(w, p)
            ad = lr.Adapters.slots(A.to(dev), B.to(dev), torch.from_numpy(w.ranks).to(dev))
            x, W = w.x.to(dev), p.W.to(dev)
            y = torch.empty(w.M, p.d, dtype=w.dtype, device=dev)
            ids1, sc = torch.from_numpy(w.ids).to(dev), torch.from_numpy(w.scales).to(dev)
            ws1 = lr.new_workspace(w.M, p.d, w.k, w.dtype, ad, device=dev)

            def go(i):
                lr.lora_linear(x, W, ad, ids1, sc, y=y, workspace=ws1, path=lr.PATH_GATHER,
                               stream=stream)
            M = w.M
            alg = [wl.algorithmic_bytes(w, p)]
        for i in range(100):
            go(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            go(i)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        with lr.Profiler():
            for i in range(steps):
                go(i)
            prof = lr.Profiler.read(reset=True)
            torch.cuda.synchronize()
        per = {k: round(prof[k]["ms"] * 1e3 / prof[k]["launches"], 2) for k in lr.KERNEL_CLASSES
               if prof[k]["launches"]}
        shr_b = sum(a["shrink_bytes"] for a in alg) - (alg[0]["M_a"] * w3.k * 2 if len(alg) == 2 else 0)
        exp_b = sum(a["expand_bytes"] for a in alg)
        out[name] = {"tokens_per_s": round(M * steps / el, 1), "ms_per_step": round(el * 1e3 / steps, 4),
                     "per_launch_us": per,
                     "shrink_gbs": round(shr_b / per["shrink"] / 1e3, 1) if "shrink" in per else None,
                     "expand_gbs": round(exp_b / per["expand"] / 1e3, 1) if "expand" in per else None}
    log("gather path: " + json.dumps(out))
    return out


if __name__ == "__main__":
    main()
