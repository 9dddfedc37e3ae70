"""Benchmark: grouped routed-MoE prefill on one GPU.

One step = the whole path on one batch: route build (histogram, prefix,
scatter), grouped FFN (schedule, gate/up GEMM + SwiGLU, down GEMM) and the
route-weighted combine, with every input already resident in HBM.

With no --workload the headline record is the 401-token prefill (d=4096,
f=2048, 256 experts, top-6, bf16, 5% of routes masked) and the same JSON
line carries sub-records for the 2048-token bias-routed prefill, the
8192-token Zipf-routed chunk (bf16) and the 8192-token fp8 chunk, each with
its own step time, tokens/s and roofline of the dominant kernel.

Printed: one JSON line with whole-path tokens/s, the dominant kernel's
roofline fraction (gate/up stage, timed with HIP events on the launch stream
inside the timed region) and the CPU oracle's throughput on a bounded sample.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
METRIC = "routed-MoE prefill tokens/s + % of MFMA/HBM roofline at T=401/2048/8192"
# the token counts the metric names, after the headline 401-token workload
SUB_WORKLOADS = ["prefill_T2048_biased_bf16", "prefill_T8192_zipf_bf16",
                 "prefill_T8192_uniform_fp8"]
KERNEL_SOURCES = ["routed_expert_prefill_amd/csrc/ffn_grouped.hip",
                  "routed_expert_prefill_amd/csrc/ffn_fp8.hip",
                  "routed_expert_prefill_amd/csrc/ring.h",
                  "routed_expert_prefill_amd/csrc/common.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """Kernel source without comments, trailing blanks and empty lines, so that
    the hash changes with the code, not with its comments."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = []
    for line in text.splitlines():
        line = re.sub(r"//.*$", "", line).rstrip()
        if line:
            out.append(line)
    return "\n".join(out)


def source_hash(root: str = None) -> str:
    """Hash of the grouped-GEMM kernel code (comments excluded)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(root or ROOT, p), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def algorithmic_work(wl, counts, T):
    """Bytes and flops the method must move/compute, from the realized histogram.

    counts: active rows per expert.  Each stage's bytes are what it must read
    and write once (weights of the experts that received rows, activations,
    h, y, route metadata); the dense all-experts work the method avoids is not
    counted.  Returns per-stage and whole-path totals.
    """
    d, f, k = wl.d, wl.f, wl.k
    R = T * k
    R_act = int(sum(counts))
    used = sum(1 for c in counts if c > 0)
    fp8 = wl.dtype == "fp8"
    wb = 1 if fp8 else 2
    sc = 4 * (f // 128) * (d // 128) if fp8 else 0  # one scale grid (bytes)
    st = {}
    st["route"] = 30 * R  # ids, mask, gates read; permutations written and re-read
    if fp8:
        st["plan"] = T * d * 2 + T * d + 4 * T  # x read, codes and scales written
        st["gate_up"] = used * 2 * (f * d + sc) + T * d + 4 * T + 4 * R_act + R_act * f * 2
        st["down"] = (R_act * f * 2 + R_act * f + 4 * R_act  # h quantised per row
                      + used * (d * f + sc) + R_act * f + 4 * R_act + R_act * d * 4)
    else:
        st["plan"] = 0
        st["gate_up"] = used * 2 * f * d * wb + T * d * 2 + 4 * R_act + R_act * f * 2
        st["down"] = used * d * f * wb + R_act * f * 2 + R_act * d * 4
    st["combine"] = R_act * d * 4 + T * d * 4
    return {"R_act": R_act, "experts_used": used, "stage_bytes": st,
            "gate_up_bytes": st["gate_up"], "gate_up_flops": 4.0 * d * f * R_act,
            "path_bytes": sum(st.values()), "path_flops": 6.0 * d * f * R_act}


def traffic_from_profiles(workload: str):
    """HBM traffic of the gate/up stage from committed rocprofv3 counter runs, if
    they were taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"gate_up_traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        rec = json.load(fh)
    if rec.get("source_sha") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def device_facts():
    """The GPU the run used and the published peaks the roofline fractions use."""
    import torch

    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", None),
            "compute_units": pr.multi_processor_count,
            "memory_gib": round(pr.total_memory / 2**30, 1),
            "peaks": {"hbm_gbs": HBM_PEAK_GBS, "mfma_tflops": MFMA_PEAK_TFLOPS,
                      "at_clock_ghz": 2.4}}


def per_token_loop(wl, r, budget_s: float, max_tokens: int = 64):
    """The literal per-token oracle loop (moe_ref_per_token) timed token by
    token on the first tokens of the workload, until budget_s seconds of CPU
    work or max_tokens tokens.  Expert weights are generated outside the timed
    calls."""
    from oracle import moe as omoe
    from routed_expert_prefill_amd import synth

    from concurrent.futures import ThreadPoolExecutor

    fp8 = wl.dtype == "fp8"
    cache = {}
    spent, n = 0.0, 0
    pool = ThreadPoolExecutor(max(1, min(16, len(os.sched_getaffinity(0)))))
    for t in range(min(max_tokens, wl.T)):
        need = sorted({int(e) for e, m in zip(r.topk_ids[t], r.route_mask[t])
                       if m and 0 <= e < wl.E and int(e) not in cache})
        cache.update(zip(need, pool.map(lambda e: synth.expert_weights(wl, e, 0), need)))
        t0 = time.perf_counter()
        omoe.moe_ref_per_token(r.x, r.topk_ids, r.topk_w, r.route_mask, cache.__getitem__, wl.E,
                               fp8=fp8, tokens=[t])
        spent += time.perf_counter() - t0
        n += 1
        if spent >= budget_s:
            break
    pool.shutdown()
    return {"value": round(n / spent, 4), "unit": "tokens/s", "tokens": n,
            "seconds": round(spent, 2), "kind": "oracle",
            "sample": f"moe_ref_per_token (fp64 numpy, one token at a time) on tokens 0..{n - 1}"}


def cpu_baseline(wl, r, budget_s: float):
    """The fp64 oracle (expert-major, BLAS) on a bounded sample of the workload.

    The fixed part (route table, combine over all routes) is timed once; then
    experts' FFNs are evaluated in chunks, in expert order, until about
    budget_s seconds of CPU work or every active expert is done.  The time for
    all active experts is extrapolated from the per-expert average.  The
    literal per-token loop is timed beside it on the first tokens.
    """
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import moe as omoe
    from oracle.route import route_table
    from routed_expert_prefill_amd import synth

    cores = len(os.sched_getaffinity(0))
    fp8 = wl.dtype == "fp8"
    rt = route_table(r.topk_ids, r.route_mask, wl.E)
    active = [e for e in range(wl.E) if rt.counts[e] > 0]
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        omoe.moe_ref_blocked(r.x, r.topk_ids, r.topk_w, r.route_mask, lambda e: None, wl.E,
                             fp8=fp8, expert_subset=[])
        t_fixed = time.perf_counter() - t0
        done, t_ffn = [], 0.0
        while len(done) < len(active) and t_fixed + t_ffn < budget_s:
            chunk = active[len(done):len(done) + 8]
            cache = {e: synth.expert_weights(wl, e, 0) for e in chunk}  # generation not timed
            t0 = time.perf_counter()
            omoe.moe_ref_blocked(r.x, r.topk_ids, r.topk_w, r.route_mask, cache.__getitem__, wl.E,
                                 fp8=fp8, expert_subset=chunk)
            t_ffn += max(time.perf_counter() - t0 - t_fixed, 0.0)
            done += chunk
        loop = per_token_loop(wl, r, max(2.0, budget_s / 4))
    t_total = t_fixed + t_ffn / len(done) * len(active)
    blas = ",".join(sorted({str(i.get("internal_api")) for i in threadpool_info()}))
    cpu_model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(wl.T / t_total, 3),
        "unit": "tokens/s",
        "cores": cores,
        "cpu": cpu_model,
        "kind": "oracle",
        "sample": (f"moe_ref_blocked (fp64 numpy, BLAS {blas}): route table and combine over all "
                   f"{wl.T} tokens plus the FFNs of {len(done)} of {len(active)} active experts "
                   f"({t_fixed + t_ffn:.1f} s measured), extrapolated to all active experts"),
        "seconds_extrapolated": round(t_total, 2),
        "per_token_loop": loop,
    }


def tree_identity():
    """Which sources produced the numbers: the git commit when a checkout is
    present, and always a hash of the library, header and benchmark sources
    (comments included), which identifies the tree where no .git travels."""
    import subprocess

    git = None
    try:
        head = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                              text=True, timeout=10)
        if head.returncode == 0:
            dirty = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"],
                                   capture_output=True, text=True, timeout=10).stdout.strip()
            git = head.stdout.strip() + ("-dirty" if dirty else "")
    except (OSError, subprocess.SubprocessError):
        git = None
    h = hashlib.sha256()
    files = []
    for sub in ("routed_expert_prefill_amd/csrc", "routed_expert_prefill_amd", "include"):
        d = os.path.join(ROOT, sub)
        files += [os.path.join(sub, n) for n in sorted(os.listdir(d))
                  if n.endswith((".hip", ".h", ".cpp", ".py"))]
    files.append("bench.py")
    for rel in files:
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return {"git_commit": git, "tree_sha256": h.hexdigest()[:16]}


def route_table_sha(rt):
    """SHA-256 of the route table the GPU built (counts, offsets, sorted_routes,
    route_rows as little-endian int32, in that order)."""
    h = hashlib.sha256()
    for t in rt:
        h.update(t.cpu().numpy().astype("<i4").tobytes())
    return h.hexdigest()


def med(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def device_bytes_needed(wl):
    """Device memory a measurement holds: weights, activations, route table,
    y, out and the workspaces, with 10% slack."""
    from routed_expert_prefill_amd import synth

    R = wl.T * wl.k
    b = wl.E * synth.weight_bytes_per_expert(wl) + wl.T * wl.d * 2 + R * 13
    b += R * wl.d * 4 + wl.T * wl.d * 4  # y, out
    b += R * wl.f * 2 + (wl.T * wl.d + R * wl.f + 8 * R if wl.dtype == "fp8" else 0)  # workspace
    return int(b * 1.1)


def chunk_workload(name, tokens):
    """The named workload's shapes and input recipe with only `tokens` tokens
    (a decode-sized chunk), under a name of its own."""
    from routed_expert_prefill_amd import synth

    base = synth.WORKLOADS[name]
    return base.replace(T=tokens, name=f"chunk_T{tokens}_d{base.d}_f{base.f}_E{base.E}_"
                                       f"{base.routing}_{base.dtype}")


def measure(name, args, dev, owner_arg=None, cpu_seconds=None, tokens=None):
    """One workload: warm-up, K timed steps, a second per-call pass, the
    dominant kernel's roofline, and (optionally) the CPU oracle's sample.
    With tokens, the workload's first-`tokens` chunk (chunk_workload)."""
    import torch

    import routed_expert_prefill_amd as rep
    from routed_expert_prefill_amd import synth

    wl = synth.WORKLOADS[name] if tokens is None else chunk_workload(name, tokens)
    name = wl.name
    fp8 = wl.dtype == "fp8"
    free, total = torch.cuda.mem_get_info(dev)
    need = device_bytes_needed(wl)
    if need > free:
        print(f"bench.py: {name} needs about {need / 2**30:.1f} GiB of device memory and "
              f"{free / 2**30:.1f} GiB of {total / 2**30:.1f} GiB are free; not running it",
              file=sys.stderr)
        sys.exit(3)
    t0 = time.perf_counter()
    r, ten = synth.device_inputs(wl, seed=0, device=dev)
    log(f"inputs for {name} generated and resident in HBM in {time.perf_counter() - t0:.1f} s")

    owner = None
    if owner_arg:
        G, g = (int(v) for v in owner_arg.split(":"))
        r = dataclasses.replace(r, route_mask=synth.owner_mask(r.topk_ids, r.route_mask, wl.E, G, g))
        ten["route_mask"] = torch.from_numpy(r.route_mask).to(dev)
        owner = f"{g} of {G}"
        log(f"owner {owner}: {int(r.route_mask.sum())} of {r.route_mask.size} routes active")

    run = rep.MoEPrefill(wl.T, wl.k, wl.E, wl.d, wl.f, fp8=fp8, device=dev)
    stream = torch.cuda.current_stream(dev)
    wargs = (ten["x"], ten["topk_ids"], ten["topk_w"], ten["route_mask"], ten["w_gate"],
             ten["w_up"], ten["w_down"], ten.get("s_gate"), ten.get("s_up"), ten.get("s_down"))

    def step(ev=None):
        return run(*wargs, stage_events=ev)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    graph = None
    if args.graph:
        # one step captured in a HIP graph (after a pass on the capture
        # stream) and replayed in the timed region: no host launch cost
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize(dev)
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize(dev)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step(evs[i])
    end.record(stream)
    torch.cuda.synchronize(dev)
    t_wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(end) / args.steps
    if graph is None:
        gu_ms = [a.elapsed_time(b) for a, b in evs]
        gu_avg = sum(gu_ms) / len(gu_ms)

    # each call timed alone: a second pass of K steps (after the timed
    # region) with events between the calls; per-step median/MAD/min from it
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(bev[i])
    torch.cuda.synchronize(dev)
    stage_names = ["route_build", "ffn_plan", "gate_up", "down", "combine"]
    per_stage = {n: [e[i].elapsed_time(e[i + 1]) for e in bev] for i, n in enumerate(stage_names)}
    per_step = [e[0].elapsed_time(e[5]) for e in bev]
    step_med = med(per_step)
    step_stats = {"median": round(step_med, 5),
                  "mad": round(med([abs(v - step_med) for v in per_step]), 5),
                  "min": round(min(per_step), 5)}
    stages_ms = {n: round(med(v), 5) for n, v in per_stage.items()}
    if graph is not None:  # gate/up timed in the per-call pass (events cannot sit in the replays)
        gu_avg = sum(per_stage["gate_up"]) / len(per_stage["gate_up"])
        del graph
    log(f"{name}: {ms_step:.4f} ms/step (wall {1e3 * t_wall / args.steps:.4f}); "
        f"per step median {step_stats['median']:.4f} ms; stages {stages_ms}")

    counts = run.rt.counts.cpu().numpy()[: wl.E].tolist()
    rt_sha = route_table_sha(run.rt)
    work = algorithmic_work(wl, counts, wl.T)
    tok_s = wl.T / (ms_step / 1e3)
    # bound of the dominant stage: HBM time vs MFMA time at the published peaks
    t_h = work["gate_up_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_m = work["gate_up_flops"] / (MFMA_PEAK_TFLOPS[wl.dtype] * 1e12)
    if t_h >= t_m:
        ach = work["gate_up_bytes"] / (gu_avg / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    else:
        ach = work["gate_up_flops"] / (gu_avg / 1e3) / 1e12
        pk = MFMA_PEAK_TFLOPS[wl.dtype]
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": pk, "unit": "TFLOP/s",
                "frac": round(ach / pk, 4)}
    roof["traffic"] = (traffic_from_profiles(name) if owner is None and tokens is None
                       else None)
    roof["kernel"] = ("grouped_gemm8_kernel<true>" if fp8 else "grouped_gemm_kernel<true>") + \
        " (gate/up GEMM, SwiGLU epilogue)"
    roof["avg_ms"] = round(gu_avg, 5)
    roof["algorithmic_bytes"] = int(work["gate_up_bytes"])
    roof["algorithmic_flops"] = work["gate_up_flops"]
    t_path_roof = max(work["path_bytes"] / (HBM_PEAK_GBS * 1e9),
                      work["path_flops"] / (MFMA_PEAK_TFLOPS[wl.dtype] * 1e12))
    del run, wargs, ten
    torch.cuda.empty_cache()

    cpu = None
    if cpu_seconds:
        log(f"timing the CPU oracle on a bounded sample of {name} ...")
        cpu = cpu_baseline(wl, r, cpu_seconds)
        log(f"cpu baseline: {cpu['value']} tokens/s ({cpu['sample']})")

    return {
        "workload": name,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "ms_per_step": round(ms_step, 5),
        "dtype": wl.dtype,
        "config": {"workload": name, "T": wl.T, "d": wl.d, "f": wl.f, "E": wl.E, "k": wl.k,
                   "routing": wl.routing, "mask_p": wl.mask_p, "weights": wl.dtype,
                   "parallelism": "single-gpu" if owner is None else f"expert owner {owner}",
                   "launch": "hip graph replay" if args.graph else "eager"},
        "path": {"tflops": round(work["path_flops"] / (ms_step / 1e3) / 1e12, 2),
                 "algorithmic_gb": round(work["path_bytes"] / 1e9, 3),
                 "hbm_gbs": round(work["path_bytes"] / (ms_step / 1e3) / 1e9, 1),
                 "roofline_frac": round(t_path_roof / (ms_step / 1e3), 4),
                 "mfma_frac": round(work["path_flops"] / (ms_step / 1e3) / 1e12
                                    / MFMA_PEAK_TFLOPS[wl.dtype], 4),
                 "active_rows": work["R_act"], "experts_used": work["experts_used"],
                 "stage_bytes": work["stage_bytes"]},
        "step_ms": step_stats,  # from the per-call pass, not the timed region
        "stages_ms": stages_ms,
        "roofline": roof,
        "route_table_sha256": rt_sha,
        "cpu_baseline": cpu,
    }


def router_timing(name, dev):
    """moe_route_topk on the workload's logits, timed on its own: the router is
    ahead of the path, whose routing is an input."""
    import torch

    import routed_expert_prefill_amd as rep
    from routed_expert_prefill_amd import synth

    wl = synth.WORKLOADS[name]
    stream = torch.cuda.current_stream(dev)
    logits = torch.from_numpy(synth.make_logits(wl, seed=0)).to(dev)
    for _ in range(3):
        rep.route_topk(logits, wl.k)
    rev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    n_router = 20
    rev[0].record(stream)
    for _ in range(n_router):
        rep.route_topk(logits, wl.k)
    rev[1].record(stream)
    torch.cuda.synchronize(dev)
    router_ms = rev[0].elapsed_time(rev[1]) / n_router
    router_bytes = wl.T * wl.E * 4 + wl.T * wl.k * 8
    return {"call": "moe_route_topk", "workload": name, "ms": round(router_ms, 5),
            "gb_s": round(router_bytes / (router_ms / 1e3) / 1e9, 1),
            "algorithmic_bytes": router_bytes}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="measure this workload alone (default: the 401-token headline plus "
                         "the 2048- and 8192-token sub-records)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="approximate CPU time spent on the oracle sample of the headline workload")
    ap.add_argument("--sub-cpu-seconds", type=float, default=6.0,
                    help="the same for each sub-record workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub-records", action="store_true")
    ap.add_argument("--owner", default=None, metavar="G:g",
                    help="measure one owner's share: experts split into G contiguous ranges, "
                         "only routes to range g stay active (the sharded layout on one GPU)")
    ap.add_argument("--tokens", type=int, default=None, metavar="N",
                    help="measure a chunk of N tokens with the workload's shapes and input "
                         "recipe (decode-sized chunks); no sub-records")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays (no host launch "
                         "cost: for decode-sized chunks); gate/up is then timed in the per-call pass")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one device-to-device copy of 1 GiB (a known-size kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library runs on a single GPU and has no "
              "multi-GPU path (sharding across GPUs is a design note, not built). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import routed_expert_prefill_amd as rep
    from routed_expert_prefill_amd import synth

    name = args.workload or synth.DEFAULT_BENCH_WORKLOAD
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} CUs={props.multi_processor_count} "
        f"arch={getattr(props, 'gcnArchName', '?')} mem={props.total_memory / 2**30:.0f} GiB")
    rep.load_library()

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        del src, dst

    head = measure(name, args, dev, owner_arg=args.owner,
                   cpu_seconds=None if args.no_cpu_baseline else args.cpu_seconds,
                   tokens=args.tokens)
    router = router_timing(name, dev) if args.tokens is None else None
    subs = []
    if (args.workload is None and args.owner is None and args.tokens is None
            and not args.no_sub_records):
        for sub in SUB_WORKLOADS:
            rec = measure(sub, args, dev,
                          cpu_seconds=None if args.no_cpu_baseline else args.sub_cpu_seconds)
            rec.pop("config", None)
            subs.append(rec)

    rec = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "path": head["path"],
        "step_ms": head["step_ms"],
        "stages_ms": head["stages_ms"],
        "roofline": head["roofline"],
        "route_table_sha256": head["route_table_sha256"],
        "router": router,
        "cpu_baseline": head["cpu_baseline"],
        "sub_records": subs,
        "device": device_facts(),
        "kernel_source_sha": source_hash(),
        "source": tree_identity(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
