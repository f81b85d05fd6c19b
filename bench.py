"""Benchmark of the bf16 routed MoE-LoRA layer on one MI355X.

One step = one full layer forward from router logits (routing, permutation,
both LoRA shrinks, gate_up GEMM with LoRA expand and SwiGLU, down GEMM with
LoRA expand, finalize) over one batch of seeded synthetic inputs already
resident in HBM.  Prints ONE JSON line on stdout; diagnostics go to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode64]

The dominant kernel's duration comes from two HIP events the library records
around it on the launch stream in every timed step; a separate pass with all
stage events gives the per-stage breakdown.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-LoRA layer tokens/s + achieved HBM GB/s (T=64 decode) and MFMA % (prefill)"
HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16

WORKLOAD_TEXT = {
    "decode64": "multi-adapter decode: T=64 tokens, hidden 2048, 128 experts top-8, inter 768 "
                "SwiGLU, 4 LoRA adapters rank 16 on gate_up and down, mapping uniform over "
                "{-1,0,1,2,3}, 4 hot experts",
    "decode16": "T=16, hidden 2048, 128 experts top-8, inter 768, 1 adapter rank 16",
    "ep_shard": "expert-parallel shard: T=64, hidden 2048, 32 of 128 experts local (offset 32), "
                "top-8, inter 768, 4 adapters rank 16",
    "prefill": "T=2048, hidden 2048, 128 experts top-8, inter 768, 4 adapters rank 64 "
               "in runs of 512 tokens",
    "tiny": "tiny: T=8, hidden 128, 8 experts top-2, inter 64, 2 adapters rank 4",
}


def log(msg: str):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


class HipEvents:
    """Minimal HIP event API through ctypes (timing on the library's stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n: int, disable_timing: bool = False):
        out = []
        for _ in range(n):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), 2 if disable_timing else 0)
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            out.append(ev.value)
        return out

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def sync(self, ev):
        self.hip.hipEventSynchronize(ctypes.c_void_p(ev))

    def destroy(self, evs):
        for ev in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(ev))


def algorithmic_cost(cfg, ids, mapping):
    """Bytes the layer must move and flops it must do, from the actual routing.

    Expert weights of every touched local expert, LoRA stacks of every touched
    (adapter, local expert) pair, plus hidden in, out, logits and mapping.
    Also the bytes of the gate_up GEMM launch alone.
    """
    import numpy as np
    T, H, I, E, k = cfg.num_tokens, cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k
    off, E_l, L = cfg.local_expert_offset, cfg.local_num_experts, cfg.num_loras
    rg, rd = cfg.rank_gate_up, cfg.rank_down
    ids = np.asarray(ids)
    local = (ids >= off) & (ids < off + E_l)
    le = np.where(local, ids - off, -1)
    touched = np.unique(le[local])
    lmap = np.repeat(np.asarray(mapping), k).reshape(ids.shape)
    lvalid = local & (lmap >= 0) & (lmap < L)
    pairs = np.unique((lmap * E_l + le)[lvalid]) if L > 0 else np.zeros(0)
    adapters = np.unique(lmap[lvalid]) if L > 0 else np.zeros(0)
    P = int(local.sum())
    P_lora = int(lvalid.sum())
    n_e, n_pairs = len(touched), len(pairs)
    # shared-outer layout: A_gu and B_dn once per touched adapter, not per pair
    n_outer = len(adapters) if getattr(cfg, "lora_shared_outer", False) else n_pairs
    w13_bytes = 2 * n_e * H * 2 * I
    w2_bytes = 2 * n_e * I * H
    lora_gu = 2 * (n_outer * rg * H + n_pairs * 2 * I * rg) if rg else 0
    lora_dn = 2 * (n_pairs * rd * I + n_outer * H * rd) if rd else 0
    io = 2 * T * H * 2 + 4 * T * E + 4 * T
    total_bytes = w13_bytes + w2_bytes + lora_gu + lora_dn + io
    flops = 2 * P * (H * 2 * I + I * H) + 2 * P_lora * (rg * (H + 2 * I) + rd * (I + H))
    # gate_up GEMM launch: W13 of touched experts, B_gu of touched pairs, the routed
    # tokens' hidden rows, the bf16 shrink rows it reads, the activation it writes
    tok_touched = int(local.any(axis=1).sum())
    gate_up_bytes = (w13_bytes + (2 * n_pairs * 2 * I * rg if rg else 0) + 2 * tok_touched * H +
                     2 * P_lora * ((rg + 7) // 8 * 8) + 2 * P * I)
    gate_up_flops = 2 * P * H * 2 * I + 2 * P_lora * rg * 2 * I
    return {
        "bytes": int(total_bytes), "flops": int(flops), "local_slots": P,
        "touched_experts": n_e, "touched_lora_pairs": n_pairs,
        "gate_up_bytes": int(gate_up_bytes), "gate_up_flops": int(gate_up_flops),
    }


# --------------------------------------------------------------------------
# rocprofv3 summaries (written under profiles/, read back for `traffic`)
# --------------------------------------------------------------------------

PROFILES = os.path.join(ROOT, "profiles")
GEMM_SOURCES = ["mixture_experts_layer_up_amd/csrc/expert_gemm.hip",
                "mixture_experts_layer_up_amd/csrc/expert_gemm_wide.hip",
                "mixture_experts_layer_up_amd/csrc/gemm_index.h",
                "mixture_experts_layer_up_amd/csrc/mfma_pipeline.h",
                "mixture_experts_layer_up_amd/csrc/lora_shrink_rows.h",
                "mixture_experts_layer_up_amd/csrc/device_common.h",
                "mixture_experts_layer_up_amd/csrc/lds_dma.h",
                "mixture_experts_layer_up_amd/csrc/kernels.h"]
# the timed region records the dominant kernel's event pair on every
# EVENT_EVERY-th step
EVENT_EVERY = 4
DOMINANT = {"decode": "expert_gemm_kernel<1, 1, true, true>", "prefill": "expert_gemm_wide_kernel<true>"}


def gemm_source_hash() -> str:
    """Hash of the GEMM kernels' code: their sources with comments and blank
    lines removed, so that a comment edit keeps the committed counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


def _kernel_short(name: str) -> str:
    name = name.replace("moe_lora::(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0]


def summarize_trace(stats_csv: str, out_md: str, command: str):
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel trace: {os.path.basename(out_md)[:-3]}", "",
             f"command: `{command}`", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{_kernel_short(r['Name'])}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_counters(fetch_csv: str, write_csv: str, out_md: str, command: str,
                       copy_mib: int, dominant: str):
    """FETCH_SIZE / WRITE_SIZE per dispatch (median), scaled by what the same
    counters read for a plain copy kernel (torch.neg) of known size."""
    import csv
    import statistics

    def per_kernel(path):
        agg = {}
        for r in csv.DictReader(open(path)):
            agg.setdefault(_kernel_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return agg

    fetch, write = per_kernel(fetch_csv), per_kernel(write_csv)
    copy = [k for k in fetch if "neg_kernel" in k]
    kib = copy_mib * 1024.0
    f_scale = kib / max(fetch[copy[0]]) if copy else None
    w_scale = kib / max(write[copy[0]]) if copy else None
    lines = [f"# HBM traffic counters: {os.path.basename(out_md)[:-3]}", "",
             f"command: `{command}` (one rocprofv3 run per counter)", "",
             f"kernel_source_sha256: {gemm_source_hash()}", "",
             f"copy calibration (torch.neg over {copy_mib} MiB, reads and writes {kib:.0f} KiB): "
             f"FETCH_SIZE factor {f_scale:.4f}, WRITE_SIZE factor {w_scale:.4f}", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |",
             "|---|---|---|---|---|"]
    dom_bytes = None
    for k in fetch:
        fk = statistics.median(fetch[k])
        wk = statistics.median(write.get(k, [0.0]))
        rb, wb = fk * f_scale * 1024, wk * w_scale * 1024
        lines.append(f"| `{k}` | {fk:.1f} | {wk:.1f} | {rb / 1e6:.2f} | {wb / 1e6:.2f} |")
        if dominant in k:
            dom_bytes = rb + wb
    lines += ["", f"dominant_kernel: `{dominant}`",
              f"traffic_bytes_per_launch: {dom_bytes:.0f}" if dom_bytes else "traffic_bytes_per_launch: none"]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_mfma(csv_path: str, out_md: str, command: str):
    """MfmaUtil (MFMA busy cycles over GRBM_GUI_ACTIVE x SIMDs, percent) and
    MfmaFlopsBF16 (bf16 MFMA operations x 512) per dispatch, median per
    kernel; TFLOP/s over the same dispatches' durations."""
    import csv
    import statistics
    util, flops, dur = {}, {}, {}
    for r in csv.DictReader(open(csv_path)):
        k = _kernel_short(r["Kernel_Name"])
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if r["Counter_Name"] == "MfmaUtil":
            util.setdefault(k, []).append(float(r["Counter_Value"]))
            dur.setdefault(k, []).append(d)
        elif r["Counter_Name"] == "MfmaFlopsBF16":
            flops.setdefault(k, []).append(float(r["Counter_Value"]))
    lines = [f"# MFMA counters: {os.path.basename(out_md)[:-3]}", "",
             f"command: `{command}`", "",
             f"kernel_source_sha256: {gemm_source_hash()}", "",
             f"peak: {MFMA_BF16_PEAK_TFLOPS:.0f} TFLOP/s dense bf16", "",
             "| kernel | dispatches | MfmaUtil % | bf16 MFMA GFLOP per dispatch | us (counter run) | TFLOP/s | of peak |",
             "|---|---|---|---|---|---|---|"]
    for k in util:
        u = statistics.median(util[k])
        f = statistics.median(flops.get(k, [0.0]))
        d = statistics.median(dur[k])
        if f <= 0:
            continue
        tf = f / d / 1e6
        lines.append(f"| `{k}` | {len(util[k])} | {u:.2f} | {f / 1e9:.3f} | {d:.1f} | {tf:.1f} | "
                     f"{tf / MFMA_BF16_PEAK_TFLOPS:.3f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def traffic_from_profile(workload: str):
    """Counter-measured HBM bytes per launch of the dominant kernel, if the
    committed profile was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"gemm_gate_up_swiglu_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    import re
    h = re.search(r"kernel_source_sha256: (\w+)", text)
    b = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    if not h or not b or h.group(1) != gemm_source_hash():
        return None
    return int(b.group(1))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, min_seconds: float):
    """Time the CPU oracle (as is) on a bounded sample of the same workload,
    on all of the host's threads and on one."""
    import numpy as np
    from oracle import oracle
    T = cfg.num_tokens
    n_tok = min(T, 64)
    toks = np.linspace(0, T - 1, n_tok).astype(np.int32) if n_tok < T else None
    ids, w = oracle.route(inp["logits"], cfg.top_k, bias=inp.get("routing_bias"),
                          method=getattr(cfg, "routing_method", 0))

    def timed(seconds, tokens):
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.forward(cfg, inp, topk_ids=ids, topk_weights=w, tokens=tokens)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return reps, el

    threads = oracle.num_threads()
    reps, el = timed(min_seconds, toks)
    sample = (f"{n_tok} of {T} tokens" + ("" if toks is None else " (evenly spaced)") +
              f" of the same seeded batch, routing precomputed, {reps} repetitions, {el:.1f} s")
    # one thread, on a quarter of the sample (the per-token work is the same)
    n1 = max(1, n_tok // 4)
    toks1 = np.linspace(0, T - 1, n1).astype(np.int32)
    oracle.set_num_threads(1)
    try:
        reps1, el1 = timed(min_seconds / 2, toks1)
    finally:
        oracle.set_num_threads(threads)
    return {"value": reps * n_tok / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": sample, "cpu_model": _cpu_model(),
            "single_core": {"value": reps1 * n1 / el1, "unit": "tokens/s",
                            "sample": f"{n1} evenly spaced tokens, {reps1} repetitions, "
                                      f"{el1:.1f} s, 1 thread"}}


def measure(args, workload: str, steps: int, warmup: int, cold_steps: int, graph: bool,
            two_stream: bool, finalize: str = "fused", lora_layout: str = "per_expert",
            routing_method: int = 0, routing_bias_sigma: float = 0.0, cpu_seconds: float = 0.0,
            copy_probe_mib: int = 0):
    """Time one workload; returns its result fields (value, roofline, layer, ...)."""
    import numpy as np
    import torch

    from mixture_experts_layer_up_amd import binding
    from mixture_experts_layer_up_amd.synth import CONFIGS, make_inputs

    cfg = CONFIGS[workload]
    if lora_layout == "shared_outer":
        cfg = cfg.replace(lora_shared_outer=True)
    if routing_method or routing_bias_sigma > 0:
        cfg = cfg.replace(routing_method=routing_method, routing_bias_sigma=routing_bias_sigma)
    log(f"[bench] generating {workload} inputs")
    inp = make_inputs(cfg)
    torch.cuda.set_device(0)
    shape, lay = binding.layer_from_host(cfg, inp)
    ws = torch.empty(binding.workspace_size(shape), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    kw = {k: v for k, v in lay.items() if k not in ("hidden", "w13_packed", "w2_packed")}

    hip = HipEvents()
    side_events = []
    if two_stream:
        side_stream = torch.cuda.Stream()   # default priority
        side_events = hip.create(2, disable_timing=True)
        kw.update(side_stream=side_stream.cuda_stream, fork_event=side_events[0],
                  join_event=side_events[1])
    ext_routing = binding.alloc_routing(shape, "cuda") if finalize == "external" else None
    expert_out = (torch.empty((cfg.num_tokens * cfg.top_k, cfg.hidden), dtype=torch.bfloat16,
                              device="cuda") if ext_routing is not None else None)

    def step(events=None):
        if ext_routing is None:
            binding.forward(shape, lay["hidden"], lay["w13_packed"], lay["w2_packed"], out=out,
                            workspace=ws, stage_events=events, **kw)
        else:
            binding.forward(shape, lay["hidden"], lay["w13_packed"], lay["w2_packed"],
                            workspace=ws, stage_events=events, routing=ext_routing,
                            expert_out=expert_out, **kw)
            binding.finalize(shape, expert_out, ext_routing, out=out)

    if copy_probe_mib > 0:
        n = copy_probe_mib * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: read {copy_probe_mib} MiB, wrote {copy_probe_mib} MiB")
        del src, dst

    log(f"[bench] {workload}: warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    K = steps
    nstage = len(binding.STAGE_NAMES)
    stream = torch.cuda.current_stream().cuda_stream

    # The timed region: K steps launched from the host.  Every EVENT_EVERY-th
    # step records the two stage events around the dominant kernel (the
    # gate_up GEMM), whose elapsed time is that kernel's live duration; every
    # recorded event costs stream time (two cost ~5 us), so the other
    # boundaries are left out and the sampled steps are spread evenly.
    gi = binding.STAGE_NAMES.index("gemm_gate_up_swiglu")  # between events gi, gi + 1
    kev = [hip.create(2) for _ in range((K + EVENT_EVERY - 1) // EVENT_EVERY)]

    def dominant_events(pair):
        ev = [None] * binding.NUM_STAGE_EVENTS
        ev[gi], ev[gi + 1] = pair
        return ev

    plan = [dominant_events(kev[s_ // EVENT_EVERY]) if s_ % EVENT_EVERY == 0 else None
            for s_ in range(K)]
    start, end = hip.create(2)
    log(f"[bench] {workload}: timing {K} steps")
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    hip.record(start, stream)
    for s_ in range(K):
        step(plan[s_])
    hip.record(end, stream)
    hip.sync(end)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    ms_per_step = hip.elapsed_ms(start, end) / K
    gate_up_ms = sum(hip.elapsed_ms(a, b) for a, b in kev) / len(kev)
    for p in kev:
        hip.destroy(p)
    hip.destroy([start, end])

    # Stage breakdown (diagnostic, outside the timed region): steps with all
    # seven stage events recorded.
    KB = min(K, 50)
    evs = [hip.create(binding.NUM_STAGE_EVENTS) for _ in range(KB)]
    for s_ in range(KB):
        step(evs[s_])
    torch.cuda.synchronize()
    stage_ms = np.zeros(nstage)
    for s_ in range(KB):
        for i in range(nstage):
            stage_ms[i] += hip.elapsed_ms(evs[s_][i], evs[s_][i + 1])
    stage_ms /= KB
    for e in evs:
        hip.destroy(e)

    # the same K steps captured into one HIP graph and replayed (the forward
    # allocates nothing and never waits on the host); reported beside `value`
    graph_ms = None
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(K):
                step()
        g.replay()
        torch.cuda.synchronize()
        gs, ge = hip.create(2)
        hip.record(gs, stream)
        g.replay()
        hip.record(ge, stream)
        hip.sync(ge)
        graph_ms = hip.elapsed_ms(gs, ge) / K
        hip.destroy([gs, ge])
        del g
        log(f"[bench] {workload}: graph replay {graph_ms * 1e3:.1f} us/step")

    # Cold cache (diagnostic, outside the timed region): before each of KC
    # steps a 512 MiB buffer is rewritten, so the 256 MiB Infinity Cache
    # holds none of the layer's data; each step is timed alone between two
    # events.  Back-to-back steps (the timed region) keep only what the
    # previous step left in that cache.
    cold = None
    if cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cev = [hip.create(2) for _ in range(cold_steps)]
        for s_, (a_, b_) in enumerate(cev):
            flush.fill_(s_ & 0xff)
            hip.record(a_, stream)
            step()
            hip.record(b_, stream)
        torch.cuda.synchronize()
        cms = np.array([hip.elapsed_ms(a_, b_) for a_, b_ in cev])
        for e in cev:
            hip.destroy(e)
        del flush
        cold = {"steps": cold_steps, "ms_median": float(np.median(cms)),
                "ms_p90": float(np.percentile(cms, 90)), "ms_min": float(cms.min()),
                "tokens_per_s_median": cfg.num_tokens / (float(np.median(cms)) / 1e3)}
        log(f"[bench] {workload}: cold cache median {cold['ms_median'] * 1e3:.1f} us/step")

    # the cost model counts what this batch's routing touches (the library's own routing)
    routing = binding.alloc_routing(shape, "cuda")
    binding.forward(shape, lay["hidden"], lay["w13_packed"], lay["w2_packed"], out=out,
                    workspace=ws, routing=routing, **kw)
    torch.cuda.synchronize()
    cost = algorithmic_cost(cfg, routing["topk_ids"].cpu().numpy(), inp["mapping"])
    hip.destroy(side_events)
    t_s = ms_per_step / 1e3
    achieved = cost["gate_up_bytes"] / (gate_up_ms / 1e3) / 1e9
    gate_up_tflops = cost["gate_up_flops"] / (gate_up_ms / 1e3) / 1e12
    layer_gbps = cost["bytes"] / t_s / 1e9
    layer_tflops = cost["flops"] / t_s / 1e12
    # the layer's roofline time: the larger of its HBM and MFMA floors
    floor_s = max(cost["bytes"] / (HBM_PEAK_GBPS * 1e9), cost["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12))

    cpu = None
    if cpu_seconds > 0:
        log("[bench] CPU oracle baseline")
        cpu = cpu_baseline(cfg, inp, cpu_seconds)

    return {
        "cfg": cfg,
        "value": cfg.num_tokens / t_s,
        "ms_per_step": ms_per_step,
        "config": {"workload": f"{workload}: {WORKLOAD_TEXT[workload]}",
                   "num_tokens": cfg.num_tokens, "hidden": cfg.hidden, "inter": cfg.inter,
                   "num_experts": cfg.num_experts, "top_k": cfg.top_k,
                   "local_expert_offset": cfg.local_expert_offset,
                   "local_num_experts": cfg.local_num_experts, "num_loras": cfg.num_loras,
                   "rank": cfg.rank_gate_up, "lora_layout": lora_layout,
                   "finalize": finalize, "two_stream": bool(two_stream),
                   "routing_method": routing_method,
                   "routing_bias_sigma": routing_bias_sigma,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "gemm_gate_up_swiglu",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic_from_profile(workload),
                     "algorithmic_bytes_per_launch": cost["gate_up_bytes"],
                     "algorithmic_flops_per_launch": cost["gate_up_flops"],
                     "mfma_tflops": gate_up_tflops,
                     "mfma_frac": gate_up_tflops / MFMA_BF16_PEAK_TFLOPS,
                     "kernel_us": gate_up_ms * 1e3},
        "layer": {"algorithmic_bytes": cost["bytes"], "flops": cost["flops"],
                  "hbm_gbps": layer_gbps, "hbm_frac": layer_gbps / HBM_PEAK_GBPS,
                  "mfma_tflops": layer_tflops, "mfma_frac": layer_tflops / MFMA_BF16_PEAK_TFLOPS,
                  "roofline_us": floor_s * 1e6, "roofline_frac": floor_s / t_s,
                  "mfma_frac_at_hbm_peak": cost["flops"] / floor_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                  "touched_experts": cost["touched_experts"],
                  "touched_lora_pairs": cost["touched_lora_pairs"],
                  "local_slots": cost["local_slots"]},
        "stages_us": {n: float(v * 1e3) for n, v in zip(binding.STAGE_NAMES, stage_ms)},
        "wall_ms_per_step": wall_s * 1e3 / K,
        "graph_replay": None if graph_ms is None else {
            "ms_per_step": graph_ms, "tokens_per_s": cfg.num_tokens / (graph_ms / 1e3),
            "layer_hbm_frac": cost["bytes"] / (graph_ms / 1e3) / 1e9 / HBM_PEAK_GBPS},
        "cold_cache": None if cold is None else {
            **cold, "layer_hbm_frac": cost["bytes"] / (cold["ms_median"] / 1e3) / 1e9 / HBM_PEAK_GBPS},
        "cpu_baseline": cpu,
    }


TIMING_TEXT = ("K host-launched steps between two HIP events on the launch stream; in every "
               f"{EVENT_EVERY}th step two more events bracket the gate_up GEMM (roofline "
               "kernel_us, the mean over those launches); stages_us comes from a separate "
               "pass with all seven stage events")


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode64", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--prefill-leg", type=int, default=1,
                    help="with the default decode64 workload, also time the T=2048 prefill "
                         "layer and report it under `prefill` (1 = yes)")
    ap.add_argument("--prefill-steps", type=int, default=100)
    ap.add_argument("--prefill-warmup", type=int, default=300,
                    help="untimed prefill steps first: after the decode leg and the CPU "
                         "baseline the GPU has idled for tens of seconds, and prefill steps "
                         "only reach their steady time after ~100 (5 warm-up steps measured "
                         "~8% slow)")
    ap.add_argument("--lora-layout", default="per_expert", choices=("per_expert", "shared_outer"),
                    help="LoRA stack layout (shared_outer: A_gu and B_dn one set per adapter)")
    ap.add_argument("--finalize", default="fused", choices=("fused", "external"),
                    help="external: the forward exports per-slot outputs and a separate "
                         "finalize call completes the step")
    ap.add_argument("--routing-method", type=int, default=0, choices=(0, 1),
                    help="0: softmax over the selected experts; 1: over all experts")
    ap.add_argument("--routing-bias-sigma", type=float, default=0.0,
                    help="> 0: a per-expert selection bias drawn N(0, sigma)")
    ap.add_argument("--two-stream", type=int, default=0,
                    help="1: gate_up LoRA shrink on a second stream beside the permute "
                         "(decode-shaped batches)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle baseline time budget (0 = skip)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain copy kernel (torch.neg) over this many MiB, "
                         "to calibrate HBM byte counters against a known size")
    ap.add_argument("--cold-steps", type=int, default=30,
                    help="steps timed one by one after a 512 MiB cache flush (0 = skip)")
    ap.add_argument("--graph", type=int, default=1,
                    help="also time the K steps as one HIP-graph replay (1 = yes)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("STATS_CSV", "OUT_MD"),
                    help="write a kernel-trace summary from rocprofv3 --stats output and exit")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_MD"),
                    help="write an HBM counter summary from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_CSV", "OUT_MD"),
                    help="write an MFMA-counter summary (rocprofv3 --pmc MfmaUtil MfmaFlopsBF16)")
    ap.add_argument("--command", default="", help="the profiling command, recorded in summaries")
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, command=args.command)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma, command=args.command)
        return
    if args.summarize_counters:
        kind = "prefill" if args.workload == "prefill" else "decode"
        summarize_counters(*args.summarize_counters, command=args.command,
                           copy_mib=args.copy_probe_mib or 256, dominant=DOMINANT[kind])
        return

    if args.gpus != 1:
        print(f"bench.py: this layer runs on one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU expert parallelism is a design note only)", file=sys.stderr)
        sys.exit(2)

    r = measure(args, args.workload, args.steps, args.warmup, args.cold_steps, bool(args.graph),
                bool(args.two_stream), args.finalize, args.lora_layout, args.routing_method,
                args.routing_bias_sigma, args.cpu_seconds, args.copy_probe_mib)
    result = {
        "metric": METRIC,
        "value": r["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy PCG64; random-init weights of the layer's shapes)",
        "config": r["config"],
        "roofline": r["roofline"],
        "layer": r["layer"],
        "stages_us": r["stages_us"],
        "timing": TIMING_TEXT,
        "wall_ms_per_step": r["wall_ms_per_step"],
        "graph_replay": r["graph_replay"],
        "cold_cache": r["cold_cache"],
        "cpu_baseline": r["cpu_baseline"],
    }
    # The metric's prefill half: the T=2048 layer, its dominant kernel against
    # the HBM roofline (it sits below the MFMA ridge) and its MFMA fraction.
    if args.workload == "decode64" and args.prefill_leg and args.lora_layout == "per_expert" \
            and args.finalize == "fused" and not args.routing_method and not args.routing_bias_sigma:
        import torch
        torch.cuda.empty_cache()
        p = measure(args, "prefill", args.prefill_steps, args.prefill_warmup,
                    min(args.cold_steps, 10), bool(args.graph), bool(args.two_stream))
        result["prefill"] = {
            "value": p["value"], "unit": "tokens/s", "steps": args.prefill_steps,
            "warmup": args.prefill_warmup,
            "ms_per_step": p["ms_per_step"], "config": p["config"], "roofline": p["roofline"],
            "layer": p["layer"], "stages_us": p["stages_us"], "graph_replay": p["graph_replay"],
            "cold_cache": p["cold_cache"],
        }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
