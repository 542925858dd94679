"""Throughput of the sparse MoE feed-forward layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: the gpt-oss-20b MoE layer at prefill, T = 4,096 tokens, hidden 2,880,
intermediate 2,880, 32 experts, top-4, bf16 activations and weights, fp32
accumulation; seeded synthetic inputs (``synth``), resident in HBM before the
timed region.  A step is one whole forward pass of the layer (router + top-k +
softmax, routing permutation, gate/up GEMM with SiLU*up, down GEMM with the
routing weight, combine), from h to out.

Prints one JSON line: tokens/s over the timed steps, the whole layer's
TFLOP/s and fraction of the bf16 MFMA peak, the roofline of the dominant
kernel (the gate/up grouped GEMM, its launch duration from HIP events recorded
around it on the launch stream during the timed steps), per-stage times from a
second pass that records every stage boundary, a decode measurement (T = 64,
the first 64 rows) against the HBM roofline, the fp64 CPU reference timed
on a bounded sample of the same workload, and decode attention with sinks at
the gpt-oss-20b head shape against the HBM roofline (with its fp64 reference
timed on the same workload).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
METRIC = "MoE-layer tokens/s + % bf16 MFMA peak (prefill), % HBM GB/s (decode)"
DOMINANT_STAGE = 2          # gate/up grouped GEMM
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gateup_gemm_c2_prefill_traffic.json")

# The other layers the method is quoted on: (synth config key, tokens, silent
# expansion factor of the gpt-oss-20b layer, 0 for none or -1 for the
# pre-normalised block around the layer, or the new expert count of an
# expansion by copy map, description).  Expanded layers run at k' = M*k unless
# NARROW_K names the top-k they are deployed with.
OTHER_WORKLOADS = {
    "c3-64a8": (3, 4096, 0, "random 64-expert top-8 layer (64a8 shape), prefill T=4096, bf16"),
    "c3-96a12": (2, 4096, 3, "gpt-oss-20b layer silently expanded x3 (96a12), top-12, prefill T=4096, bf16"),
    "c4": (4, 8192, 0, "gpt-oss-120b-shaped layer (128 experts, top-4), MXFP4 experts, 8 hot experts ~50% of "
                       "assignments, prefill T=8192"),
    "c5": (5, 2048, 0, "220a20b-shaped layer (248 experts, top-20), MXFP4 experts, prefill T=2048"),
    "c5-decode": (5, 32, 0, "220a20b-shaped layer (248 experts, top-20), MXFP4 experts, decode T=32"),
    "c3-64a4": (2, 4096, 2, "deploy-narrow 64a4: gpt-oss-20b layer silently expanded x2 (64 experts), run at top-4, "
                            "prefill T=4096, bf16"),
    "c3-96a4": (2, 4096, 3, "deploy-narrow 96a4: gpt-oss-20b layer silently expanded x3 (96 experts), run at top-4, "
                            "prefill T=4096, bf16"),
    "c4-248a20": (4, 2048, 248, "248 expert rows (128 base + 120 added, added row 128+j a copy of base row j) built "
                                "from the 120b-shaped MXFP4 layer, top-20, prefill T=2048"),
    "block-c2": (2, 4096, -1, "pre-normalised block x + MoE(RMSNorm(x)) on the gpt-oss-20b layer, prefill T=4096, "
                              "bf16, eps 1e-5"),
    "block-c2-decode": (2, 64, -1, "pre-normalised block x + MoE(RMSNorm(x)) on the gpt-oss-20b layer, decode T=64, "
                                   "bf16, eps 1e-5"),
}
BLOCK_EPS = 1e-5
NARROW_K = {"c3-64a4": 4, "c3-96a4": 4, "c4-248a20": 20}
COPY_MAP = {"c4-248a20": list(range(128)) + list(range(120))}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--attn-steps", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=2048)
    ap.add_argument("--workload", default="c2",
                    help="c2 (default: the contract line) or a comma-separated list of "
                         + ", ".join(OTHER_WORKLOADS) + " (one JSON line each)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (reference for HBM byte counters)")
    return ap.parse_args()


def layer_flops(T, H, I, E, k):
    return 2.0 * T * E * H + 6.0 * T * k * H * I


def gateup_flops(T, H, I, k):
    return 4.0 * T * k * H * I


def weight_bytes_touched(counts, H, I, elem_bytes):
    return int((counts > 0).sum()) * 3 * H * I * elem_bytes


def measured_traffic():
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3
    counter summary, valid only while the kernel source and the route scan
    (which cuts the kernel's per-XCD work ranges) are unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        csrc = os.path.join(ROOT, "sparse_mixture_experts_token_amd", "csrc")
        for key, name in (("source_sha256", "gemm_bf16.hip"), ("route_scan_sha256", "route_scan.hip")):
            digest = hashlib.sha256(open(os.path.join(csrc, name), "rb").read()).hexdigest()
            if rec.get(key) != digest:
                return None
        return rec.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        return None


def cpu_baseline(key, T_sample):
    """The fp64 reference as it stands, on the first T_sample tokens."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    L = synth.make_layer(key, T=T_sample)
    c = L.cfg
    w = oracle.LayerWeights.from_storage(c.act, c.expert, L.w_router, L.b_router, L.expert)
    h = oracle.widen(L.h, c.act)
    t0 = time.perf_counter()
    oracle.moe_forward(h, w, c.k)
    dt = time.perf_counter() - t0
    return {"value": T_sample / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {T_sample} of the {c.T} prefill tokens, whole layer in fp64 (NumPy), "
                      f"expert weights generated and widened on the fly; {dt:.1f} s"}


def attention_leg(smoe, torch, dev, steps, cpu=True):
    """Decode attention with sinks at the gpt-oss-20b head shape (64 query
    heads, 8 key/value heads, head dim 64): 64 sequences of 4096 cached keys,
    full attention, seeded N(0, 1) bf16 inputs.  HBM roofline on the bytes the
    step must read and write: every visible key and value row, q, sinks, out."""
    B, Hq, Hkv, Tk, D = 64, 64, 8, 4096, 64
    P = smoe.AttnProblem(B, Hq, Hkv, Tk, D, 0)
    g = torch.Generator(device=dev).manual_seed(20261203)
    q = torch.randn((B, Hq, D), generator=g, device=dev).bfloat16()
    kc = torch.randn((B, Hkv, Tk, D), generator=g, device=dev).bfloat16()
    vc = torch.randn((B, Hkv, Tk, D), generator=g, device=dev).bfloat16()
    sinks = torch.randn((Hq,), generator=g, device=dev).bfloat16()
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(smoe.moe_attn_workspace_bytes(P), dtype=torch.uint8, device=dev)

    def astep():
        smoe.moe_attn_sink_decode(P, q, kc, vc, sinks, None, out, workspace=ws)

    for _ in range(10):
        astep()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        astep()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    byts = 2 * B * Hkv * Tk * D * 2 + 2 * B * Hq * D * 2 + Hq * 2
    gbps = byts / (ms * 1e-3) / 1e9
    res = {"workload": f"decode attention with sinks, {B} sequences x {Tk} keys, {Hq} query / {Hkv} kv heads, "
                       f"head dim {D}, full, bf16", "ms_per_step": round(ms, 4), "alg_bytes": byts,
           "hbm_GBps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
           "sequences_per_s": round(B / (ms * 1e-3), 1), "kernels": "attn_partial_kernel + attn_merge_kernel"}
    if cpu:
        res["cpu_baseline"] = attention_cpu_baseline(Hq, Hkv, Tk, D, n_seq=B)
    return res


def attention_cpu_baseline(Hq, Hkv, Tk, D, n_seq):
    """The fp64 attention reference as it stands on n_seq sequences of the
    same shape (seeded N(0, 1) bf16 inputs, every key visible)."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    inp = synth.attn_inputs(20261203, n_seq, Hq, Hkv, Tk, D)
    w = lambda a: oracle.widen(a, "bf16")
    q, k, v, sinks = w(inp["q"]), w(inp["k"]), w(inp["v"]), w(inp["sinks"])
    t0 = time.perf_counter()
    oracle.attn_sink_decode(q, k, v, sinks, np.full(n_seq, Tk), 0, 1.0 / np.sqrt(D))
    dt = time.perf_counter() - t0
    return {"value": round(n_seq / dt, 2), "unit": "sequences/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_seq} sequences of {Tk} keys (the whole workload), fp64 NumPy, one (sequence, head) "
                      f"at a time; {dt:.2f} s"}


def other_workloads(names, args):
    """One JSON line per named workload: warmup, then args.steps timed steps
    with no events (wall clock around the whole loop), then a second pass with
    an event at every stage boundary for the split.  Prefill lines report
    layer TFLOP/s against the bf16 MFMA peak; decode lines report the touched
    experts' weight bytes (MXFP4: 4.25 bits per parameter) against 8 TB/s."""
    import torch
    import sparse_mixture_experts_token_amd as smoe
    import synth

    dev = torch.device("cuda:0")
    DT = {"f32": smoe.MOE_F32, "bf16": smoe.MOE_BF16, "mxfp4": smoe.MOE_MXFP4}
    layers = {}

    def tod(a, fmt):
        if fmt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    for name in names:
        key, T, M, desc = OTHER_WORKLOADS[name]
        print(f"[bench] {name}", file=sys.stderr, flush=True)
        if key not in layers:
            layers.clear()
            torch.cuda.empty_cache()
            L = synth.make_layer(key)
            st = L.stacked()
            c = L.cfg
            w = {"w_router": tod(L.w_router, c.act), "b_router": tod(L.b_router, c.act)}
            for n in ("gate", "up", "down"):
                w["w_" + n] = tod(st[n], c.expert)
                if c.expert == "mxfp4":
                    w["s_" + n] = tod(st["s_" + n], "u8")
            del st
            layers[key] = (L, w)
        L, w = layers[key]
        c = L.cfg
        E, k = c.E, c.k
        if name in COPY_MAP:  # expansion by a copy map on the device
            cmap = COPY_MAP[name]
            base = smoe.Problem(0, c.H, c.I, E, k, DT[c.act], DT[c.expert])
            w = {n: torch.empty((len(cmap),) + tuple(t.shape[1:]), dtype=t.dtype, device=dev)
                 for n, t in layers[key][1].items()}
            smoe.moe_expand_copies(base, layers[key][1], cmap, w)
            E = len(cmap)
        elif M > 1:  # silent expansion on the device: every expert tensor repeated M times
            base = smoe.Problem(0, c.H, c.I, E, k, DT[c.act], DT[c.expert])
            w = {n: torch.empty((M * t.shape[0],) + tuple(t.shape[1:]), dtype=t.dtype, device=dev)
                 for n, t in layers[key][1].items()}
            smoe.moe_expand_silent(base, layers[key][1], M, w)
            E, k = M * E, M * k
        k = NARROW_K.get(name, k)
        prob = smoe.Problem(T, c.H, c.I, E, k, DT[c.act], DT[c.expert])
        offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
        if M < 0:  # the pre-normalised block: x = h with rows rescaled, gain g
            x_np, g_np = synth.block_inputs(L)
            h, gain = tod(x_np[:T], c.act), tod(g_np, c.act)
            nb = smoe.moe_block_workspace_bytes(prob)
        else:
            h = tod(L.h[:T], c.act)
            nb = smoe.moe_workspace_bytes(prob)
        out = torch.empty((T, c.H), dtype=h.dtype, device=dev)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)

        def step():
            if M < 0:
                smoe.moe_block_forward(prob, w, gain, BLOCK_EPS, h, out, routing={"expert_offsets": offs},
                                       workspace=ws, workspace_bytes=nb)
            else:
                smoe.moe_forward(prob, w, h, out, routing={"expert_offsets": offs}, workspace=ws,
                                 workspace_bytes=nb)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        smoe.moe_profile_begin(args.steps)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        stage_ms, calls = smoe.moe_profile_end()
        F = layer_flops(T, c.H, c.I, E, k)
        res = {"metric": METRIC, "value": round(T / dt, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
               "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 4), "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
               "config": {"workload": desc, "T": T, "hidden": c.H, "intermediate": c.I, "experts": E, "top_k": k,
                          "experts_format": c.expert},
               "layer_tflops": round(F / dt / 1e12, 2), "layer_mfma_frac": round(F / dt / 1e12 / PEAK_BF16_TFLOPS, 4),
               "stage_ms_profiled_pass": {smoe.moe_stage_name(i): round(x / calls, 5)
                                          for i, x in enumerate(stage_ms)}}
        if T <= 64:
            counts = np.diff(offs.cpu().numpy())
            per_expert = 3 * c.H * c.I * (17 / 32 if c.expert == "mxfp4" else 2)
            Bd = int((counts > 0).sum() * per_expert) + E * c.H * 2 + E * 2 + 2 * T * c.H * 2
            res["decode"] = {"experts_touched": int((counts > 0).sum()), "alg_bytes": Bd,
                             "hbm_GBps": round(Bd / dt / 1e9, 1), "hbm_frac": round(Bd / dt / 1e9 / PEAK_HBM_GBPS, 4)}
        print(json.dumps(res), flush=True)
        del w, h, out, ws


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.workload != "c2":
        names = args.workload.split(",")
        unknown = [n for n in names if n not in OTHER_WORKLOADS]
        if unknown:
            print(json.dumps({"error": f"unknown workload(s) {unknown}", "known": ["c2"] + list(OTHER_WORKLOADS)}))
            sys.exit(2)
        other_workloads(names, args)
        return

    import torch
    import sparse_mixture_experts_token_amd as smoe
    import synth

    if args.calibrate_copy:
        n = 1 << 30
        a = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}))
        return

    key = 2
    c = synth.CONFIGS[key]
    L = synth.make_layer(key)
    st = L.stacked()
    dev = torch.device("cuda:0")

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    w = {"w_router": bf16(L.w_router), "b_router": bf16(L.b_router), "w_gate": bf16(st["gate"]),
         "w_up": bf16(st["up"]), "w_down": bf16(st["down"])}
    del st
    h = bf16(L.h)
    T, H, I, E, k = c.T, c.H, c.I, c.E, c.k
    prob = smoe.Problem(T, H, I, E, k, smoe.MOE_BF16, smoe.MOE_BF16)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws_bytes = smoe.moe_workspace_bytes(prob)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    routing = {"expert_offsets": offsets}

    def step():
        smoe.moe_forward(prob, w, h, out, routing=routing, workspace=ws, workspace_bytes=ws_bytes)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed steps: HIP events only around the dominant kernel (each event costs
    # a few microseconds of device time) ...
    smoe.moe_profile_begin_mask(args.steps, (1 << DOMINANT_STAGE) | (1 << (DOMINANT_STAGE + 1)))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    dom_ms, calls = smoe.moe_profile_end()
    ms_step = dt * 1e3 / args.steps
    # ... and the per-stage split from a second pass with every boundary recorded
    smoe.moe_profile_begin(args.steps)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    stage_ms, scalls = smoe.moe_profile_end()
    stage_avg = [x / scalls for x in stage_ms]
    F = layer_flops(T, H, I, E, k)
    tok_s = T / (dt / args.steps)

    g_ms = dom_ms[DOMINANT_STAGE] / calls
    g_tflops = gateup_flops(T, H, I, k) / (g_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(g_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(g_tflops / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                "kernel": "gateup_bf16_kernel (gate/up grouped GEMM + SiLU*up)", "flops_per_launch": gateup_flops(T, H, I, k),
                "avg_launch_ms": round(g_ms, 5)}

    # ---- decode: first 64 tokens, HBM roofline on the touched experts' weights ----
    Td = c.T_decode
    pd = smoe.Problem(Td, H, I, E, k, smoe.MOE_BF16, smoe.MOE_BF16)
    hd = h[:Td].contiguous()
    outd = torch.empty((Td, H), dtype=torch.bfloat16, device=dev)
    wsd_bytes = smoe.moe_workspace_bytes(pd)
    wsd = torch.empty(wsd_bytes, dtype=torch.uint8, device=dev)
    offd = torch.empty(E + 1, dtype=torch.int32, device=dev)
    def dstep():
        smoe.moe_forward(pd, w, hd, outd, routing={"expert_offsets": offd}, workspace=wsd, workspace_bytes=wsd_bytes)

    for _ in range(20):
        dstep()
    torch.cuda.synchronize()
    # timed without the per-stage events (at this size they would add ~6%) ...
    t1 = time.perf_counter()
    for _ in range(args.decode_steps):
        dstep()
    torch.cuda.synchronize()
    ddt = (time.perf_counter() - t1) / args.decode_steps
    # ... and the per-stage split from a second pass with them
    smoe.moe_profile_begin(args.decode_steps)
    for _ in range(args.decode_steps):
        dstep()
    torch.cuda.synchronize()
    dstage, dcalls = smoe.moe_profile_end()
    counts_d = np.diff(offd.cpu().numpy())
    Bd = weight_bytes_touched(counts_d, H, I, 2) + E * H * 2 + E * 2 + 2 * Td * H * 2
    # ... and cold: a 1 GiB read before every step evicts the weights from
    # the 256 MB Infinity Cache (a read, so the evicted lines are clean and
    # cost no write-back inside the step); the reads are timed alone and
    # subtracted
    flush = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    n_cold = max(1, args.decode_steps // 4)
    for _ in range(3):
        torch.sum(flush, dim=0, out=sink)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(n_cold):
        torch.sum(flush, dim=0, out=sink)
        dstep()
    torch.cuda.synchronize()
    t_both = time.perf_counter() - t2
    t3 = time.perf_counter()
    for _ in range(n_cold):
        torch.sum(flush, dim=0, out=sink)
    torch.cuda.synchronize()
    cold = (t_both - (time.perf_counter() - t3)) / n_cold
    del flush, sink
    decode = {"workload": f"first {Td} tokens, same layer", "tokens_per_s": round(Td / ddt, 1),
              "ms_per_step": round(ddt * 1e3, 4), "alg_bytes": Bd, "hbm_GBps": round(Bd / ddt / 1e9, 1),
              "hbm_frac": round(Bd / ddt / 1e9 / PEAK_HBM_GBPS, 4),
              "cold_ms_per_step": round(cold * 1e3, 4), "cold_hbm_frac": round(Bd / cold / 1e9 / PEAK_HBM_GBPS, 4),
              "stage_ms_profiled_pass": [round(x / dcalls, 5) for x in dstage]}

    del wsd, outd, hd
    attention = attention_leg(smoe, torch, dev, args.attn_steps, cpu=not args.no_cpu_baseline)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(key, args.cpu_sample_tokens)

    res = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gpt-oss-20b MoE layer prefill, T=4096, hidden 2880, intermediate 2880, "
                               "32 experts, top-4, bf16, fp32 accumulate", "T": T, "hidden": H,
                   "intermediate": I, "experts": E, "top_k": k},
        "layer_tflops": round(F / (ms_step * 1e-3) / 1e12, 2),
        "layer_mfma_frac": round(F / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "stage_ms_profiled_pass": {smoe.moe_stage_name(i): round(x, 5) for i, x in enumerate(stage_avg)},
        "roofline": roofline, "decode": decode, "attention": attention, "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
