#!/usr/bin/env python3
"""Benchmark of the 2-bit routed-expert MoE forward on one MI355X.

Default workload (the decode shape the metric is quoted on): one MoE layer with K=4096, I=2048,
E=256, top-8, uniform routing, 2-bit codes uniform over {-4,-1,1,4}, UE8M0 block-32 exponents
uniform in [-10,-6], bf16 N(0,1) activations. One step runs the whole forward (route, gate_up +
SiLU, down, combine) once for each decode batch T = 1, 8 and 32 (41 tokens per step), each call on
a fresh routing instance (cycling through --instances seeded instances) and on alternating copies
of the layer's planes, so consecutive calls never find their weights in the 256 MB last-level
cache. Inputs are resident in HBM before timing. The timed steps are captured in one HIP graph and
replayed (a serving loop replays captured decode steps the same way); value = tokens per second
over that replay, wall clock between two device synchronisations. eager_tokens_per_s is the same
work launched call by call from Python.

The JSON line also carries:
  roofline      - the dominant kernel (the decode gate_up kernel): algorithmic bytes (weights of
                  the activated experts, x read, gated intermediate written) / its average launch
                  duration, from HIP events around a graph of back-to-back launches of that stage
                  (same inputs, same launch configuration) on the stream it runs on;
  per_batch     - per-T forward time, whole-forward algorithmic HBM rate and its fraction of peak;
  cold_calls    - per-call forward times (p10 / median / p90 over 100 calls per T) with a 1 GiB
                  scratch copy before every call, so no call finds weights in the 256 MB last-level
                  cache, timed with an event pair each (the pair's own cost is reported beside);
  prefill       - the 8192-token prefill workload (K=6144, Zipf(1.1) routing): tokens/s and matrix
                  core rate of the two grouped GEMMs against the dense bf16/fp16 peak;
  zipf_decode   - the 64-token Zipf-routed decode batch at K=6144: time, active experts, HBM rate;
  slots         - the expert-slot forward against the plain forward at T=8 and 32;
  w4            - the FP4 (MXFP4) expert planes: decode at T=1, 8, 32 and the prefill GEMMs;
  nvfp4         - the NVFP4 expert planes (e2m1, E4M3 per 16, fp32 scale_2): decode at T=1, 8, 32 and
                  the prefill GEMMs;
  requant       - the three load-time re-quantizers (NVFP4, FP8 block-128, MXFP4) over 256 tensors;
  sweep         - the sign-bias diagnostic: 8 synthetic expert tensors of [2048, 6144] against all
                  1239 candidate codebooks, with the symmetric / asymmetric statistics it finds;
  cpu_baseline  - the f64 CPU oracle on a bounded sample of the same workload (the prefill, Zipf
                  decode and re-quantizer legs carry their own oracle timing).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix peak
MFMA_FP6_PEAK_TFLOPS = 10100.0  # MI355X dense fp6 / fp4 matrix peak (the instruction the GEMMs issue)
A_PARTS = 3                     # the GEMMs' activations enter as three e2m3 parts: 3 instructions per product
COLD_CALLS = 100                # per-call timing: calls per batch shape, each after a 1 GiB scratch copy
REQUANT_THREADS = max(1, min(16, os.cpu_count() or 1))   # OpenMP threads of the C re-quantizer oracle
CPU_WORKERS = 1                 # CPU oracle legs: the oracle as it stands (one expert at a time, BLAS threads inside)
DECODE_TS = (1, 8, 32)
DIRECT_MAX_PAIRS = 8            # pairs up to which the forward takes the two-kernel direct path
# VALU issue peak: 256 CUs x 4 SIMDs x 2.4 GHz, one wave64 instruction per SIMD every 4 cycles
VALU_PEAK_LANE_OPS = 256 * 4 * 2.4e9 / 4 * 64
# VALU instructions per element per candidate exponent in the codebook sweep's main loop (the
# high-word-select, no-zero variant taken by e2m1 codebooks): 335 per 32 elements in the gfx950
# assembly hipcc -O3 emits for sweep.hip
SWEEP_VALU_PER_EVAL = 335 / 32


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--instances", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-iters", type=int, default=5)
    ap.add_argument("--no-requant", action="store_true")
    ap.add_argument("--no-slots", action="store_true")
    ap.add_argument("--no-w4", action="store_true")
    ap.add_argument("--requant-iters", type=int, default=5)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-shards", action="store_true")
    ap.add_argument("--sweep-tensors", type=int, default=8)
    ap.add_argument("--sweep-iters", type=int, default=2)
    ap.add_argument("--eager", action="store_true",
                    help="launch every timed call from Python instead of replaying HIP graphs (for profilers)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the 2-bit prefill leg (for counter profiles of the grouped GEMMs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run three 1 GiB device-to-device copies (a plain copy kernel of known size, "
                         "to scale the HBM byte counters of a profile)")
    return ap.parse_args()


def expert_bytes(K, I):
    """Bytes of one expert's 2-bit planes: codes (2 bits) + one UE8M0 byte per 32 weights."""
    gu = 2 * I * K // 4 + 2 * I * K // 32
    dn = K * I // 4 + K * I // 32
    return gu, dn


DECODE_SOURCES = ("common.h", "internal.h", "decode.hip")


def kernel_source_hash(files=DECODE_SOURCES):
    """Hash of the sources a kernel is built from: a counter summary taken on other sources is stale."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bit_routed_expert_amd", "csrc")
    for f in files:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(name, src_hash):
    """HBM bytes per launch from a committed counter summary (profiles/<name>_traffic.txt, lines
    `source_hash: <hex>` and `bytes_per_launch: <int>`), if it was taken on these sources."""
    p = os.path.join(ROOT, "profiles", f"{name}_traffic.txt")
    if not os.path.exists(p):
        return None
    fields = {}
    with open(p) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_hash") != src_hash or "bytes_per_launch" not in fields:
        return None
    return int(fields["bytes_per_launch"])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_routed_expert_amd as moe
    import workloads

    torch.cuda.set_device(0)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.prefill_only:
        args.no_cpu_baseline = True
        res, _, _ = bench_prefill(args, moe, workloads, torch, dev, zipf=False)
        print(json.dumps(dict(prefill=res)), flush=True)
        return
    c = workloads.DECODE
    K, I, E, top_k = c["K"], c["I"], c["E"], c["top_k"]
    canon = workloads.decode_layer()
    d_canon = [dev(canon[k]) for k in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")]
    layers = [moe.moe_w2_pack(*d_canon), moe.moe_w2_pack(*d_canon)]   # two copies at distinct addresses
    del d_canon
    torch.cuda.empty_cache()

    R = args.instances
    inst = {}
    for T in DECODE_TS:
        lst = []
        for d in workloads.decode_instances(T, R):
            lst.append(dict(
                x=torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).cuda(),
                ids=dev(d["topk_ids"]), w=dev(d["topk_w"]), ids_np=d["topk_ids"], host=d))
        inst[T] = lst
    ws = {T: moe.alloc_workspace(layers[0], T, top_k) for T in DECODE_TS}
    ys = {T: torch.empty((T, K), dtype=torch.bfloat16, device="cuda") for T in DECODE_TS}
    gu_b, dn_b = expert_bytes(K, I)

    def n_active(ids):
        v = ids[(ids >= 0) & (ids < E)]
        return len(np.unique(v))

    # algorithmic bytes per call
    def call_bytes(T, ids):
        na = n_active(ids)
        gate_up = na * gu_b + T * K * 2 + T * top_k * I * 2
        full = na * (gu_b + dn_b) + 2 * T * K * 2 + T * top_k * 8
        return gate_up, full

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def fwd(s, i, T):
        call = 3 * s + i
        d = inst[T][s % R]
        moe.moe_w2_forward(layers[call % 2], d["x"], d["ids"], d["w"], workspace=ws[T], y=ys[T])

    for s in range(args.warmup):
        for i, T in enumerate(DECODE_TS):
            fwd(s, i, T)
    torch.cuda.synchronize()
    # eager reference: the same steps launched one by one from Python
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, T in enumerate(DECODE_TS):
            fwd(s, i, T)
    torch.cuda.synchronize()
    eager_elapsed = time.perf_counter() - t0
    # ---- timed region: the K steps captured once in a HIP graph and replayed; nothing else runs ----
    def timed_steps():
        for s in range(args.steps):
            for i, T in enumerate(DECODE_TS):
                fwd(s, i, T)
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            timed_steps()
        # untimed warm replays, at least ~50 ms of GPU work: the GPU idles while the graph is
        # captured, and its clocks take a few milliseconds of load to come back up
        replay_s = max(eager_elapsed, 1e-4)     # one replay runs about as long as the eager steps
        for _ in range(max(2, int(math.ceil(0.05 / replay_s)))):
            graph.replay()
    torch.cuda.synchronize()
    g0, g1 = ev(), ev()
    t0 = time.perf_counter()
    g0.record(stream)
    if args.eager:
        timed_steps()
    else:
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    tokens = sum(DECODE_TS) * args.steps
    value = tokens / elapsed

    # ---- per-kernel timing: each stage launched back-to-back between one pair of events ----
    # (an event between two launches leaves an idle gap on the stream, so none is placed there)
    kws = {T: [moe.alloc_workspace(layers[0], T, top_k) for _ in range(R)] for T in DECODE_TS}
    for T in DECODE_TS:
        for r in range(R):
            d = inst[T][r]
            moe.moe_w2_forward(layers[0], d["x"], d["ids"], d["w"], workspace=kws[T][r], y=ys[T])
    torch.cuda.synchronize()
    n_rep = max(2, args.steps)
    per_batch, gu_bytes_all, gu_ms_all, n_gu = {}, 0, 0.0, 0
    for T in DECODE_TS:
        res = {}
        for name, stage in (("gate_up", moe.STAGE_GATE_UP), ("down", moe.STAGE_DOWN), ("forward", None)):
            a0, a1 = ev(), ev()
            def loop():
                nb_gu = nb_full = 0
                for k in range(n_rep):
                    r = k % R
                    d = inst[T][r]
                    layer = layers[k % 2]
                    if stage is None:
                        moe.moe_w2_forward(layer, d["x"], d["ids"], d["w"], workspace=kws[T][r], y=ys[T])
                    else:
                        moe.moe_w2_forward_stage(stage, layer, d["x"], d["ids"], d["w"], ys[T], kws[T][r])
                    gb, fb = call_bytes(T, d["ids_np"])
                    nb_gu += gb
                    nb_full += fb
                return nb_gu, nb_full
            if args.eager:
                loop()
                torch.cuda.synchronize()
                a0.record(stream)
                nbytes_gu, nbytes_full = loop()
                a1.record(stream)
            else:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    nbytes_gu, nbytes_full = loop()
                g.replay()
                torch.cuda.synchronize()
                a0.record(stream)
                g.replay()
                a1.record(stream)
            torch.cuda.synchronize()
            ms = a0.elapsed_time(a1) / n_rep
            res[name] = ms
            if name == "gate_up":
                res["gu_GBps"] = nbytes_gu / n_rep / (ms * 1e-3) / 1e9
                if T * top_k > DIRECT_MAX_PAIRS:
                    # the routed decode gate/up kernel (T = 1 takes the direct kernel instead)
                    gu_bytes_all += nbytes_gu
                    gu_ms_all += ms * n_rep
                    n_gu += n_rep
            if name == "forward":
                res["fwd_GBps"] = nbytes_full / n_rep / (ms * 1e-3) / 1e9
        per_batch[f"T{T}"] = dict(
            fwd_us=round(res["forward"] * 1e3, 2), gate_up_us=round(res["gate_up"] * 1e3, 2),
            down_us=round(res["down"] * 1e3, 2), fwd_hbm_GBps=round(res["fwd_GBps"], 1),
            fwd_hbm_frac=round(res["fwd_GBps"] / HBM_PEAK_GBPS, 4),
            fwd_us_at_70pct_hbm=round(nbytes_full / n_rep / (0.7 * HBM_PEAK_GBPS * 1e3), 2),
            gate_up_hbm_GBps=round(res["gu_GBps"], 1), tokens_per_s=round(T / (res["forward"] * 1e-3), 1))
    achieved = gu_bytes_all / (gu_ms_all * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    traffic = traffic_from_profiles("decode_gate_up", src_hash)
    roofline = dict(bound="hbm", kernel="decode_gate_up_kernel<4,0,0> (routed decode, 2-bit planes; T=8 and T=32 calls)",
                    scope="the dominant kernel alone; whole_forward_frac has each decode shape's whole forward",
                    achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBPS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBPS, 4),
                    traffic=traffic, launches=n_gu, avg_launch_us=round(gu_ms_all / n_gu * 1e3, 3),
                    algorithmic_bytes_per_launch=int(gu_bytes_all / n_gu),
                    whole_forward_frac={k: v["fwd_hbm_frac"] for k, v in per_batch.items()})
    del kws

    out = {
        "metric": "routed-expert tokens/sec (decode, K=4096 I=2048 E=256 top-8, T in {1,8,32})",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "gpu_ms_per_step": round(g0.elapsed_time(g1) / args.steps, 4),
        "eager_tokens_per_s": round(tokens / eager_elapsed, 1),
        "timing": ("eager launches" if args.eager else
                   "timed steps captured in one HIP graph and replayed; per-kernel times from graphs "
                   "of back-to-back launches of that stage between one event pair"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3(split x2/x3)*e2m1->f32",
        "dtype_note": ("bf16 x and fp16 gated intermediate enter the block-scaled matrix instruction as exact "
                       "e4m3 parts (two for x, three for the intermediate) times the e2m1 weights with their UE8M0 "
                       "scales; fp32 accumulation; bf16 output = RNE of the fp32 result"),
        "data": "synthetic",
        "config": {"workload": "moe_w2 decode: K=4096 I=2048 E=256 top-8 uniform routing, "
                               "one forward each at T=1,8,32 per step (41 tokens)",
                   "tokens_per_step": sum(DECODE_TS), "routing_instances": R, "plane_copies": 2},
        "roofline": roofline,
        "per_batch": per_batch,
        "source_hash": src_hash,
    }

    out["cold_calls"] = bench_cold_calls(torch, moe, layers, inst, ws, ys, per_batch)
    # the 2-bit prefill leg (the other headline workload) next, then the secondary legs
    zipf_host = None
    if not args.no_prefill:
        out["prefill"], out["zipf_decode"], zipf_host = bench_prefill(args, moe, workloads, torch, dev)
    if not args.no_shards:
        out["tp_shards"] = bench_shards(args, moe, workloads, torch, dev, inst)
    if not args.no_slots:
        out["slots"] = bench_slots(args, moe, torch, dev, canon, inst, E, top_k, K)
    if not args.no_w4:
        out["w4"] = bench_w4(args, moe, workloads, torch, dev, inst, E, top_k, K, I)
        out["nvfp4"] = bench_nvfp4(args, moe, workloads, torch, dev, inst, E, top_k, K, I)
    if not args.no_requant:
        out["requant"] = bench_requant(args, moe, workloads, torch, dev)
    if not args.no_sweep:
        out["sweep"] = bench_sweep(args, moe, workloads, torch, dev)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(canon, inst)
        if not args.no_prefill and zipf_host is not None:
            out["prefill"]["cpu_baseline"] = cpu_baseline_prefill(zipf_host, out["prefill"])
            out["zipf_decode"]["cpu_baseline"] = cpu_baseline_zipf(zipf_host["planes"], workloads)
        if not args.no_requant:
            out["requant"]["cpu_baseline"] = cpu_baseline_requant(workloads)
    print(json.dumps(out), flush=True)


def cold_call_times(torch, call, n, flush_bytes=1 << 30):
    """n calls of call(k), each after a copy of a flush_bytes scratch buffer (which displaces the
    last-level cache) and between its own event pair on the current stream; also n empty event
    pairs after the same copy. Returns (per-call us, empty-pair us) as numpy arrays."""
    src = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    pairs, empty = [], []
    for k in range(n):
        dst.copy_(src)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call(k)
        b.record(stream)
        pairs.append((a, b))
    for k in range(n):
        dst.copy_(src)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        b.record(stream)
        empty.append((a, b))
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
    e = np.array([a.elapsed_time(b) * 1e3 for a, b in empty])
    del src, dst
    torch.cuda.empty_cache()
    return t, e


def pct(a):
    p10, p50, p90 = np.percentile(a, [10, 50, 90])
    return dict(p10=round(float(p10), 2), median=round(float(p50), 2), p90=round(float(p90), 2))


def bench_cold_calls(torch, moe, layers, inst, ws, ys, per_batch):
    """Per-call forward times at T = 1, 8, 32 (COLD_CALLS calls each, cycling the routing instances
    and the two plane copies), every call after a 1 GiB scratch copy: the distribution behind the
    graph-replay figures, and the check that those figures do not come from weights left in the
    256 MB last-level cache (graph_vs_cold = back-to-back graph time / cold median, the latter
    minus the event pair's own cost)."""
    out = {}
    for T in DECODE_TS:
        R = len(inst[T])

        def call(k):
            d = inst[T][k % R]
            moe.moe_w2_forward(layers[k % 2], d["x"], d["ids"], d["w"], workspace=ws[T], y=ys[T])
        call(0)
        t, e = cold_call_times(torch, call, COLD_CALLS)
        pe = float(np.median(e))
        out[f"T{T}"] = dict(**pct(t), event_pair_us=round(pe, 2), calls=COLD_CALLS,
                            graph_vs_cold=round(per_batch[f"T{T}"]["fwd_us"] / (float(np.median(t)) - pe), 4))
    out["note"] = ("each call between its own event pair after a 1 GiB device copy; the pair alone (event_pair_us, "
                   "after the same copy) costs a few us, so medians minus event_pair_us compare with per_batch")
    return out


def bench_shards(args, moe, workloads, torch, dev, inst):
    """One GPU's share of the layer under tensor parallelism over the expert intermediate size
    (G = 2, 4 ranks: I = 1024, 512; the pages ship kernels for these shard widths): each rank holds
    gate_up rows I/G and the down reduction I/G of every expert, sees every token and produces a
    partial y (the cross-rank sum is out of scope). Decode at K=4096 T = 1, 8, 32 with the decode
    workload's routing instances and x, and the Zipf T=64 batch at K=6144; each shape timed as a
    graph of back-to-back forwards over two plane copies; algorithmic bytes per call = the
    instance's active experts' shard planes + x + y + ids + w."""
    E, top_k = 256, 8
    stream = torch.cuda.current_stream()
    n_rep = max(2, args.steps)

    def timed(layers, insts, K, I):
        R = len(insts)
        T = insts[0]["x"].shape[0]
        ws = [moe.alloc_workspace(layers[0], T, top_k) for _ in range(R)]
        y = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
        gu_b, dn_b = expert_bytes(K, I)
        nb = 0
        def loop():
            nb = 0
            for k in range(n_rep):
                d = insts[k % R]
                moe.moe_w2_forward(layers[k % 2], d["x"], d["ids"], d["w"], workspace=ws[k % R], y=y)
                ids = d["ids_np"]
                nb += len(np.unique(ids[(ids >= 0) & (ids < E)])) * (gu_b + dn_b) + 2 * T * K * 2 + T * top_k * 8
            return nb
        loop()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            nb = loop()
        g.replay()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        g.replay()
        a1.record(stream)
        torch.cuda.synchronize()
        us = a0.elapsed_time(a1) / n_rep * 1e3
        gbps = nb / n_rep / (us * 1e-6) / 1e9
        return dict(fwd_us=round(us, 2), hbm_GBps=round(gbps, 1), hbm_frac=round(gbps / HBM_PEAK_GBPS, 4),
                    tokens_per_s=round(T / (us * 1e-6), 1))

    # the 8192-token prefill batch (the prefill leg's Zipf instance) on a rank's share at K=6144:
    # forward and GEMM stage times, algorithmic flops 2*P*3*(I/G)*K against the bf16 peak
    pre = None
    if not args.no_prefill:
        cp = workloads.PREFILL
        dp = workloads.zipf_instances(cp["T"], 1, cp["seed"], cp["K"], E, top_k)[0]
        pre = (torch.from_numpy(dp["x"].view(np.int16)).view(torch.bfloat16).cuda(), dev(dp["topk_ids"]),
               dev(dp["topk_w"]))

    def prefill_stages(planes, K, I):
        x, ids, w = pre
        T = x.shape[0]
        ws = moe.alloc_workspace(planes, T, top_k)
        y = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
        for _ in range(2):
            moe.moe_w2_forward(planes, x, ids, w, workspace=ws, y=y)
        torch.cuda.synchronize()
        t = {}
        for name, st in (("forward", None), ("gate_up", moe.STAGE_GATE_UP), ("down", moe.STAGE_DOWN)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.prefill_iters):
                if st is None:
                    moe.moe_w2_forward(planes, x, ids, w, workspace=ws, y=y)
                else:
                    moe.moe_w2_forward_stage(st, planes, x, ids, w, y, ws)
            e1.record(stream)
            torch.cuda.synchronize()
            t[name] = e0.elapsed_time(e1) / args.prefill_iters
        del ws, y
        fl = 2.0 * T * top_k * 3 * I * K
        return dict(fwd_ms=round(t["forward"], 4), gate_up_ms=round(t["gate_up"], 4), down_ms=round(t["down"], 4),
                    gemm_mfma_frac=round(fl / ((t["gate_up"] + t["down"]) * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                    fwd_mfma_frac=round(fl / (t["forward"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4))

    out = {}
    cz = workloads.DECODE_ZIPF
    zi = workloads.zipf_instances(cz["T"], 16, cz["seed"], cz["K"], E, top_k)
    zinst = [dict(x=torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).cuda(), ids=dev(d["topk_ids"]),
                  w=dev(d["topk_w"]), ids_np=d["topk_ids"]) for d in zi]
    for G in (2, 4):
        res = {}
        for K, insts_by_T in ((4096, {T: inst[T] for T in DECODE_TS}), (cz["K"], {cz["T"]: zinst})):
            I = 2048 // G
            canon = workloads.draw_planes(np.random.default_rng([20, G, K]), E, K, I)
            d_canon = [dev(canon[k]) for k in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")]
            layers = [moe.moe_w2_pack(*d_canon), moe.moe_w2_pack(*d_canon)]
            del canon, d_canon
            for T, insts in insts_by_T.items():
                key = f"T{T}" if K == 4096 else f"zipf_T{T}_K{K}"
                res[key] = timed(layers, insts, K, I)
            if K == cz["K"] and pre is not None:
                res["prefill_T8192_K6144"] = prefill_stages(layers[0], K, I)
            for h in layers:
                h.free()
            torch.cuda.empty_cache()
        out[f"tp{G}_I{2048 // G}"] = res
    out["workload"] = ("one rank's share under tensor parallelism over I: moe_w2 decode K=4096 E=256 top-8 uniform "
                       "routing at T=1,8,32 and the Zipf(1.1) T=64 batch at K=6144, I = 2048/G; with the prefill "
                       "leg, the T=8192 Zipf(1.1) batch at K=6144 on the same shard planes (GEMM stages)")
    return out


def w4_expert_bytes(K, I):
    """Bytes of one expert's FP4 planes: e2m1 codes (4 bits) + one UE8M0 byte per 32 weights."""
    return 2 * I * K // 2 + 2 * I * K // 32, K * I // 2 + K * I // 32


def nvfp4_expert_bytes(K, I):
    """Bytes of one expert's NVFP4 planes: e2m1 codes (4 bits) + one E4M3 byte per 16 weights
    (scale_2, 12 bytes per expert, is left out)."""
    return 2 * I * K // 2 + 2 * I * K // 16, K * I // 2 + K * I // 16


def time_decode_layers(args, moe, torch, layers, inst, E, top_k, K, gu_b, dn_b):
    """Per decode T: back-to-back moe_w4_forward calls over the routing instances (two plane
    copies alternated) captured in one graph; returns ({"T<n>": ...}, total microseconds)."""
    stream = torch.cuda.current_stream()
    n_rep = max(2, args.steps)
    res, total_us = {}, 0.0
    for T in DECODE_TS:
        R = len(inst[T])
        ws = [moe.alloc_workspace(layers[0], T, top_k) for _ in range(R)]
        y = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
        def loop():
            nb = 0
            for k in range(n_rep):
                d = inst[T][k % R]
                moe.moe_w4_forward(layers[k % 2], d["x"], d["ids"], d["w"], workspace=ws[k % R], y=y)
                ids = d["ids_np"]
                na = len(np.unique(ids[(ids >= 0) & (ids < E)]))
                nb += na * (gu_b + dn_b) + 2 * T * K * 2 + T * top_k * 8
            return nb
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            nbytes = loop()
        g.replay()
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        g.replay()
        a1.record(stream)
        torch.cuda.synchronize()
        ms = a0.elapsed_time(a1) / n_rep
        total_us += ms * 1e3
        gbps = nbytes / n_rep / (ms * 1e-3) / 1e9
        res[f"T{T}"] = dict(fwd_us=round(ms * 1e3, 2), fwd_hbm_GBps=round(gbps, 1),
                            fwd_hbm_frac=round(gbps / HBM_PEAK_GBPS, 3), tokens_per_s=round(T / (ms * 1e-3), 1))
        del ws
    return res, total_us


def bench_w4(args, moe, workloads, torch, dev, inst, E, top_k, K, I):
    """FP4 expert planes on the decode workload (same routing instances and x as the 2-bit decode
    leg; two plane copies alternated), each T timed as a graph of back-to-back forwards; and the
    prefill GEMM stages on the 8192-token Zipf workload."""
    rng = np.random.default_rng(12)
    layers = []
    for _ in range(2):
        canon = workloads.draw_planes_fp4(rng, E, K, I)
        layers.append(moe.moe_w4_pack(*[dev(canon[k]) for k in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")]))
        del canon
    torch.cuda.empty_cache()
    res, total_us = time_decode_layers(args, moe, torch, layers, inst, E, top_k, K, *w4_expert_bytes(K, I))
    for h in layers:
        h.free()
    torch.cuda.empty_cache()
    out = dict(workload="moe_w4 (FP4 e2m1 + UE8M0/32 experts) decode: K=4096 I=2048 E=256 top-8 uniform "
                        "routing, T=1,8,32", decode_tokens_per_s=round(sum(DECODE_TS) / (total_us * 1e-6), 1), **res)
    if not args.no_prefill:
        out["prefill"] = bench_prefill(args, moe, workloads, torch, dev, fmt="w4")
    return out


def bench_nvfp4(args, moe, workloads, torch, dev, inst, E, top_k, K, I):
    """NVFP4 expert planes (e2m1 + E4M3/16 + fp32 scale_2) on the decode workload, as bench_w4."""
    rng = np.random.default_rng(13)
    names = ("gu_codes", "gu_scales", "gu_scale2", "dn_codes", "dn_scales", "dn_scale2")
    layers = []
    for _ in range(2):
        canon = workloads.draw_planes_nvfp4(rng, E, K, I)
        layers.append(moe.moe_w4_pack_nvfp4(*[dev(canon[k]) for k in names]))
        del canon
    torch.cuda.empty_cache()
    res, total_us = time_decode_layers(args, moe, torch, layers, inst, E, top_k, K, *nvfp4_expert_bytes(K, I))
    for h in layers:
        h.free()
    torch.cuda.empty_cache()
    out = dict(workload="moe_w4 (NVFP4 e2m1 + E4M3/16 + fp32 scale_2 experts) decode: K=4096 I=2048 E=256 "
                        "top-8 uniform routing, T=1,8,32",
               decode_tokens_per_s=round(sum(DECODE_TS) / (total_us * 1e-6), 1), **res)
    if not args.no_prefill:
        out["prefill"] = bench_prefill(args, moe, workloads, torch, dev, fmt="nvfp4")
    return out


def bench_slots(args, moe, torch, dev, canon, inst, E, top_k, K):
    """Expert-slot forward (moe_w2_forward_slots) on the decode workload: every expert resident in
    a permuted slot (so each call streams what moe_w2_forward streams), against moe_w2_forward on
    expert-ordered planes, both timed as graphs of back-to-back calls over two plane copies. The
    difference is the cost of the id -> slot pass; the outputs are compared bit for bit."""
    rng = np.random.default_rng(11)
    K_, I = canon["gu_codes"].shape[2] * 4, canon["gu_codes"].shape[1] // 2
    plain, slotted = [], []
    for c in range(2):
        d_canon = [dev(canon[k]) for k in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")]
        plain.append(moe.moe_w2_pack(*d_canon))
        perm = rng.permutation(E).astype(np.int32)
        h = moe.moe_w2_planes_create(E, K_, I)
        for e in range(E):
            moe.moe_w2_pack_slot(h, int(perm[e]), *[t[e] for t in d_canon])
        slotted.append((h, dev(perm)))
        del d_canon
    torch.cuda.empty_cache()
    stream = torch.cuda.current_stream()
    n_rep = max(2, args.steps)
    res = {}
    for T in (8, 32):
        R = len(inst[T])
        ws = [moe.alloc_workspace(plain[0], T, top_k) for _ in range(R)]
        y = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
        y2 = torch.empty_like(y)
        d0 = inst[T][0]
        moe.moe_w2_forward(plain[0], d0["x"], d0["ids"], d0["w"], workspace=ws[0], y=y)
        moe.moe_w2_forward_slots(slotted[0][0], slotted[0][1], d0["x"], d0["ids"], d0["w"], workspace=ws[1 % R], y=y2)
        torch.cuda.synchronize()
        same = bool(torch.equal(y.view(torch.int16), y2.view(torch.int16)))
        out = {"forward": [], "forward_slots": []}
        for name in ("forward", "forward_slots") * 3:   # alternated; medians reported
            def loop():
                for k in range(n_rep):
                    d = inst[T][k % R]
                    if name == "forward":
                        moe.moe_w2_forward(plain[k % 2], d["x"], d["ids"], d["w"], workspace=ws[k % R], y=y)
                    else:
                        h, m = slotted[k % 2]
                        moe.moe_w2_forward_slots(h, m, d["x"], d["ids"], d["w"], workspace=ws[k % R], y=y)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                loop()
            g.replay()
            torch.cuda.synchronize()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            g.replay()
            a1.record(stream)
            torch.cuda.synchronize()
            out[name].append(a0.elapsed_time(a1) / n_rep * 1e3)
        f, fs = float(np.median(out["forward"])), float(np.median(out["forward_slots"]))
        res[f"T{T}"] = dict(fwd_us=round(f, 2), slots_fwd_us=round(fs, 2), slot_pass_us=round(fs - f, 2),
                            bit_identical=same)
        del ws
    for h, _ in slotted:
        h.free()
    for h in plain:
        h.free()
    torch.cuda.empty_cache()
    return dict(workload="moe_w2_forward_slots: decode layer K=4096 I=2048 E=256 top-8, all experts "
                         "resident in permuted slots", **res)


def bench_prefill(args, moe, workloads, torch, dev, fmt="w2", zipf=True):
    """The 8192-token prefill layer (Zipf(1.1) routing) on planes of the given format: "w2" (2-bit),
    "w4" (MXFP4) or "nvfp4"; per-stage times and matrix-core rates."""
    c = workloads.PREFILL
    T, K, I, E, top_k = c["T"], c["K"], c["I"], c["E"], c["top_k"]
    host = None
    fp4 = fmt != "w2"
    if fmt == "w4":
        canon = workloads.draw_planes_fp4(np.random.default_rng(13), E, K, I)
        planes = moe.moe_w4_pack(*[dev(canon[k]) for k in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")])
    elif fmt == "nvfp4":
        canon = workloads.draw_planes_nvfp4(np.random.default_rng(14), E, K, I)
        planes = moe.moe_w4_pack_nvfp4(*[dev(canon[k]) for k in ("gu_codes", "gu_scales", "gu_scale2", "dn_codes",
                                                                  "dn_scales", "dn_scale2")])
    else:
        canon = workloads.zipf_layer(c["seed"], K, I, E)
        dcanon = [dev(canon[k]) for k in ("gu_codes", "gu_scales", "dn_codes", "dn_scales")]
        planes = moe.moe_w2_pack(*dcanon)
        if not args.no_cpu_baseline:
            host = canon          # kept for the CPU oracle legs at the end of the run
    del canon
    d = workloads.zipf_instances(T, 1, c["seed"], K, E, top_k)[0]
    if host is not None:
        host = dict(planes=host, inst=d)
    x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).cuda()
    ids, w = dev(d["topk_ids"]), dev(d["topk_w"])
    ws = moe.alloc_workspace(planes, T, top_k)
    y = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    a = (planes, x, ids, w, y, ws)
    for _ in range(2):
        moe.moe_w2_forward(planes, x, ids, w, workspace=ws, y=y)
    torch.cuda.synchronize()
    t = {}
    n = args.prefill_iters
    for name, stage in (("forward", None), ("route", moe.STAGE_ROUTE), ("gate_up", moe.STAGE_GATE_UP),
                        ("down", moe.STAGE_DOWN), ("combine", moe.STAGE_COMBINE)):
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(n):
            if stage is None:
                moe.moe_w2_forward(planes, x, ids, w, workspace=ws, y=y)
            else:
                moe.moe_w2_forward_stage(stage, *a)
        e1.record(stream)
        torch.cuda.synchronize()
        t[name] = e0.elapsed_time(e1) / n
    fwd, rt, gu, dn, cb = t["forward"], t["route"], t["gate_up"], t["down"], t["combine"]
    P = T * top_k
    f_gu = 2.0 * P * 2 * I * K
    f_dn = 2.0 * P * K * I
    gemm_tflops = (f_gu + f_dn) / ((gu + dn) * 1e-3) / 1e12
    fwd_tflops = (f_gu + f_dn) / (fwd * 1e-3) / 1e12
    del ws, y
    zipf_decode = None
    if not fp4 and zipf:
        zipf_decode = bench_zipf_decode(args, moe, workloads, torch, dev, [planes, moe.moe_w2_pack(*dcanon)])
        del dcanon
    del planes
    torch.cuda.empty_cache()
    label = {"w2": "moe_w2", "w4": "moe_w4 (FP4)", "nvfp4": "moe_w4 (NVFP4)"}[fmt]
    res = dict(
        workload=label + " prefill: T=8192 K=6144 I=2048 E=256 top-8 Zipf(1.1)",
        tokens_per_s=round(T / (fwd * 1e-3), 1), fwd_ms=round(float(fwd), 4),
        route_ms=round(float(rt), 4), gate_up_ms=round(float(gu), 4), down_ms=round(float(dn), 4),
        combine_ms=round(float(cb), 4),
        gate_up_tflops=round(f_gu / (gu * 1e-3) / 1e12, 1), down_tflops=round(f_dn / (dn * 1e-3) / 1e12, 1),
        gemm_tflops=round(gemm_tflops, 1), gemm_mfma_frac=round(gemm_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        fwd_tflops=round(fwd_tflops, 1), fwd_mfma_frac=round(fwd_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        peak_tflops=MFMA_BF16_PEAK_TFLOPS,
        iters=args.prefill_iters)
    if fmt == "nvfp4":
        # the 16 x 16 x 32 bf16 / fp16 instructions, one per product: instruction flops are the
        # algorithmic ones, against the same dense bf16 / fp16 peak
        res.update(gemm_instr_tflops=round(gemm_tflops, 1), gemm_instr_frac=round(gemm_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                   instr_peak_tflops=MFMA_BF16_PEAK_TFLOPS,
                   frac_note="bf16 (gate_up) and fp16 (down) instructions with the weights formed in registers: "
                             "instruction flops = algorithmic flops (2*P*3*I*K), against the dense bf16/fp16 peak")
    else:
        # the instructions actually issued: fp6 (e2m3) activations x fp4 weights, three activation
        # parts per product, against the dense fp6 / fp4 matrix peak
        res.update(gemm_instr_tflops=round(A_PARTS * gemm_tflops, 1),
                   gemm_instr_frac=round(A_PARTS * gemm_tflops / MFMA_FP6_PEAK_TFLOPS, 4),
                   instr_peak_tflops=MFMA_FP6_PEAK_TFLOPS,
                   frac_note=("mfma_frac: algorithmic flops (2*P*3*I*K) per second against the dense bf16 peak; "
                              "instr_frac: the fp6 x fp4 instruction flops issued (3 parts) against the dense "
                              "fp6/fp4 peak"))
    return (res, zipf_decode, host) if not fp4 else res


def bench_zipf_decode(args, moe, workloads, torch, dev, layers, R=16, n_rep=32):
    """The Zipf-routed decode batch: T=64 tokens, K=6144 I=2048 E=256 top-8 with Zipf(1.1) expert
    popularity (R seeded routing instances). The planes are the prefill layer's (same shape; the
    weight values do not change the time), packed twice at distinct addresses and alternated so that
    no call finds its weights in the 256 MB last-level cache. n_rep forwards captured in one HIP
    graph; algorithmic bytes = each instance's active experts' planes + x + y + ids + w."""
    c = workloads.DECODE_ZIPF
    T, K, I, E, top_k = c["T"], c["K"], c["I"], c["E"], c["top_k"]
    insts = workloads.zipf_instances(T, R, c["seed"], K, E, top_k)
    xs = [torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).cuda() for d in insts]
    ids = [dev(d["topk_ids"]) for d in insts]
    ws_ = [dev(d["topk_w"]) for d in insts]
    wss = [moe.alloc_workspace(layers[0], T, top_k) for _ in range(R)]
    y = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    gu_b, dn_b = expert_bytes(K, I)
    nact = [len(np.unique(d["topk_ids"][(d["topk_ids"] >= 0) & (d["topk_ids"] < E)])) for d in insts]

    def timed(path):
        def loop():
            nbytes = 0
            for k in range(n_rep):
                r = k % R
                moe.moe_w2_forward(layers[k % 2], xs[r], ids[r], ws_[r], workspace=wss[r], y=y, path=path)
                nbytes += nact[r] * (gu_b + dn_b) + 2 * T * K * 2 + T * top_k * 8
            return nbytes
        loop()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            nbytes = loop()
        g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n_rep * 1e3, nbytes
    us, nbytes = timed(moe.PATH_AUTO)            # P = 512: the sorted decode organisation
    us_gemm, _ = timed(moe.PATH_GEMM)
    us_routed, _ = timed(moe.PATH_DECODE)
    gbps = nbytes / n_rep / (us * 1e-6) / 1e9

    def call(k):
        r = k % R
        moe.moe_w2_forward(layers[k % 2], xs[r], ids[r], ws_[r], workspace=wss[r], y=y)
    ct, ce = cold_call_times(torch, call, COLD_CALLS)
    cold = dict(**pct(ct), event_pair_us=round(float(np.median(ce)), 2), calls=COLD_CALLS)
    return dict(workload="moe_w2 decode: T=64 K=6144 I=2048 E=256 top-8 Zipf(1.1) routing",
                fwd_us=round(us, 2), tokens_per_s=round(T / (us * 1e-6), 1),
                mean_active_experts=round(float(np.mean(nact)), 1), hbm_GBps=round(gbps, 1),
                hbm_frac=round(gbps / HBM_PEAK_GBPS, 4), us_at_70pct_hbm=round(nbytes / n_rep / (0.7 * HBM_PEAK_GBPS * 1e3), 1),
                gemm_path_fwd_us=round(us_gemm, 2), routed_decode_fwd_us=round(us_routed, 2),
                routing_instances=R, calls=n_rep, cold_calls=cold)


def bench_requant(args, moe, workloads, torch, dev):
    """nvfp4_to_w2 over the n=256 tensors of [2048, 6144]: one synchronous call per iteration,
    timed with events on its stream (the call's flag clear, kernel and status read-back)."""
    c = workloads.REQUANT
    n, R, C = c["n"], c["R"], c["C"]
    e2m1 = torch.empty((n, R, C // 2), dtype=torch.uint8, device="cuda")
    e4m3 = torch.empty((n, R, C // 16), dtype=torch.uint8, device="cuda")
    s2 = np.zeros(n, np.float32)
    for i in range(n):
        a, b, s = workloads.nvfp4_tensor(i)
        e2m1[i].copy_(torch.from_numpy(a))
        e4m3[i].copy_(torch.from_numpy(b))
        s2[i] = s
    s2d = dev(s2)
    codes = torch.empty((n, R, C // 4), dtype=torch.uint8, device="cuda")
    scales = torch.empty((n, R, C // 32), dtype=torch.uint8, device="cuda")
    moe.nvfp4_to_w2(e2m1, e4m3, s2d, codes, scales)
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(args.requant_iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        moe.nvfp4_to_w2(e2m1, e4m3, s2d, codes, scales)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    nbytes = n * R * (C // 2 + C // 16 + C // 4 + C // 32) + 4 * n
    blocks = n * R * (C // 32)
    del e2m1, e4m3, s2d
    torch.cuda.empty_cache()
    out = dict(workload="nvfp4_to_w2: 256 tensors of [2048, 6144] (e2m1 x e4m3/16 x fp32 scale_2 -> 2-bit + UE8M0/32)",
               ms=round(ms, 4), hbm_GBps=round(nbytes / (ms * 1e-3) / 1e9, 1),
               hbm_frac=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
               blocks_per_s=round(blocks / (ms * 1e-3), 1), algorithmic_bytes=nbytes, iters=args.requant_iters)

    def timed(call):
        call()
        ts = []
        for _ in range(args.requant_iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    # FP8 block-quant: e4m3 [n, R, C] + fp32 [n, R/128, C/128]
    e4 = torch.empty((n, R, C), dtype=torch.uint8, device="cuda")
    bs = torch.empty((n, R // 128, C // 128), dtype=torch.float32, device="cuda")
    for i in range(n):
        a, b = workloads.fp8_block_tensor(i, R, C)
        e4[i].copy_(torch.from_numpy(a))
        bs[i].copy_(torch.from_numpy(b))
    ms = timed(lambda: moe.fp8_block128_to_w2(e4, bs, codes, scales))
    nb8 = n * R * (C + C // 4 + C // 32) + 4 * n * (R // 128) * (C // 128)
    out["fp8_block128"] = dict(workload="fp8_block128_to_w2: 256 tensors of [2048, 6144] (e4m3 x fp32 per 128x128 -> "
                                        "2-bit + UE8M0/32)", ms=round(ms, 4),
                               hbm_GBps=round(nb8 / (ms * 1e-3) / 1e9, 1), blocks_per_s=round(blocks / (ms * 1e-3), 1),
                               algorithmic_bytes=nb8)
    del e4, bs
    torch.cuda.empty_cache()
    # MXFP4: e2m1 [n, R, C/2] + UE8M0 [n, R, C/32]
    e2 = torch.empty((n, R, C // 2), dtype=torch.uint8, device="cuda")
    ue = torch.empty((n, R, C // 32), dtype=torch.uint8, device="cuda")
    for i in range(n):
        a, b = workloads.mxfp4_tensor(i, R, C)
        e2[i].copy_(torch.from_numpy(a))
        ue[i].copy_(torch.from_numpy(b))
    ms = timed(lambda: moe.mxfp4_to_w2(e2, ue, codes, scales))
    nb4 = n * R * (C // 2 + C // 32 + C // 4 + C // 32)
    out["mxfp4"] = dict(workload="mxfp4_to_w2: 256 tensors of [2048, 6144] (e2m1 x UE8M0/32 -> 2-bit + UE8M0/32)",
                        ms=round(ms, 4), hbm_GBps=round(nb4 / (ms * 1e-3) / 1e9, 1),
                        blocks_per_s=round(blocks / (ms * 1e-3), 1), algorithmic_bytes=nb4)
    del e2, ue, codes, scales
    torch.cuda.empty_cache()
    return out


def _threads():
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()] + [CPU_WORKERS])


def cpu_baseline(canon, inst, steps=1):
    """The f64 oracle on `steps` bench steps: routing instances 0.. at T = 1, 8 and 32 of the decode
    workload."""
    from oracle import formats, forward

    t0 = time.perf_counter()
    tokens = 0
    for s in range(steps):
        for T in DECODE_TS:
            h = inst[T][s]["host"]
            forward.moe_forward(formats.bf16_bits_to_f64(h["x"]), h["topk_ids"], h["topk_w"], canon["gu_codes"],
                                canon["gu_scales"], canon["dn_codes"], canon["dn_scales"], workers=CPU_WORKERS)
            tokens += T
    dt = time.perf_counter() - t0
    return dict(value=round(tokens / dt, 3), unit="tokens/s", cores=int(_threads()), kind="oracle",
                sample=f"{steps} bench steps: routing instances 0..{steps - 1} at T=1, 8 and 32 of the decode workload "
                       f"({tokens} tokens, every activated expert dequantized in f64), {dt:.1f} s wall; "
                       f"host has {os.cpu_count()} logical CPUs")


def cpu_baseline_prefill(host, gpu_res, stride=4):
    """The f64 oracle on the 8192-token prefill, restricted to whole expert groups: every
    `stride`-th expert in descending group size (so large and small groups alike), all of their
    pairs. Rate = sampled pairs / wall time, reported per token (top_k pairs)."""
    from oracle import formats, forward

    d, pl = host["inst"], host["planes"]
    ids = d["topk_ids"]
    E, top_k = pl["gu_codes"].shape[0], ids.shape[1]
    counts = np.bincount(ids.ravel(), minlength=E)
    experts = np.argsort(-counts, kind="stable")[::stride]
    sel = np.isin(ids, experts)
    tokens = np.nonzero(sel.any(axis=1))[0]
    x = formats.bf16_bits_to_f64(d["x"])
    t0 = time.perf_counter()
    forward.moe_forward(x, np.where(sel, ids, -1).astype(np.int32), d["topk_w"], pl["gu_codes"], pl["gu_scales"],
                        pl["dn_codes"], pl["dn_scales"], tokens=tokens, workers=CPU_WORKERS)
    dt = time.perf_counter() - t0
    pairs = int(sel.sum())
    tps = pairs / top_k / dt
    return dict(value=round(tps, 2), unit="tokens/s", cores=int(_threads()), kind="oracle",
                gpu_over_cpu=round(gpu_res["tokens_per_s"] / tps, 1),
                sample=f"{len(experts)} of {E} experts (every {stride}th by group size), all {pairs} of their pairs "
                       f"({pairs / ids.size:.1%} of the 65,536), {dt:.1f} s wall; tokens/s = pairs/s / top_k")


def cpu_baseline_zipf(planes, workloads, n_inst=1):
    """The f64 oracle on whole Zipf-routed decode batches (T=64, K=6144), routing instances 0.."""
    from oracle import formats, forward

    c = workloads.DECODE_ZIPF
    insts = workloads.zipf_instances(c["T"], n_inst, c["seed"], c["K"], c["E"], c["top_k"])
    t0 = time.perf_counter()
    for d in insts:
        forward.moe_forward(formats.bf16_bits_to_f64(d["x"]), d["topk_ids"], d["topk_w"], planes["gu_codes"],
                            planes["gu_scales"], planes["dn_codes"], planes["dn_scales"], workers=CPU_WORKERS)
    dt = time.perf_counter() - t0
    return dict(value=round(n_inst * c["T"] / dt, 3), unit="tokens/s", cores=int(_threads()), kind="oracle",
                sample=f"routing instances 0..{n_inst - 1} (whole batches of {c['T']} tokens), {dt:.1f} s wall")


def cpu_baseline_requant(workloads, n=32):
    """The exact C re-quantizer oracle (integer SSE, OpenMP over REQUANT_THREADS threads) on the first
    n of the 256 NVFP4 tensors; input generation is outside the timed region."""
    from oracle import requant

    c = workloads.REQUANT
    R, C = c["R"], c["C"]
    tensors = [workloads.nvfp4_tensor(i) for i in range(n)]
    requant.requant_rows(tensors[0][0][:8], tensors[0][1][:8], tensors[0][2], nthreads=REQUANT_THREADS)   # load
    t0 = time.perf_counter()
    for a, b, s2 in tensors:
        requant.requant_rows(a, b, s2, nthreads=REQUANT_THREADS)
    dt = time.perf_counter() - t0
    blocks = n * R * (C // 32)
    nbytes = n * R * (C // 2 + C // 16 + C // 4 + C // 32) + 4 * n
    return dict(value=round(blocks / dt, 1), unit="blocks/s", cores=REQUANT_THREADS, kind="oracle",
                GBps=round(nbytes / dt / 1e9, 3), ms_for_256_tensors=round(dt / n * 256 * 1e3, 1),
                sample=f"the first {n} of the 256 tensors of [{R}, {C}] ({blocks} blocks), {dt:.1f} s wall")


def bench_sweep(args, moe, workloads, torch, dev):
    """moe_w2_codebook_sweep over --sweep-tensors synthetic tensors of [2048, 6144] (the sign-bias
    diagnostic's own workload) and all 1239 candidate codebooks: time per call (synchronous, so
    wall time between event records that bracket it), candidate-block evaluations per second, and
    what the sweep finds: per tensor the least-error symmetric and asymmetric codebooks with their
    relative RMS error and bias, and the bias of {-4,-1,1,4}."""
    c = workloads.SWEEP
    n, R, C = args.sweep_tensors, c["R"], c["C"]
    fam = workloads.codebook_family()
    x = torch.empty((n, R, C), dtype=torch.float32, device="cuda")
    for i in range(n):
        x[i].copy_(torch.from_numpy(workloads.sweep_tensor(i)))
    moe.moe_w2_codebook_sweep(x, fam)        # warm-up (module load, first allocation)
    ts = []
    for _ in range(args.sweep_iters):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        st, mo, best = moe.moe_w2_codebook_sweep(x, fam)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    st, best = st.cpu().numpy(), best.cpu().numpy()
    M = len(fam)
    i_sym = int(np.where((fam == np.array([-4, -1, 1, 4], np.float32)).all(1))[0][0])
    per = []
    for t in range(n):
        bs, ba = int(best[t, 0]), int(best[t, 1])
        per.append(dict(best_sym=fam[bs].tolist(), sym_rel_rms=round(float(st[t, bs, 2]), 5),
                        sym_bias=float(f"{st[t, bs, 3]:.3e}"), best_asym=fam[ba].tolist(),
                        asym_rel_rms=round(float(st[t, ba, 2]), 5), asym_bias=float(f"{st[t, ba, 3]:.3e}"),
                        w2_rel_rms=round(float(st[t, i_sym, 2]), 5), w2_bias=float(f"{st[t, i_sym, 3]:.3e}")))
    ab = np.array([abs(p["asym_bias"]) for p in per])
    sb = np.array([abs(p["sym_bias"]) for p in per])
    blocks = n * R * C // 32
    del x
    torch.cuda.empty_cache()
    return dict(workload=f"moe_w2_codebook_sweep: {n} synthetic tensors of [{R}, {C}] x {M} codebooks "
                         "(4 distinct e2m1 values, max magnitude 3/4/6)",
                ms=round(ms, 2), candidate_blocks_per_s=round(blocks * M / (ms * 1e-3), 1),
                element_exponent_evals_per_s=round(blocks * M * 320 / (ms * 1e-3), 1),
                roofline=dict(bound="alu", achieved=round(blocks * M * 320 * SWEEP_VALU_PER_EVAL / (ms * 1e-3) / 1e12, 2),
                              peak=round(VALU_PEAK_LANE_OPS / 1e12, 2), unit="T VALU lane-ops/s",
                              frac=round(blocks * M * 320 * SWEEP_VALU_PER_EVAL / (ms * 1e-3) / VALU_PEAK_LANE_OPS, 4)),
                median_abs_bias_asym_over_sym=round(float(np.median(ab / np.maximum(sb, 1e-300))), 2),
                asym_bias_negative=int(np.sum([p["asym_bias"] < 0 for p in per])),
                tensors=per, iters=args.sweep_iters)

if __name__ == "__main__":
    main()

