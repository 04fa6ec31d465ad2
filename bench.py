"""Benchmarks of the routed-expert MoE FFN layer on one MI355X.

Default (--workload decode): one decode MoE layer at batch 1 (d_model 2816,
128 routed experts, top-8, expert d_ff 704, shared d_ff 2112, int4 group-64
experts, int8 router with a Zipf logit bias), one token per call, tokens iid
N(0, 1) in bf16, already resident in HBM.  A step is one batch-1 forward of
the whole layer (router GEMV, softmax top-K, shared + routed gate/up SiLU,
down + weighted combine).  The timed steps are replayed from HIP graphs; the
per-kernel durations come from extended-launch HIP events in a second pass
over the same tokens.  Prints one JSON line, which also carries a short
prefill summary (128-token chunk of the d_model 2048 / 256-expert layer) and
a short leg of the 30-layer decode stack (32 steps of its recurrence).

Other workloads (one JSON line each):
  --workload prefill : 128-token chunks, d_model 2048, 256 experts, top-8,
                       d_ff 512, shared 512 (also 512 / 2048 tokens as chunks)
  --workload stack   : 30 decode layers of the default shape, 256 steps,
                       h <- h + MoE(rmsnorm(h)), next input = output + N(0, 0.1)
  --workload stream  : 40 layers of the prefill shape, routed experts in
                       pinned host memory behind a 16-slot LFU cache per layer,
                       Zipf s = 1.1 and 60% reuse of the previous step's experts,
                       256 steps, next to the same stack with all experts in HBM

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--workload ...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense MFMA
PROFILE_DIR = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("decode.hip", "prefill.hip", "device.hpp", "kernels.hpp", "layout.hpp", "topk.hpp"):
        with open(os.path.join(ROOT, "routed_expert_ffn_int8_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None
    if there is none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^\s*([a-z_0-9]+)\s*[:=]\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, arrays, n_tokens: int, tokens_per_call: int = 1, n_single: int = 0):
    """The fp64 oracle, timed on this host's cores over a bounded sample: once
    with its OpenMP loops on every core, and once on a single core."""
    from gen.workloads import make_tokens
    from oracle import oracle as O
    OL = O.OracleLayer.from_workload(w, arrays)
    x = make_tokens(w, n_tokens, stream=4242)
    OL.forward(x[:1])  # warm (page in, thread pool)

    def timed(n):
        t0 = time.perf_counter()
        for t in range(0, n, tokens_per_call):
            OL.forward(x[t:t + tokens_per_call])
        return time.perf_counter() - t0

    cores = O.threads()
    dt = timed(n_tokens)
    res = {"value": round(n_tokens / dt, 3), "unit": "tok/s", "cores": cores, "kind": "oracle",
           "sample": f"{n_tokens} tokens of the same layer in calls of {tokens_per_call} "
                     f"(fp64 plain loops, OpenMP over output rows), {dt:.1f} s",
           "cpu_model": cpu_model(), "nproc": os.cpu_count()}
    if n_single:
        O.set_threads(1)
        try:
            dt1 = timed(n_single)
        finally:
            O.set_threads(cores)
        res["single_thread"] = {"value": round(n_single / dt1, 4), "unit": "tok/s", "cores": 1,
                                "sample": f"{n_single} tokens, {dt1:.1f} s"}
    return res


def kernel_table(prof: dict, alg: dict, flops: dict | None = None) -> dict:
    out = {}
    for k, (launches, ms) in prof.items():
        avg_us = ms * 1e3 / launches
        e = {"launches": launches, "avg_us": round(avg_us, 3)}
        if k in alg:
            e["alg_bytes"] = int(alg[k])
            e["gbps"] = round(alg[k] / (avg_us * 1e3), 1)
        if flops and k in flops:
            e["tflops"] = round(flops[k] / (avg_us * 1e6), 2)
        out[k] = e
    return out


def gated_profile(M, torch, layer, calls, stream, chunk):
    """Per-kernel durations (extended-launch HIP events) over `calls`, each
    chunk enqueued behind a short bounded spin on the stream."""
    M.moe_layer_profile(layer, True)
    gpu_ms = 0.0
    for c0 in range(0, len(calls), chunk):
        torch.cuda._sleep(20_000_000)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for fn in calls[c0:c0 + chunk]:
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        gpu_ms += e0.elapsed_time(e1)
    prof = M.moe_layer_profile_read(layer)
    M.moe_layer_profile(layer, False)
    return prof, gpu_ms


def graph_time(torch, calls, chunk):
    """Capture `calls` into graphs of `chunk` calls, replay once to upload,
    then time one replay of every graph.  Returns seconds."""
    cap = torch.cuda.Stream()
    graphs = []
    for c0 in range(0, len(calls), chunk):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for fn in calls[c0:c0 + chunk]:
                fn(cap)
        graphs.append(g)
    torch.cuda.synchronize()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


# --------------------------------------------------------------------- decode
def run_decode(args, M, torch, np):
    from gen.workloads import WORKLOADS, make_layer, make_tokens, matrix_bytes, router_bytes
    w = WORKLOADS[1]
    arrays = make_layer(w)
    desc, keep = M.make_desc(arrays, w.d, w.E, w.K, w.f, w.fs, M.MOE_ACT_BF16, 1)
    layer = M.moe_layer_create(desc)
    del keep
    n = args.steps + args.warmup
    x = torch.from_numpy(make_tokens(w, n, stream=1).view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    timed = range(args.warmup, n)

    def fwd(path):
        def call(i, s):
            M.moe_layer_forward_ex(x[i], layer, out[i], 1, M.fwd_opts(path=path), s)
        return call

    def measure(path):
        call = fwd(path)
        for i in range(args.warmup):
            call(i, stream)
        torch.cuda.synchronize()
        if args.mode == "graph":
            dt = graph_time(torch, [lambda s, i=i: call(i, s) for i in timed], args.chunk)
        else:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in timed:
                call(i, stream)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
        prof, gated_ms = gated_profile(M, torch, layer, [lambda i=i: call(i, stream) for i in timed], stream,
                                       args.chunk)
        return dt, prof, gated_ms

    gu, dn = matrix_bytes(w.f, w.d), matrix_bytes(w.d, w.f)
    sgu, sdn = matrix_bytes(w.fs, w.d), matrix_bytes(w.d, w.fs)
    act = 2 * w.d
    alg = {"route_shared": router_bytes(w) + 2 * sgu + act,
           "routed_gate_up": w.K * 2 * gu + act,
           "down_combine": w.K * dn + sdn + act,
           "fused_layer": router_bytes(w) + 2 * sgu + sdn + w.K * (2 * gu + dn) + 2 * act}
    # the split (three-kernel) path first, for context; then the production path
    dt3, prof3, _ = measure(M.MOE_PATH_DECODE)
    path = M.MOE_PATH_FUSED if args.decode_path == "fused" else M.MOE_PATH_DECODE
    dt, prof, gated_ms = measure(path)
    tok_s = args.steps / dt
    kernels = kernel_table(prof, alg)
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches"])
    achieved = kernels[dom]["gbps"]
    # Cold: a 512 MB device copy before every token evicts the 256 MB
    # Infinity Cache; the layer's own kernel events time each token, so the
    # copies are outside the measurement.
    cold = None
    if not args.no_extra:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        call = fwd(path)
        M.moe_layer_profile(layer, True)
        for i in list(timed)[:200]:
            dst.copy_(src)
            call(i, stream)
        torch.cuda.synchronize()
        pc = kernel_table(M.moe_layer_profile_read(layer), alg)
        M.moe_layer_profile(layer, False)
        del src, dst
        tot_us = sum(v["avg_us"] for v in pc.values())
        cold_bytes = w.K * (2 * gu + dn) + 2 * sgu + sdn + router_bytes(w)
        cold = {"tokens": min(200, args.steps), "flush": "512 MB device copy before each token",
                "kernel_us_per_token": round(tot_us, 3), "hbm_gbps": round(cold_bytes / (tot_us * 1e3), 1),
                "kernels": pc}
    bytes_token = w.K * (2 * gu + dn) + 2 * sgu + sdn + router_bytes(w)
    # sticky kernel error flags over every pass above (0: every output valid)
    flags = M.moe_layer_check_errors(layer)
    result = {
        "metric": "MoE FFN tok/s (decode b=1, one layer, int4 g64 experts, int8 router)",
        "value": round(tok_s, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode-layer-d2816-e128-k8-f704-fs2112-b1", "tokens_per_call": 1,
                   "d_model": w.d, "experts": w.E, "top_k": w.K, "d_ff": w.f, "d_ff_shared": w.fs,
                   "weights": "int4 affine g64, int8 router"},
        "mode": args.mode,
        "direct_launch_gpu_tok_s": round(args.steps / (gated_ms / 1e3), 1),
        "layer_hbm_gbps": round(bytes_token * tok_s / 1e9, 1),
        "layer_hbm_frac": round(bytes_token * tok_s / 1e9 / PEAK_HBM_GBPS, 4),
        "bytes_per_token": bytes_token,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": read_traffic(dom, "decode_layer"),
                     "kernel": dom},
        "decode_path": args.decode_path,
        "kernels": kernels,
        "three_kernel_path": {"tok_s": round(args.steps / dt3, 1), "kernels": kernel_table(prof3, alg)},
        "cold": cold,
        "error_flags": flags,
    }
    M.moe_layer_destroy(layer)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, arrays, args.cpu_tokens, n_single=args.cpu_single_tokens)
    return result


# --------------------------------------------------------------------- prefill
def run_prefill(args, M, torch, np, chunks=None, summary=False):
    from gen.workloads import WORKLOADS, make_layer, make_tokens, matrix_bytes, router_bytes
    w = WORKLOADS[3]
    arrays = make_layer(w)
    desc, keep = M.make_desc(arrays, w.d, w.E, w.K, w.f, w.fs, M.MOE_ACT_BF16, 2048)
    layer = M.moe_layer_create(desc)
    del keep
    C = 128
    nch = chunks or (8 if summary else 40)
    x = torch.from_numpy(make_tokens(w, C * nch, stream=3).view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.empty_like(x)
    ids = torch.empty((C * nch, w.K), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src

    def call(i, s):
        o = M.fwd_opts(topk_ids=ids[i * C:(i + 1) * C], path=M.MOE_PATH_PREFILL)
        M.moe_layer_forward_ex(x[i * C:(i + 1) * C], layer, out[i * C:(i + 1) * C], C, o, s)

    for i in range(min(nch, 3)):
        call(i, stream)
    torch.cuda.synchronize()
    dt = graph_time(torch, [lambda s, i=i: call(i, s) for i in range(nch)], 10)
    prof, _ = gated_profile(M, torch, layer, [lambda i=i: call(i, stream) for i in range(nch)], stream, 10)
    ids_h = ids.cpu().numpy()
    distinct = float(np.mean([len(np.unique(ids_h[i * C:(i + 1) * C])) for i in range(nch)]))
    eb = 2 * matrix_bytes(w.f, w.d) + matrix_bytes(w.d, w.f)
    gu_b, dn_b = 2 * matrix_bytes(w.f, w.d), matrix_bytes(w.d, w.f)
    sgu, sdn = 2 * matrix_bytes(w.fs, w.d), matrix_bytes(w.d, w.fs)
    chunk_bytes = distinct * eb + sgu + sdn + router_bytes(w)
    flop_routed = C * w.K * (2 * 2 * w.d * w.f + 2 * w.f * w.d)
    flop_shared = C * (2 * 2 * w.d * w.fs + 2 * w.fs * w.d)
    flop_router = C * 2 * w.d * w.E
    flops = flop_routed + flop_shared + flop_router
    alg = {"prefill_gate_up": distinct * gu_b + sgu + C * w.d * 2,
           "prefill_down": distinct * dn_b + sdn,
           "route_shared": router_bytes(w) + C * w.d * 2}
    kflops = {"prefill_gate_up": C * w.K * 2 * 2 * w.d * w.f + C * 2 * 2 * w.d * w.fs,
              "prefill_down": C * w.K * 2 * w.f * w.d + C * 2 * w.fs * w.d}
    kernels = kernel_table(prof, alg, kflops)
    chunk_s = dt / nch
    dom = max(("prefill_gate_up", "prefill_down"), key=lambda k: kernels[k]["avg_us"])
    res = {
        "metric": "MoE FFN prefill tok/s (128-token chunks, one layer) and MFMA utilisation",
        "value": round(C / chunk_s, 1),
        "unit": "tok/s",
        "n_gpus": 1, "steps": nch, "warmup": 3, "ms_per_step": round(chunk_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill-chunk128-d2048-e256-k8-f512-fs512", "tokens_per_call": C},
        "chunk_gflop": round(flops / 1e9, 3),
        "mfma_util": round(flops / chunk_s / 1e12 / PEAK_BF16_TFLOPS, 5),
        "tflops": round(flops / chunk_s / 1e12, 2),
        "distinct_experts_per_chunk": round(distinct, 1),
        "hbm_gbps_distinct_expert_bytes": round(chunk_bytes / chunk_s / 1e9, 1),
        "hbm_frac": round(chunk_bytes / chunk_s / 1e9 / PEAK_HBM_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": kernels[dom]["gbps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(kernels[dom]["gbps"] / PEAK_HBM_GBPS, 4),
                     "traffic": read_traffic(dom, "prefill_chunk"), "kernel": dom},
        "kernels": kernels,
    }
    if not summary and not args.no_extra:
        # Dense routing: every token forced to experts 0..K-1, so each expert
        # tile is full and only K + 1 experts are read (~460 flop/B, past the
        # bf16 ridge): the GEMMs' own compute efficiency.
        forced = torch.arange(w.K, dtype=torch.int32, device="cuda").repeat(C, 1).contiguous()

        def dense(i, s):
            o = M.fwd_opts(forced_ids=forced, path=M.MOE_PATH_PREFILL)
            M.moe_layer_forward_ex(x[i * C:(i + 1) * C], layer, out[i * C:(i + 1) * C], C, o, s)

        dense(0, stream)
        torch.cuda.synchronize()
        ddt = graph_time(torch, [lambda s, i=i: dense(i, s) for i in range(nch)], 10) / nch
        dprof, _ = gated_profile(M, torch, layer, [lambda i=i: dense(i, stream) for i in range(nch)], stream, 10)
        dk = kernel_table(dprof, {}, kflops)
        res["dense_routing"] = {
            "what": "all tokens forced to experts 0..7 (full 16-token tiles, 9 experts read)",
            "ms_per_chunk": round(ddt * 1e3, 4), "tflops": round(flops / ddt / 1e12, 2),
            "mfma_util": round(flops / ddt / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernels": {k: dk[k] for k in ("prefill_gate_up", "prefill_down") if k in dk}}
        # The shared expert at T = 128 is one 128-row dense GEMM; in the dense
        # case every launched expert has that shape (9 x 128 rows, d_ff 512),
        # so the launches' utilisation is the shared expert's.
        res["shared_expert_T128"] = {
            "from": "dense-routing launches: 9 experts of 128 rows, the shared expert one of them",
            **{k + "_mfma_util": round(dk[k]["tflops"] / PEAK_BF16_TFLOPS, 4)
               for k in ("prefill_gate_up", "prefill_down") if k in dk and "tflops" in dk[k]}}
        for T in (512, 2048):  # longer prompts as sequential 128-token chunks inside one call
            if T > C * nch:
                continue
            xt = x[:T]
            ot = torch.empty_like(xt)
            M.moe_layer_forward_ex(xt, layer, ot, T, M.fwd_opts(path=M.MOE_PATH_PREFILL), stream)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(3):
                M.moe_layer_forward_ex(xt, layer, ot, T, M.fwd_opts(path=M.MOE_PATH_PREFILL), stream)
            torch.cuda.synchronize()
            res[f"tok_s_T{T}"] = round(3 * T / (time.perf_counter() - t0), 1)
        if not args.no_cpu:
            res["cpu_baseline"] = cpu_baseline(w, arrays, 32, tokens_per_call=32)
    M.moe_layer_destroy(layer)
    return res


# --------------------------------------------------------------------- stack
def run_stack(args, M, torch, np, steps=None):
    from gen.workloads import WORKLOADS, make_layer, make_tokens, make_noise, matrix_bytes, router_bytes
    w = WORKLOADS[2]
    layers = []
    for l in range(w.layers):
        arrays = make_layer(w, layer=l)
        desc, keep = M.make_desc(arrays, w.d, w.E, w.K, w.f, w.fs, M.MOE_ACT_BF16, 1)
        layers.append(M.moe_layer_create(desc))
        del keep, arrays
        print(f"[bench] stack layer {l + 1}/{w.layers} created", file=sys.stderr, flush=True)
    stack = M.moe_stack_create(layers, 1e-6)
    steps = steps or w.steps
    noise = torch.from_numpy(make_noise(w, steps)).cuda()
    h0 = torch.from_numpy(make_tokens(w, 1, stream=5).view(np.int16)).view(torch.bfloat16).cuda()
    h = h0.clone()
    stream = torch.cuda.current_stream()

    def step(t, s):
        M.moe_stack_forward(h, stack, 1, stream=s)
        with torch.cuda.stream(s):
            h.copy_((h.float() + noise[t]).to(torch.bfloat16))

    for t in range(4):
        step(t, stream)
    torch.cuda.synchronize()
    h.copy_(h0)
    dt = graph_time(torch, [lambda s, t=t: step(t, s) for t in range(steps)], 32)
    finite = bool(torch.isfinite(h.float()).all())
    # per-layer kernel durations (HIP events on each launch) over the same
    # steps, launched directly: their share of the graph-timed step is what
    # the launch gaps and the per-step noise update leave
    for L in layers:
        M.moe_layer_profile(L, True)
    h.copy_(h0)
    for t in range(steps):
        step(t, stream)
    torch.cuda.synchronize()
    kern_ms, kern_n = 0.0, 0
    for L in layers:
        for _, (n, ms) in M.moe_layer_profile_read(L).items():
            kern_ms += ms
            kern_n += n
        M.moe_layer_profile(L, False)
    flags = 0
    for L in layers:
        flags |= M.moe_layer_check_errors(L)
    per_layer = w.K * (2 * matrix_bytes(w.f, w.d) + matrix_bytes(w.d, w.f)) + \
        2 * matrix_bytes(w.fs, w.d) + matrix_bytes(w.d, w.fs) + router_bytes(w)
    bytes_step = per_layer * w.layers
    res = {
        "metric": "MoE FFN stack tok/s (decode b=1, 30 layers, h <- h + MoE(rmsnorm(h)))",
        "value": round(steps / dt, 1), "unit": "tok/s", "n_gpus": 1, "steps": steps, "warmup": 4,
        "ms_per_step": round(dt * 1e3 / steps, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode-stack30-d2816-e128-k8-f704-fs2112-b1", "layers": w.layers},
        "stack_hbm_gbps": round(bytes_step * steps / dt / 1e9, 1),
        "stack_hbm_frac": round(bytes_step * steps / dt / 1e9 / PEAK_HBM_GBPS, 4),
        "bytes_per_token": bytes_step, "finite": finite,
        "layer_kernel_us": round(kern_ms * 1e3 / max(1, kern_n), 3),
        "kernel_share_of_step": round(kern_ms / steps / (dt * 1e3 / steps), 4),
        "error_flags": flags,
    }
    M.moe_stack_destroy(stack)
    for L in layers:
        M.moe_layer_destroy(L)
    return res


# --------------------------------------------------------------------- stream
def run_stream(args, M, torch, np):
    from gen.workloads import WORKLOADS, make_layer, make_tokens, make_noise, make_reuse_coins
    w = WORKLOADS[4]
    res_layers, st_layers = [], []
    for l in range(w.layers):
        arrays = make_layer(w, layer=l)
        d1, k1 = M.make_desc(arrays, w.d, w.E, w.K, w.f, w.fs, M.MOE_ACT_BF16, 1)
        res_layers.append(M.moe_layer_create(d1))
        d2, k2 = M.make_desc(arrays, w.d, w.E, w.K, w.f, w.fs, M.MOE_ACT_BF16, 1, M.MOE_STREAMED)
        L = M.moe_layer_create(d2)
        M.moe_cache_attach(L, w.slots)
        st_layers.append(L)
        del k1, k2, arrays
        print(f"[bench] stream layer {l + 1}/{w.layers} created", file=sys.stderr, flush=True)
    steps = w.steps
    coins = make_reuse_coins(w, steps).astype(np.uint8)
    noise = torch.from_numpy(make_noise(w, steps)).cuda()
    h0 = torch.from_numpy(make_tokens(w, 1, stream=6).view(np.int16)).view(torch.bfloat16).cuda()
    out = {}
    finals = {}
    _, eb = M.moe_layer_bytes(st_layers[0])
    pool = None

    def to_pool():  # the same layers, one LRU cache of the same total bytes
        nonlocal pool
        for L in st_layers:
            M.moe_cache_detach(L)
        pool = M.moe_cache_pool_create(w.layers * w.slots * eb, eb)
        for L in st_layers:
            M.moe_cache_attach_pool(L, pool)

    # resident on its fastest path; then resident on the streamed layers' path
    # (the split kernels), which the streamed runs must match bit for bit;
    # then streamed with 16 LFU slots per layer, then with one shared LRU pool
    for name, layers, path in (("resident", res_layers, M.MOE_PATH_AUTO),
                               ("resident_split", res_layers, M.MOE_PATH_DECODE),
                               ("streamed", st_layers, M.MOE_PATH_AUTO),
                               ("streamed_lru", st_layers, M.MOE_PATH_AUTO)):
        if name == "streamed_lru":
            lfu_stats = [M.moe_cache_stats_get(L) for L in st_layers]
            to_pool()
        for L in layers:
            M.moe_layer_set_default_path(L, path)
        stack = M.moe_stack_create(layers, 1e-6)
        if layers is res_layers:  # untimed warm-up (the streamed runs start from empty caches on purpose),
            # long enough for the GPU's clocks to leave the idle state of layer creation: the first
            # timed run was otherwise up to 3x slow on the fused kernel
            hw = h0.clone()
            t_end, t = time.perf_counter() + 0.5, 0
            while t < 8 or time.perf_counter() < t_end:
                M.moe_stack_forward(hw, stack, 1, reuse_mask=coins[t % steps])
                t += 1
                if t % 16 == 0:
                    torch.cuda.synchronize()
            torch.cuda.synchronize()
        h = h0.clone()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(steps):
            M.moe_stack_forward(h, stack, 1, reuse_mask=coins[t])
            h.copy_((h.float() + noise[t]).to(torch.bfloat16))
        torch.cuda.synchronize()
        out[name] = steps / (time.perf_counter() - t0)
        print(f"[bench] {name}: {out[name]:.1f} tok/s", file=sys.stderr, flush=True)
        finals[name] = h.clone()
        M.moe_stack_destroy(stack)
    tot = {k: sum(s[k] for s in lfu_stats) for k in lfu_stats[0]}
    lru = M.moe_cache_pool_stats(pool)
    # A harder trace for the two policies: a fresh N(0, 1) token every step
    # (no recurrence), same reuse coins, both caches starting empty.
    xs = torch.from_numpy(make_tokens(w, steps, stream=7).view(np.int16)).view(torch.bfloat16).cuda()
    hard = {}
    for name in ("lfu", "lfu_prefetch8", "lru"):
        for L in st_layers:
            M.moe_cache_detach(L)
        if name.startswith("lfu"):
            for L in st_layers:
                M.moe_cache_attach(L, w.slots)
        else:
            M.moe_cache_pool_destroy(pool)
            pool = M.moe_cache_pool_create(w.layers * w.slots * eb, eb)
            for L in st_layers:
                M.moe_cache_attach_pool(L, pool)
        stack = M.moe_stack_create(st_layers, 1e-6)
        if name == "lfu_prefetch8":  # fetch the next layer's 8 most chosen absent experts ahead
            M.moe_stack_set_prefetch(stack, 8)
        h = xs[0:1].clone()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(steps):
            h.copy_(xs[t:t + 1])
            M.moe_stack_forward(h, stack, 1, reuse_mask=coins[t])
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        M.moe_stack_destroy(stack)
        if name.startswith("lfu"):
            ss = [M.moe_cache_stats_get(L) for L in st_layers]
            st = {k: sum(s[k] for s in ss) for k in ss[0]}
        else:
            st = M.moe_cache_pool_stats(pool)
        hard[name] = {"tok_s": round(steps / dt, 2), "hit_rate": round(st["hits"] / max(1, st["accesses"]), 4),
                      "misses_per_token": st["misses"] / steps,
                      "h2d_mb_per_token": round(st["h2d_bytes"] / steps / 1e6, 2)}
        if st["prefetches"]:
            hard[name]["prefetches_per_token"] = st["prefetches"] / steps
            hard[name]["prefetch_used_frac"] = round(st["prefetch_used"] / st["prefetches"], 4)
        print(f"[bench] independent tokens, {name}: {hard[name]}", file=sys.stderr, flush=True)
    res = {
        "metric": "MoE FFN expert-streaming stack tok/s (decode b=1, 40 layers, 16-slot LFU per layer)",
        "value": round(out["streamed"], 2), "unit": "tok/s", "n_gpus": 1, "steps": steps, "warmup": 0,
        "ms_per_step": round(1e3 / out["streamed"], 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "stream-stack40-d2048-e256-k8-f512-lfu16-zipf1.1-reuse0.6"},
        "all_resident_tok_s": round(out["resident"], 1),
        "all_resident_split_path_tok_s": round(out["resident_split"], 1),
        "hit_rate": round(tot["hits"] / max(1, tot["accesses"]), 4),
        "h2d_bytes_per_token": tot["h2d_bytes"] / steps,
        "h2d_gbps_during_fills": round(tot["h2d_bytes"] / max(1, tot["h2d_ns"]), 2),
        "misses_per_token": tot["misses"] / steps,
        # one-token calls compute their hits in kernels queued before the cache
        # step (the device expert table marks them), the misses after the fill
        "slots_computed_ahead_frac": round(tot["ahead_slots"] / (steps * w.layers * w.K), 4),
        "fill_ms_per_token": round(tot["h2d_ns"] / steps / 1e6, 4),
        # step time above the resident layers on the same kernels: the host
        # hand-off of every layer plus the fill time not overlapped
        "exposed_ms_per_token": round(1e3 / out["streamed"] - 1e3 / out["resident_split"], 4),
        "streamed_equals_resident_same_path": bool(torch.equal(finals["resident_split"], finals["streamed"])),
        "lru_shared_pool": {
            "policy": "one LRU cache over (layer, expert), budget = 40 x 16 expert slots",
            "tok_s": round(out["streamed_lru"], 2),
            "hit_rate": round(lru["hits"] / max(1, lru["accesses"]), 4),
            "misses_per_token": lru["misses"] / steps,
            "h2d_bytes_per_token": lru["h2d_bytes"] / steps,
            "equals_resident_same_path": bool(torch.equal(finals["resident_split"], finals["streamed_lru"])),
        },
        "independent_tokens_lfu_vs_lru": hard,  # also LFU with fetch-ahead
    }
    M.moe_cache_pool_destroy(pool)
    for L in res_layers + st_layers:
        M.moe_layer_destroy(L)
    res["prefill_through_cache"] = run_stream_prefill(M, torch, np, w)
    return res


def run_stream_prefill(M, torch, np, w, nch=4):
    """Prefill (128-token chunks) of one streaming-shape layer whose experts
    live in host memory: each chunk's experts go through the 16-slot LFU cache
    in groups; against the same layer resident in HBM."""
    from gen.workloads import make_layer, make_tokens
    arrays = make_layer(w, layer=0)
    d1, k1 = M.make_desc(arrays, w.d, w.E, w.K, w.f, w.fs, M.MOE_ACT_BF16, 128)
    d2, k2 = M.make_desc(arrays, w.d, w.E, w.K, w.f, w.fs, M.MOE_ACT_BF16, 128, M.MOE_STREAMED)
    res_l, st_l = M.moe_layer_create(d1), M.moe_layer_create(d2)
    del k1, k2, arrays
    M.moe_cache_attach(st_l, w.slots)
    x = torch.from_numpy(make_tokens(w, 128 * nch, stream=8).view(np.int16)).view(torch.bfloat16).cuda()
    outs = {}
    times = {}
    for name, L in (("resident", res_l), ("streamed", st_l)):
        out = torch.empty_like(x)
        M.moe_layer_forward_ex(x[:128], L, out[:128], 128, M.fwd_opts(path=M.MOE_PATH_PREFILL))  # warm-up
        torch.cuda.synchronize()
        if name == "streamed":
            M.moe_cache_reset(L, 1)  # the timed chunks start from an empty cache and zero counts
        t0 = time.perf_counter()
        for i in range(nch):
            M.moe_layer_forward_ex(x[i * 128:(i + 1) * 128], L, out[i * 128:(i + 1) * 128], 128,
                                   M.fwd_opts(path=M.MOE_PATH_PREFILL))
        torch.cuda.synchronize()
        times[name] = (time.perf_counter() - t0) / nch
        outs[name] = out
    st = M.moe_cache_stats_get(st_l)
    r = {"chunks": nch, "ms_per_chunk": round(times["streamed"] * 1e3, 3),
         "tok_s": round(128 / times["streamed"], 1), "resident_ms_per_chunk": round(times["resident"] * 1e3, 4),
         "misses_per_chunk": st["misses"] / nch, "hits_per_chunk": st["hits"] / nch,
         "h2d_mb_per_chunk": round(st["h2d_bytes"] / nch / 1e6, 1),
         "h2d_gbps": round(st["h2d_bytes"] / nch / times["streamed"] / 1e9, 2),
         "equals_resident": bool(torch.equal(outs["resident"], outs["streamed"]))}
    print(f"[bench] prefill through the cache: {r}", file=sys.stderr, flush=True)
    M.moe_layer_destroy(res_l)
    M.moe_layer_destroy(st_l)
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", choices=("decode", "prefill", "stack", "stream"), default="decode")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="decode: without the prefill summary; prefill: without the dense-routing run")
    ap.add_argument("--cpu-tokens", type=int, default=160, help="oracle tokens on every core")
    ap.add_argument("--cpu-single-tokens", type=int, default=6, help="oracle tokens on one core")
    ap.add_argument("--stack-steps", type=int, default=32, help="steps of the 30-layer stack leg (default line)")
    ap.add_argument("--decode-path", choices=("fused", "split"), default="fused",
                    help="fused: one kernel per layer and token; split: router+shared | routed gate/up | down")
    ap.add_argument("--mode", choices=("graph", "direct"), default="graph",
                    help="graph: timed decode tokens replayed from HIP graphs; direct: one call per token")
    ap.add_argument("--chunk", type=int, default=100, help="decode tokens per captured graph")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 256 MiB device copy first (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(no collectives, no sharding); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))

    import numpy as np
    import torch
    import routed_expert_ffn_int8_amd as M

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.workload == "decode":
        result = run_decode(args, M, torch, np)
        if not args.no_extra:
            p = run_prefill(args, M, torch, np, summary=True)
            result["prefill_128"] = {k: p[k] for k in ("value", "unit", "ms_per_step", "mfma_util", "tflops",
                                                       "hbm_gbps_distinct_expert_bytes", "hbm_frac",
                                                       "distinct_experts_per_chunk")}
            st = run_stack(args, M, torch, np, steps=args.stack_steps)
            result["stack30"] = {k: st[k] for k in ("value", "unit", "steps", "ms_per_step", "stack_hbm_gbps",
                                                    "stack_hbm_frac", "layer_kernel_us", "kernel_share_of_step",
                                                    "finite", "error_flags", "config")}
    elif args.workload == "prefill":
        result = run_prefill(args, M, torch, np)
    elif args.workload == "stack":
        result = run_stack(args, M, torch, np)
    else:
        result = run_stream(args, M, torch, np)
    if rank == 0:
        print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
