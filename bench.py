"""Benchmark of the routed-expert MoE FFN layer on one MI355X.

Default workload: one decode MoE layer at batch 1 (d_model 2816, 128 routed
experts, top-8, expert d_ff 704, shared d_ff 2112, int4 group-64 experts,
int8 router with a Zipf logit bias), one token per call, tokens iid N(0, 1)
in bf16, already resident in HBM.  A step is one batch-1 forward of the whole
layer (router GEMV, softmax top-K, shared + routed gate/up SiLU, down +
weighted combine).  Prints one JSON line.

  python bench.py [--gpus 1] [--steps 1000] [--warmup 50] [--no-cpu]
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
PROFILE_DIR = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("decode.hip", "device.hpp", "kernels.hpp", "layout.hpp"):
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


def cpu_baseline(w, arrays, n_tokens: int):
    """The fp64 oracle, timed on this host's cores over a bounded sample."""
    from gen.workloads import make_tokens
    from oracle import oracle as O
    OL = O.OracleLayer.from_workload(w, arrays)
    x = make_tokens(w, n_tokens, stream=4242)
    OL.forward(x[:1])  # warm (page in, thread pool)
    t0 = time.perf_counter()
    for t in range(n_tokens):
        OL.forward(x[t:t + 1])
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tok/s", "cores": O.threads(), "kind": "oracle",
            "sample": f"{n_tokens} batch-1 tokens of the same layer (fp64 plain loops, "
                      f"OpenMP over output rows), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-tokens", type=int, default=48)
    ap.add_argument("--mode", choices=("graph", "direct"), default="graph",
                    help="graph: the timed tokens are replayed from HIP graphs captured in chunks "
                         "(no host launch cost); direct: one library call per token")
    ap.add_argument("--chunk", type=int, default=100, help="tokens per captured graph")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 256 MiB device copy first (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(no collectives, no sharding); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))

    import numpy as np
    import torch
    import routed_expert_ffn_int8_amd as M
    from gen.workloads import WORKLOADS, make_layer, make_tokens, matrix_bytes, router_bytes

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = WORKLOADS[1]
    arrays = make_layer(w)
    desc, keep = M.make_desc(arrays, w.d, w.E, w.K, w.f, w.fs, M.MOE_ACT_BF16, 1)
    layer = M.moe_layer_create(desc)
    del keep

    n = args.steps + args.warmup
    x_host = make_tokens(w, n, stream=1)
    x = torch.from_numpy(x_host.view(np.int16)).view(torch.bfloat16).cuda()
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        M.moe_layer_forward(x[i], layer, out[i], 1, stream)
    torch.cuda.synchronize()

    graphs = []
    if args.mode == "graph":
        # the timed tokens (each a full batch-1 forward with its own input and
        # output row) are captured into HIP graphs and replayed
        cap = torch.cuda.Stream()
        for c0 in range(args.warmup, n, args.chunk):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for i in range(c0, min(n, c0 + args.chunk)):
                    M.moe_layer_forward(x[i], layer, out[i], 1, cap)
            graphs.append(g)
        torch.cuda.synchronize()
        for g in graphs:  # first replays upload the graphs
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.warmup, n):
            M.moe_layer_forward(x[i], layer, out[i], 1, stream)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0

    # Per-kernel durations: HIP events around every kernel on the launch
    # stream, over the same tokens launched directly.  Each chunk waits behind
    # a short bounded spin on that stream so the host has enqueued the whole
    # chunk before its first kernel starts: the events then time kernels that
    # run back to back, not host launch latency.
    M.moe_layer_profile(layer, True)
    gated_ms = 0.0
    for c0 in range(args.warmup, n, args.chunk):
        torch.cuda._sleep(20_000_000)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(c0, min(n, c0 + args.chunk)):
            M.moe_layer_forward(x[i], layer, out[i], 1, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        gated_ms += e0.elapsed_time(e1)
    prof = M.moe_layer_profile_read(layer)
    M.moe_layer_profile(layer, False)

    tok_s = args.steps / dt
    ms_step = dt * 1e3 / args.steps
    gu, dn = matrix_bytes(w.f, w.d), matrix_bytes(w.d, w.f)
    sgu, sdn = matrix_bytes(w.fs, w.d), matrix_bytes(w.d, w.fs)
    act = 2 * w.d
    alg = {  # algorithmic HBM bytes per launch (weights streamed + token in/out)
        "route_shared": router_bytes(w) + 2 * sgu + act,
        "routed_gate_up": w.K * 2 * gu + act,
        "down_combine": w.K * dn + sdn + act,
    }
    kernels = {}
    for k, (launches, ms) in prof.items():
        avg_us = ms * 1e3 / launches
        kernels[k] = {"launches": launches, "avg_us": round(avg_us, 3),
                      "alg_bytes": alg.get(k), "gbps": round(alg[k] / (avg_us * 1e3), 1) if k in alg else None}
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches"])
    achieved = kernels[dom]["gbps"]
    workload = "decode_layer"
    roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": read_traffic(dom, workload),
                "kernel": dom}
    bytes_token = w.K * (2 * gu + dn) + 2 * sgu + sdn + router_bytes(w)
    result = {
        "metric": "MoE FFN tok/s (decode b=1, one layer, int4 g64 experts, int8 router)",
        "value": round(tok_s, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode-layer-d2816-e128-k8-f704-fs2112-b1",
                   "tokens_per_call": 1, "d_model": w.d, "experts": w.E, "top_k": w.K,
                   "d_ff": w.f, "d_ff_shared": w.fs, "weights": "int4 affine g64, int8 router"},
        "mode": args.mode,
        "direct_launch_gpu_tok_s": round(args.steps / (gated_ms / 1e3), 1),
        "layer_hbm_gbps": round(bytes_token * tok_s / 1e9, 1),
        "bytes_per_token": bytes_token,
        "roofline": roofline,
        "kernels": kernels,
    }
    M.moe_layer_destroy(layer)
    if rank == 0 and not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, arrays, args.cpu_tokens)
    if rank == 0:
        print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
