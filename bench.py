"""Benchmark of the routed-MoE layer on one MI355X.

One step = one call of moe_layer_forward (route, group, gate/up + SwiGLU,
down, shared expert, combine) over one batch of T synthetic tokens on one
layer weight set.  Decode workloads cycle through distinct resident weight
sets (byte copies at distinct addresses) so each step streams its weights
from HBM rather than from the last-level cache.  Steps are replayed from a
captured HIP graph; inputs are resident in HBM before the timed region.

Prints one JSON line.  `value` is tokens/s over the timed steps.  The
`roofline` object covers the dominant kernel (the routed gate/up expert
kernel): algorithmic bytes (decode, HBM-bound) or flops (prefill, MFMA-bound)
per launch over its average launch duration, measured with HIP events
bracketing each launch on the launch stream.  The
`cpu_baseline` object times the CPU oracle on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer µs & tokens/s; HBM GB/s %peak (decode T=1-8), MFMA %peak (prefill)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP4_PEAK_TFLOPS = 10100.0
GEMV_MAX_ROWS = 16  # calls with more tokens run the tiled grouped GEMM


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def expert_bytes(q) -> int:
    """Stored bytes of one expert of a projection (codes + scales + tensor scale)."""
    return q.nbytes_per_expert()


def layer_algorithmic_bytes(L, ids, T) -> int:
    """Bytes a layer call must read/write at least: each active expert's three
    projections once, the shared expert, the router, x in and out."""
    active = set(int(e) for e in ids.reshape(-1))
    n = len(active) * (expert_bytes(L.gate) + expert_bytes(L.up) + expert_bytes(L.down))
    if L.has_shared:
        n += expert_bytes(L.sh_gate) + expert_bytes(L.sh_up) + expert_bytes(L.sh_down)
    n += L.router_w.nbytes + (L.router_bias.nbytes if L.router_bias is not None else 0)
    n += 2 * T * L.H * 2
    return n


def layer_flops(L, T) -> int:
    P = T * L.top_k
    f = 2 * P * (2 * L.I * L.H + L.H * L.I)
    if L.has_shared:
        f += 2 * T * 3 * L.I_shared * L.H
    f += 2 * T * L.H * L.E
    return f


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode_t1_nvfp4")
    ap.add_argument("--weight-sets", type=int, default=None)
    ap.add_argument("--kernel-launches", type=int, default=192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(collectives are out of scope); use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import quantized_moe_expert_02_amd as moe
    from quantized_moe_expert_02_amd.device import DeviceLayer, bf16_tensor

    w = synth.WORKLOADS[args.workload]
    T = w.T
    nsets = args.weight_sets or w.weight_sets
    steps = args.steps if args.steps is not None else (nsets * 100 if T <= 8 else 200)
    warmup = args.warmup if args.warmup is not None else (nsets * 10 if T <= 8 else 20)

    t0 = time.time()
    L = synth.make_layer(w)
    x_bits = synth.make_x(w)
    log(f"[bench] generated {w.name} in {time.time() - t0:.1f}s "
        f"({synth.layer_bytes(L) / 1e9:.3f} GB per weight set, {nsets} sets)")

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    base = DeviceLayer(L, dev)
    sets = [base] + [base.copy() for _ in range(nsets - 1)]
    x = bf16_tensor(x_bits, dev)
    out = torch.empty((T, L.H), dtype=torch.bfloat16, device=dev)
    ws = base.workspace(T)
    ids = torch.empty((T, L.top_k), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    # one eager call, checked against the oracle's routing
    moe.moe_layer_forward(base.desc, x, T, out, ws, dbg_ids=ids)
    torch.cuda.synchronize()
    ids_np = ids.cpu().numpy()
    from oracle import layer as O
    ref_route = O.route(x_bits, L.router_w, L.router_bias, L.top_k, L.renormalize)
    routing_exact = bool(np.array_equal(ids_np, ref_route.ids))
    log(f"[bench] routing matches the oracle: {routing_exact}")

    # graph of one pass over the weight sets
    def capture(n):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(n):
                moe.moe_layer_forward(sets[i % nsets].desc, x, T, out, ws)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(n):
                moe.moe_layer_forward(sets[i % nsets].desc, x, T, out, ws)
        return g

    per_graph = nsets if T <= 8 else 1
    g_full = capture(per_graph)
    rem = steps % per_graph
    g_rem = capture(rem) if rem else None

    def run_steps(k):
        for _ in range(k // per_graph):
            g_full.replay()
        if k % per_graph:
            (g_rem if k % per_graph == rem else capture(k % per_graph)).replay()

    run_steps(warmup)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    run_steps(steps)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    wall_s = ms / 1e3
    us_per_layer = ms * 1e3 / steps
    tokens_per_s = steps * T / wall_s
    alg_bytes = layer_algorithmic_bytes(L, ids_np, T)
    flops = layer_flops(L, T)
    layer_gbs = alg_bytes / (us_per_layer * 1e-6) / 1e9
    layer_tflops = flops / (us_per_layer * 1e-6) / 1e12
    log(f"[bench] {steps} steps: {us_per_layer:.2f} us/layer, {tokens_per_s:.1f} tokens/s, "
        f"{layer_gbs:.0f} GB/s algorithmic")

    # ---- dominant kernel: routed gate/up expert kernel, timed per launch ----
    E, k = L.E, L.top_k
    P = T * k
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    p2 = torch.empty(P, dtype=torch.int32, device=dev)
    q2 = torch.empty(P, dtype=torch.int32, device=dev)
    act = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pws = torch.empty(moe.moe_permute_workspace_size(T, k, E), dtype=torch.uint8, device=dev)
    moe.moe_permute(ids, T, k, E, counts, offsets, p2, q2, act, pws)
    h = torch.empty((P, L.I), dtype=torch.bfloat16, device=dev)
    M = args.kernel_launches
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(M)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(M)]
    for i in range(min(M, 2 * nsets)):  # warm
        moe.moe_expert_gemm(moe.MOE_OP_GATE_UP_SWIGLU, sets[i % nsets].desc, 0, offsets, p2, act, T,
                            x, h, ws)
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(50_000_000)  # let the host queue every launch before the GPU reaches them
    for i in range(M):
        starts[i].record()
        moe.moe_expert_gemm(moe.MOE_OP_GATE_UP_SWIGLU, sets[i % nsets].desc, 0, offsets, p2, act, T,
                            x, h, ws)
        ends[i].record()
    torch.cuda.synchronize()
    kt = sorted(s.elapsed_time(e) * 1e3 for s, e in zip(starts, ends))
    k_avg_us = sum(kt) / len(kt)
    active = np.unique(ids_np)
    k_bytes = len(active) * (expert_bytes(L.gate) + expert_bytes(L.up)) + T * L.H * 2 + P * L.I * 2
    k_gbs = k_bytes / (k_avg_us * 1e-6) / 1e9
    k_flops = 2 * P * 2 * L.I * L.H
    k_tflops = k_flops / (k_avg_us * 1e-6) / 1e12
    log(f"[bench] gate/up kernel: {k_avg_us:.2f} us avg over {M} launches "
        f"(median {kt[len(kt) // 2]:.2f}), {k_bytes / 1e6:.2f} MB -> {k_gbs:.0f} GB/s, "
        f"{k_tflops:.1f} TFLOP/s")
    if T <= GEMV_MAX_ROWS:
        # weights streamed once per group: bound by HBM
        roof = {"kernel": "expert_gemv_kernel (routed gate/up + SwiGLU)",
                "bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                "avg_launch_us": round(k_avg_us, 3), "algorithmic_bytes_per_launch": k_bytes}
    else:
        # bf16 x bf16 -> fp32 contraction on the matrix cores
        roof = {"kernel": "grouped_gemm_kernel (routed gate/up + SwiGLU)",
                "bound": "mfma", "achieved": round(k_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(k_tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "avg_launch_us": round(k_avg_us, 3), "algorithmic_flops_per_launch": k_flops,
                "fp4_peak_frac": round(k_tflops / FP4_PEAK_TFLOPS, 5)}

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms / steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "T": T, "H": L.H, "E": L.E, "I": L.I, "top_k": L.top_k,
            "routed_format": w.fmt, "shared": (f"{w.shared_fmt} I={w.I_shared}" if w.I_shared else None),
            "zipf_s": w.zipf_s, "weight_sets": nsets, "global_batch": T, "seq_len": 1,
            "parallelism": "single-gpu",
        },
        "us_per_layer": round(us_per_layer, 3),
        "layer_algorithmic_bytes": alg_bytes,
        "layer_hbm_gbs": round(layer_gbs, 1),
        "layer_hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
        "layer_tflops": round(layer_tflops, 3),
        "layer_bf16_mfma_frac": round(layer_tflops / BF16_PEAK_TFLOPS, 5),
        "layer_fp4_mfma_frac": round(layer_tflops / FP4_PEAK_TFLOPS, 5),
        "unique_experts": int(len(active)),
        "routing_matches_oracle": routing_exact,
        "roofline": roof,
    }

    # ---- CPU baseline: the oracle on a bounded sample ----
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, L, x_bits, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline(w, L, x_bits, budget_s):
    from oracle import layer as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    T = x_bits.shape[0]
    if T <= 64:
        tokens = None
        sample = f"full layer calls on the same {T}-token batch and weight set, repeated for ~{budget_s:.0f}s"
        per = T
    else:
        n = 64
        tokens = list(range(0, T, T // n))[:n]
        sample = f"routing of all {T} tokens plus expert FFNs and combine for {n} sampled tokens"
        per = n
    t0 = time.time()
    done = 0
    while True:
        O.layer_forward(L, x_bits, tokens=tokens)
        done += 1
        el = time.time() - t0
        if el >= budget_s or (tokens is not None):
            break
    return {"value": round(done * per / el, 4), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", "sample": sample, "seconds": round(el, 2), "calls": done}


if __name__ == "__main__":
    main()
