"""Benchmark of the routed-MoE layer on one MI355X.

One step = one call of moe_layer_forward (route, group, gate/up + SwiGLU,
down, shared expert, combine) over one batch of T synthetic tokens on one
layer weight set.  Decode workloads cycle through distinct resident weight
sets (byte copies at distinct addresses) so each step streams its weights
from HBM rather than from the last-level cache.  Steps are replayed from a
captured HIP graph; inputs are resident in HBM before the timed region.

Prints one JSON line.  `value` is tokens/s over the timed steps, with
p10/p50/p90 microseconds per layer over the graph replays.  The `roofline`
object covers the dominant kernel, the gate/up kernel the layer runs (the
decode lowering's gate/up launch, routed and shared experts, for T <= 8 and
for up to 32 rows on aligned shapes; else the expert GEMV up to 64 rows; the
grouped GEMM above): algorithmic bytes
(decode, HBM-bound) or flops (prefill, MFMA-bound) per launch over its
average launch duration, measured with one pair of HIP events around a batch
of back-to-back launches on the launch stream;
`traffic` is the counter-measured HBM bytes per launch from
profiles/traffic_<workload>.json when those counters were taken on the
current kernel sources (null otherwise).  The
`cpu_baseline` object times the CPU oracle on a bounded sample, at the BLAS
thread count and at one thread, and names the host CPU.

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
FP8_PEAK_TFLOPS = 5000.0
GEMV_MAX_ROWS = 64  # calls with more tokens run the tiled grouped GEMM
DECODE_ROWS = 8     # calls with at most this many tokens run the decode lowering
DECODE_MAX_ROWS = 32  # ... and up to this many when every launch has its aligned tile


def decode_lowering(w):
    """Whether moe_layer_forward runs the decode lowering for this workload
    (the library's rule: T <= 8, or T <= 32 with T*k <= 512 when every
    projection has the aligned tile)."""
    if w.T <= DECODE_ROWS:
        return True
    if w.T > DECODE_MAX_ROWS or w.T * w.top_k > 512:
        return False
    fp4 = ("nvfp4", "mxfp4")
    if w.fmt not in fp4 or w.H % 2048 != 0 or w.H > 4096 or w.H % 64 != 0:
        return False
    def down_ok(fmt, K):
        return fmt in fp4 + ("fp8_b128",) and K % 512 == 0 and K <= 4096
    if not down_ok(w.down_fmt or w.fmt, w.I):
        return False
    if w.I_shared:
        if w.shared_fmt not in fp4 + ("fp8_b128",):
            return False
        if not down_ok(w.shared_down_fmt or w.shared_fmt, w.I_shared):
            return False
    return True

# Opt-in lossy activation modes: (C code, arithmetic type, dense MFMA peak of
# the operand pair in TFLOP/s).  An E4M3 x E2M1 pair runs at the FP8 rate.
ACT_MODES = {
    "exact": (0, "bf16", BF16_PEAK_TFLOPS),
    "mxfp8": (1, "fp8e4m3xfp4e2m1", FP8_PEAK_TFLOPS),
    "mxfp4": (2, "fp4e2m1", FP4_PEAK_TFLOPS),
    "fp8_t128": (3, "fp8e4m3", FP8_PEAK_TFLOPS),
}


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
    ap.add_argument("--act-mode", default="exact", choices=list(ACT_MODES),
                    help="activation mode of the expert GEMMs (lossy modes are opt-in levers; "
                         "they apply to the prefill lowering, T > 64)")
    ap.add_argument("--weight-sets", type=int, default=None)
    ap.add_argument("--kernel-launches", type=int, default=192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--pmc-probe", action="store_true",
                    help="for rocprofv3 --pmc runs: a plain copy of known size, then a few "
                         "launches of the dominant kernel; no timing")
    ap.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn the FETCH_SIZE and WRITE_SIZE runs of --pmc-probe into "
                         "profiles/traffic_<workload>.json")
    args = ap.parse_args()
    if args.pmc_summarize:
        pmc_summarize(args.workload, args.act_mode, *args.pmc_summarize)
        return

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
    mode = args.act_mode
    mode_code, mode_dtype, mode_peak = ACT_MODES[mode]
    lossy = mode != "exact" and T > GEMV_MAX_ROWS
    if mode != "exact" and not ((mode in ("mxfp8", "mxfp4") and w.fmt == synth.FMT_MXFP4) or
                                (mode == "fp8_t128" and w.fmt == synth.FMT_FP8)):
        print(f"--act-mode {mode} does not apply to the {w.fmt} routed experts of {w.name}",
              file=sys.stderr)
        sys.exit(2)
    nsets = args.weight_sets or w.weight_sets
    cycled = T <= GEMV_MAX_ROWS  # weight-streaming lowerings cycle the weight sets
    steps = args.steps if args.steps is not None else (
        nsets * 100 if T <= 8 else (nsets * 20 if cycled else 200))
    warmup = args.warmup if args.warmup is not None else (nsets * 10 if cycled else 20)

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
    moe.moe_layer_forward_ex(base.desc, x, T, out, ws, mode_code, dbg_ids=ids)
    torch.cuda.synchronize()
    ids_np = ids.cpu().numpy()
    from oracle import layer as O
    ref_route = O.route(x_bits, L.router_w, L.router_bias, L.top_k, L.renormalize)
    routing_exact = bool(np.array_equal(ids_np, ref_route.ids))
    log(f"[bench] routing matches the oracle: {routing_exact}")

    if args.pmc_probe:
        pmc_probe(moe, torch, dev, L, w, sets, nsets, x, ids, ws, mode_code if lossy else 0)
        return

    # graph of one pass over the weight sets
    def capture(n):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(n):
                moe.moe_layer_forward_ex(sets[i % nsets].desc, x, T, out, ws, mode_code)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(n):
                moe.moe_layer_forward_ex(sets[i % nsets].desc, x, T, out, ws, mode_code)
        return g

    per_graph = nsets if cycled else 1
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
    # one event before the first replay and one after each: the first to the
    # last is the timed region; consecutive pairs give each replay's
    # per-layer time for the percentiles
    nrep, rem_steps = divmod(steps, per_graph)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nrep + 2)]
    evs[0].record()
    for i in range(nrep):
        g_full.replay()
        evs[i + 1].record()
    if rem_steps:
        (g_rem if rem_steps == rem else capture(rem_steps)).replay()
    evs[-1].record()
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1])
    per_layer = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 / per_graph for i in range(nrep))
    pct = {q: round(float(np.percentile(per_layer, q)), 3) for q in (10, 50, 90)} if per_layer else {}
    wall_s = ms / 1e3
    us_per_layer = ms * 1e3 / steps
    tokens_per_s = steps * T / wall_s
    alg_bytes = layer_algorithmic_bytes(L, ids_np, T)
    flops = layer_flops(L, T)
    layer_gbs = alg_bytes / (us_per_layer * 1e-6) / 1e9
    layer_tflops = flops / (us_per_layer * 1e-6) / 1e12
    log(f"[bench] {steps} steps: {us_per_layer:.2f} us/layer, {tokens_per_s:.1f} tokens/s, "
        f"{layer_gbs:.0f} GB/s algorithmic; p10/p50/p90 {pct.get(10)}/{pct.get(50)}/{pct.get(90)} us")

    # ---- dominant kernel: routed gate/up expert kernel, timed per launch ----
    E, k = L.E, L.top_k
    P = T * k
    offsets, p2, act, h = dominant_inputs(moe, torch, dev, L, ids)
    M = args.kernel_launches
    launch_gate_up = dominant_launcher(moe, torch, dev, L, w, x, ids, offsets, p2, act, h, ws,
                                       mode_code if lossy else 0)
    for i in range(min(M, 2 * nsets)):  # warm
        launch_gate_up(sets[i % nsets])
    torch.cuda.synchronize()
    # M launches back to back between one pair of events on the launch stream
    # (the current stream); the average includes the dispatch gap between
    # consecutive launches, which the profiler's per-kernel duration does not.
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(50_000_000)  # let the host queue every launch before the GPU reaches them
    k0.record()
    for i in range(M):
        launch_gate_up(sets[i % nsets])
    k1.record()
    torch.cuda.synchronize()
    k_avg_us = k0.elapsed_time(k1) * 1e3 / M
    active = np.unique(ids_np)
    k_bytes = len(active) * (expert_bytes(L.gate) + expert_bytes(L.up)) + T * L.H * 2 + P * L.I * 2
    dec = decode_lowering(w) and not lossy
    if dec and L.has_shared:
        # the decode gate/up launch computes the shared expert's gate/up too
        k_bytes += expert_bytes(L.sh_gate) + expert_bytes(L.sh_up) + T * L.I_shared * 2
    k_gbs = k_bytes / (k_avg_us * 1e-6) / 1e9
    k_flops = 2 * P * 2 * L.I * L.H
    k_tflops = k_flops / (k_avg_us * 1e-6) / 1e12
    log(f"[bench] gate/up kernel: {k_avg_us:.2f} us avg over {M} back-to-back launches, "
        f"{k_bytes / 1e6:.2f} MB -> {k_gbs:.0f} GB/s, "
        f"{k_tflops:.1f} TFLOP/s")
    if T <= GEMV_MAX_ROWS:
        # weights streamed once per group: bound by HBM
        what = (" (routed and shared gate/up + SwiGLU)" if dec and L.has_shared
                else " (routed gate/up + SwiGLU)")
        roof = {"kernel": dominant_kernel_name(w, mode) + what,
                "bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                "avg_launch_us": round(k_avg_us, 3), "algorithmic_bytes_per_launch": k_bytes}
    elif not lossy:
        # bf16 x bf16 -> fp32 contraction on the matrix cores
        roof = {"kernel": dominant_kernel_name(w, mode) + " (routed gate/up + SwiGLU)",
                "bound": "mfma", "achieved": round(k_tflops, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(k_tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
                "avg_launch_us": round(k_avg_us, 3), "algorithmic_flops_per_launch": k_flops,
                "fp4_peak_frac": round(k_tflops / FP4_PEAK_TFLOPS, 5)}
    else:
        # quantized activations x checkpoint codes on the scaled matrix cores
        roof = {"kernel": dominant_kernel_name(w, mode) + " (routed gate/up + SwiGLU)",
                "bound": "mfma", "achieved": round(k_tflops, 2), "peak": mode_peak,
                "unit": "TFLOP/s", "frac": round(k_tflops / mode_peak, 4), "traffic": None,
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
        "dtype": mode_dtype if lossy else "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "T": T, "H": L.H, "E": L.E, "I": L.I, "top_k": L.top_k,
            "routed_format": w.fmt, "shared": (f"{w.shared_fmt} I={w.I_shared}" if w.I_shared else None),
            "zipf_s": w.zipf_s, "weight_sets": nsets, "global_batch": T, "seq_len": 1,
            "parallelism": "single-gpu", "act_mode": mode if lossy else "exact",
        },
        "us_per_layer": round(us_per_layer, 3),
        "us_per_layer_p10_p50_p90": [pct.get(10), pct.get(50), pct.get(90)],
        "percentiles_over": (f"{nrep} replays of a graph of {per_graph} layer calls "
                             "(per-layer mean within each replay)"),
        "layer_algorithmic_bytes": alg_bytes,
        "layer_hbm_gbs": round(layer_gbs, 1),
        "layer_hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
        "layer_tflops": round(layer_tflops, 3),
        "layer_bf16_mfma_frac": round(layer_tflops / BF16_PEAK_TFLOPS, 5),
        "layer_fp4_mfma_frac": round(layer_tflops / FP4_PEAK_TFLOPS, 5),
        "unique_experts": int(len(active)),
        "routing_matches_oracle": routing_exact,
        "roofline": dict(roof, traffic=load_traffic(w, mode if lossy else "exact")),
    }

    # ---- CPU baseline: the oracle on a bounded sample ----
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, L, x_bits, args.cpu_seconds,
                                              mode if lossy else None)
    print(json.dumps(result), flush=True)


def dominant_inputs(moe, torch, dev, L, ids):
    """Grouping of the routed pairs for standalone launches of the routed
    gate/up kernel (the layer's dominant kernel)."""
    T, k, E = ids.shape[0], L.top_k, L.E
    P = T * k
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    p2 = torch.empty(P, dtype=torch.int32, device=dev)
    q2 = torch.empty(P, dtype=torch.int32, device=dev)
    act = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pws = torch.empty(moe.moe_permute_workspace_size(T, k, E), dtype=torch.uint8, device=dev)
    moe.moe_permute(ids, T, k, E, counts, offsets, p2, q2, act, pws)
    h = torch.empty((P, L.I), dtype=torch.bfloat16, device=dev)
    return offsets, p2, act, h


def dominant_launcher(moe, torch, dev, L, w, x, ids, offsets, p2, act, h, ws, mode_code):
    """A function launching the gate/up kernel the layer runs, on one weight
    set: the decode lowering's (routed and shared experts, on the layer's
    routing), the expert GEMV or grouped GEMM's, or (lossy mode) the
    scaled-MFMA one on x quantized once."""
    T = w.T
    if decode_lowering(w) and mode_code == 0:
        hp = torch.empty((T * L.top_k, L.I), dtype=torch.bfloat16, device=dev)
        hs = (torch.empty((T, L.I_shared), dtype=torch.bfloat16, device=dev)
              if L.has_shared else None)
        return lambda s: moe.moe_decode_gate_up(s.desc, x, T, ids, hp, hs)
    if mode_code == 0:
        return lambda s: moe.moe_expert_gemm(moe.MOE_OP_GATE_UP_SWIGLU, s.desc, 0, offsets, p2,
                                             act, T, x, h, ws)
    H = L.H
    codes = torch.empty((T, H // 2 if mode_code == moe.MOE_ACT_MXFP4 else H), dtype=torch.uint8,
                        device=dev)
    scales = torch.empty((T, 4 * ((H + 127) // 128)), dtype=torch.uint8, device=dev)
    moe.moe_quantize_act(mode_code, x, T, H, codes, scales)
    return lambda s: moe.moe_expert_gemm_q(mode_code, moe.MOE_OP_GATE_UP_SWIGLU, s.desc, 0,
                                           offsets, p2, act, T, codes, scales, h, ws)


PMC_COPY_BYTES = 256 << 20
PMC_COPIES = 4
PMC_LAUNCHES = 8


def pmc_probe(moe, torch, dev, L, w, sets, nsets, x, ids, ws, mode_code):
    """Dispatches for a counter run: PMC_COPIES plain copies of PMC_COPY_BYTES
    (x * 1 into another buffer; the calibration: bytes per counted KiB), then
    PMC_LAUNCHES launches of
    the dominant kernel, cycling weight sets as the timed run does."""
    T = ids.shape[0]
    offsets, p2, act, h = dominant_inputs(moe, torch, dev, L, ids)
    launch_gate_up = dominant_launcher(moe, torch, dev, L, w, x, ids, offsets, p2, act, h, ws,
                                       mode_code)
    src = torch.ones(PMC_COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(PMC_COPIES):  # an elementwise kernel that reads and writes every byte once
        torch.mul(src, 1, out=dst)
    torch.cuda.synchronize()
    for i in range(PMC_LAUNCHES):
        launch_gate_up(sets[(i + 1) % nsets])
    torch.cuda.synchronize()
    log(f"[bench] pmc probe: {PMC_COPIES} copies of {PMC_COPY_BYTES} B, "
        f"{PMC_LAUNCHES} dominant-kernel launches")


def dominant_kernel_name(w, mode="exact"):
    """Template instance of the routed gate/up kernel for the workload."""
    if mode != "exact" and w.T > GEMV_MAX_ROWS:
        # K = H a multiple of 128: the LDS-DMA variant (whole K steps)
        base = "grouped_gemm_qd_kernel" if w.H % 128 == 0 else "grouped_gemm_q_kernel"
        return f"{base}<{ACT_MODES[mode][0]}, 0>"
    codes = {"nvfp4": 1, "mxfp4": 2, "fp8_b128": 3, "mxfp8": 4}
    fmt = codes[w.fmt]
    if decode_lowering(w):
        sfmt = codes[w.shared_fmt] if w.I_shared else 0
        # the register-lean instance when every tile of the launch has an
        # aligned FP4 (routed) / FP4 or FP8 (shared) form
        lean = (w.fmt in ("nvfp4", "mxfp4") and sfmt in (0, 1, 2, 3)
                and w.H % 2048 == 0 and w.H <= 4096)
        return f"decode_gateup_kernel<{fmt}, {sfmt}, {'true' if lean else 'false'}>"
    if w.T <= GEMV_MAX_ROWS:
        base = "expert_gemv_kernel"
    elif w.fmt in ("nvfp4", "mxfp4") and w.H % 64 == 0:
        base = "grouped_gemm_d_kernel"  # FP4 gate/up with whole 64-K steps: the LDS-DMA variant
    else:
        base = "grouped_gemm_kernel"
    return f"{base}<{fmt}, 0>"


def dominant_sources(w, mode="exact"):
    pkg = os.path.join(ROOT, "quantized_moe_expert_02_amd", "csrc")
    files = ["moe_device.cuh", "gemv_core.cuh"]
    T = w.T
    if mode == "exact" and decode_lowering(w):
        files += ["decode.hip"]
    elif T <= GEMV_MAX_ROWS:
        files += ["expert_gemv.hip"]
    else:
        files += ["expert_gemm.hip", "expert_gemm_d.hip"] if mode == "exact" else ["expert_gemm_q.hip"]
    return [os.path.join(pkg, f) for f in files]


def source_hash(w, mode="exact"):
    import hashlib
    hsh = hashlib.sha256()
    for f in dominant_sources(w, mode):
        with open(f, "rb") as fh:
            hsh.update(fh.read())
    return hsh.hexdigest()[:16]


def traffic_path(workload, mode="exact"):
    tag = "" if mode == "exact" else "_" + mode
    return os.path.join(ROOT, "profiles", f"traffic_{workload}{tag}.json")


def load_traffic(w, mode="exact"):
    """Counter-measured HBM bytes per launch of the dominant kernel, if the
    counters were taken on the kernel sources as they are now; else None."""
    p = traffic_path(w.name, mode)
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        t = json.load(fh)
    if t.get("source_hash") != source_hash(w, mode):
        return None
    return t["bytes_per_launch"]


def _pmc_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def pmc_summarize(workload, mode, fetch_dir, write_dir):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the --pmc-probe runs,
    scaled by what the same counter reads for the plain copy (which moves
    PMC_COPY_BYTES each way), averaged over the dominant kernel's launches."""
    w = __import__("synth").WORKLOADS[workload]
    out = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _pmc_rows(d) if r.get("Counter_Name", r.get("Counter-Name")) == name]
        val = lambda r: float(r.get("Counter_Value", r.get("Counter-Value")))  # noqa: E731
        copy = [val(r) for r in rows if "elementwise" in r["Kernel_Name"]
                and "Fill" not in r["Kernel_Name"]]
        kname = dominant_kernel_name(w, mode)
        kern = [val(r) for r in rows if r["Kernel_Name"].startswith("void moe::(anonymous namespace)::" + kname)]
        kern = kern[-PMC_LAUNCHES:]  # the probe's own launches come last
        if not copy or not kern:
            raise SystemExit(f"{name}: no copy or kernel dispatches in {d}")
        kib_copy = sorted(copy)[len(copy) // 2]
        factor = PMC_COPY_BYTES / kib_copy       # bytes per counted KiB
        out[name] = {"copy_kib": kib_copy, "bytes_per_kib": factor,
                     "kernel_kib_avg": sum(kern) / len(kern), "launches": len(kern),
                     "kernel_bytes_avg": factor * sum(kern) / len(kern)}
    res = {"workload": workload, "act_mode": mode, "kernel": dominant_kernel_name(w, mode),
           "source_hash": source_hash(w, mode),
           "bytes_per_launch": round(out["FETCH_SIZE"]["kernel_bytes_avg"]
                                     + out["WRITE_SIZE"]["kernel_bytes_avg"]),
           "fetch": out["FETCH_SIZE"], "write": out["WRITE_SIZE"]}
    with open(traffic_path(workload, mode), "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res))


def cpu_model() -> str:
    """The host CPU's model name with its family / model / stepping numbers
    (some virtualised hosts report only a short name)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if ":" not in line:
                    if fields:
                        break  # first processor only
                    continue
                k, v = (t.strip() for t in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping") and k not in fields:
                    fields[k] = v
    except OSError:  # pragma: no cover
        pass
    if "model name" not in fields:
        import platform
        return platform.processor() or "unknown"
    ids = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields)
    return f"{fields['model name']} ({ids})" if ids else fields["model name"]


def cpu_baseline(w, L, x_bits, budget_s, mode=None):
    """The oracle on the host's cores, at the BLAS library's full thread count
    (the reported value) and again limited to one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    res = _cpu_run(w, L, x_bits, budget_s, mode)
    with threadpool_limits(limits=1):
        one = _cpu_run(w, L, x_bits, budget_s, mode)
    res.update({"cores": int(cores), "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
                "value_1thread": one["value"], "seconds_1thread": one["seconds"],
                "calls_1thread": one["calls"]})
    return res


def _cpu_run(w, L, x_bits, budget_s, mode=None):
    from oracle import layer as O
    from oracle import lossy as Q
    T = x_bits.shape[0]
    if T <= 64:
        tokens = None
        sample = f"full layer calls on the same {T}-token batch and weight set, repeated for ~{budget_s:.0f}s"
        per = T
    else:
        # wide experts decode far more weight per sampled token
        n = 64 if w.H * w.I <= 2048 * 512 else 4
        tokens = list(range(0, T, T // n))[:n]
        sample = f"routing of all {T} tokens plus expert FFNs and combine for {n} sampled tokens"
        per = n
    if mode is not None:
        sample += f", activation mode {mode}"
    t0 = time.time()
    done = 0
    while True:
        if mode is None:
            O.layer_forward(L, x_bits, tokens=tokens)
        else:
            Q.layer_forward(L, x_bits, mode, tokens=tokens)
        done += 1
        el = time.time() - t0
        if el >= budget_s or (tokens is not None):
            break
    return {"value": round(done * per / el, 4), "unit": "tokens/s", "kind": "oracle",
            "sample": sample, "seconds": round(el, 2), "calls": done}


if __name__ == "__main__":
    main()
