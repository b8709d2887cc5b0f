"""Throughput of the fused MX mixture-of-experts layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]

One step is one moe_fused call over one batch: top-k routing of the router
logits, permutation by expert, (MXFP8 quantization of x), FC1 + SiLU(gate)*up,
FC2 + routing-weighted combine (+ shared expert) and the bf16 output.  Inputs
and packed weights are synthetic, seeded and resident in HBM before the timed
region starts.

By default every workload is timed in this one process (the decode and
prefill workloads share one weight set): W untimed warm-up steps, then K
steps, each bracketed by HIP events on the layer's stream; a workload's time
per step is the median over its K steps.  The printed JSON line is headed by
the decode workload (T=64, H=7168, I=2048, E=384 resident MXFP4 experts,
top-8, bf16 activations); "workloads" holds every workload's line, each with
the roofline of its dominant kernel (FC1, timed with HIP events on the
library's stream in a second pass of K steps).  The CPU oracle is timed on a
bounded sample of the decode workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Published MI355X peaks (dense, no sparsity).
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp6": 10100.0, "fp4": 10100.0}

HEADLINE = "decode_w4a16"
ORDER = ("tiny_w4a16", "decode_w4a16", "prefill_w4a8", "skew_w4a16", "w6a8_shared")

# Which roof bounds each workload's dominant kernel (FC1), and the MFMA rate it
# issues at: MXFP8 x MXFP4/MXFP6 scaled MFMAs run at the FP8 rate, bf16
# activations use the bf16 MFMA after in-register dequantization.
BOUND = {
    "tiny_w4a16": ("hbm", "bf16"),
    "decode_w4a16": ("hbm", "bf16"),
    "prefill_w4a8": ("mfma", "fp8"),
    "skew_w4a16": ("mfma", "bf16"),
    "w6a8_shared": ("hbm", "fp8"),
}
# FC1 kernel that bench times per workload (the dominant kernel of the layer)
FC1_KERNEL = {
    "tiny_w4a16": "k_fc_small_routed<1, 1>",  # 16 tokens: FC1 routes the batch itself
    "decode_w4a16": "k_fc_small<true, 4>",
    "prefill_w4a8": "k_fc_wide<true, 0>",
    "skew_w4a16": "k_fc_mid<true, 128>",
    "w6a8_shared": "k_fc_tiled<true, 2, 128, false>",
}

# Sources of the GEMM kernels: a committed HBM-traffic summary counts only
# while these are unchanged since it was taken.
KERNEL_SOURCES = tuple(f"block_scaled_precision_amd/csrc/{f}" for f in (
    "batch_route.h", "copy_ring.h", "gemm.h", "gemm_mid.hip", "gemm_small.hip", "gemm_stream.hip", "gemm_tiled.hip",
    "gemm_wide.hip", "internal.h", "mx_device.h", "tiled_count.h", "topk_device.h", "wide_count.h"))


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all",
                    help="one workload name, 'all' (default), or 'small_batches' / 'dense_gemm' "
                         "for those parts of the default run alone")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-tokens", type=int, default=16,
                    help="tokens of the decode workload the CPU oracle runs on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale HBM counters)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, src_hash: str):
    """HBM bytes per FC1 launch from the committed rocprofv3 --pmc summary of
    this workload, or None if there is none or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", f"fc1_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != src_hash:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 5}), flush=True)


def build_weights(torch, m, gen, w, seed):
    """All packed weights of a workload on the GPU: fp32 weights drawn on the
    GPU per expert and quantized by mx_quantize into place."""
    dev = "cuda"
    bits = m.FORMAT_BITS[w.wfmt]
    w1 = torch.empty((w.E, 2 * w.I, w.H * bits // 8), dtype=torch.uint8, device=dev)
    s1 = torch.empty((w.E, 2 * w.I, w.H // 32), dtype=torch.uint8, device=dev)
    w2 = torch.empty((w.E, w.H, w.I * bits // 8), dtype=torch.uint8, device=dev)
    s2 = torch.empty((w.E, w.H, w.I // 32), dtype=torch.uint8, device=dev)
    for e in range(w.E):
        m.mx_quantize(gen.expert_w1(w, e, seed, device=dev), w.wfmt, codes=w1[e], scales=s1[e])
        m.mx_quantize(gen.expert_w2(w, e, seed, device=dev), w.wfmt, codes=w2[e], scales=s2[e])
    mw = m.MoeWeights(w1, s1, w2, s2, w.wfmt)
    if w.I_shared:
        mw.ws1, mw.ws1_scale = m.mx_quantize(gen.shared_w1(w, seed, device=dev), w.wfmt)
        mw.ws2, mw.ws2_scale = m.mx_quantize(gen.shared_w2(w, seed, device=dev), w.wfmt)
    torch.cuda.synchronize()
    return mw


def algorithmic_work(w, counts):
    """Bytes and flops the method must move / compute for this routing.

    Per active expert (>= 1 assignment): its packed W1 and W2 plus their E8M0
    scales.  Per call: x (bf16) read once, y (bf16) written once, the fp32
    logits read once, shared-expert weights.  FLOPs: 2*A*(2I)*H + 2*A*H*I
    (+ the shared expert on all T tokens).  The FC1 row gives what the FC1
    kernel alone must move: W1 + scales of active experts, x, and the
    intermediate h it writes (bf16, or E4M3 codes + scales)."""
    b = {"e2m1": 4, "e3m2": 6}[w.wfmt]
    active = int((counts > 0).sum())
    A = w.T * w.k
    w1_e = 2 * w.I * w.H * b / 8 + 2 * w.I * w.H / 32
    w2_e = w.H * w.I * b / 8 + w.H * w.I / 32
    sh1 = 2 * w.I_shared * w.H * b / 8 + 2 * w.I_shared * w.H / 32
    sh2 = w.H * w.I_shared * b / 8 + w.H * w.I_shared / 32
    io = w.T * w.H * 2 * 2 + w.T * w.E * 4
    layer_bytes = active * (w1_e + w2_e) + sh1 + sh2 + io
    flops = 2.0 * A * 2 * w.I * w.H + 2.0 * A * w.H * w.I
    flops += 2.0 * w.T * 2 * w.I_shared * w.H + 2.0 * w.T * w.H * w.I_shared
    h_bytes = A * w.I * (2 if w.act == "bf16" else 1 + 1 / 32)
    fc1_bytes = active * w1_e + w.T * w.H * 2 + h_bytes
    fc1_flops = 2.0 * A * 2 * w.I * w.H
    return dict(active_experts=active, assignments=A, per_expert_w1_bytes=w1_e, per_expert_w2_bytes=w2_e,
                layer_bytes=layer_bytes, layer_flops=flops, fc1_bytes=fc1_bytes, fc1_flops=fc1_flops)


def time_workload(torch, np, m, gen, w, mw, args):
    """Warm up, then K steps each bracketed by HIP events; a second pass of K
    steps records the per-stage events.  Returns the workload's line."""
    seed = args.seed
    logits = gen.router_logits(w, seed, device="cuda")
    x = gen.hidden_states(w, seed, device="cuda")
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared)
    ws = torch.empty((max(m.moe_fused_workspace_bytes(prob), 1),), dtype=torch.uint8, device="cuda")
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    # arguments checked and marshalled once: a step costs the host only the C call
    step = m.FusedCall(prob, x, mw, router_logits=logits, y=y, workspace=ws, topk_ids_out=ids, topk_w_out=wts,
                       stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = m.HipEvents(K + 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(0, stream)
    for i in range(K):
        step()
        ev.record(i + 1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = [ev.elapsed_ms(i, i + 1) for i in range(K)]
    ms_med = statistics.median(per_step)
    ms_mean = ev.elapsed_ms(0, K) / K
    # stage breakdown (events at every stage boundary cost a few us per step)
    ns = m.MOE_NUM_STAGES + 1
    stage_ev = [m.HipEvents(ns) for _ in range(K)]
    for i in range(K):
        step(stage_ev[i].handles)
    torch.cuda.synchronize()
    stage_ms = {name: float(statistics.median([stage_ev[i].elapsed_ms(s, s + 1) for i in range(K)]))
                for s, name in enumerate(m.STAGES)}
    log(f"# {w.name}: {K} steps, median {ms_med:.4f} ms (mean {ms_mean:.4f}, wall {1e3 * wall / K:.4f}); "
        + " ".join(f"{k}={v:.4f}" for k, v in stage_ms.items()))

    counts = torch.bincount(ids.flatten().long(), minlength=w.E).cpu().numpy()
    work = algorithmic_work(w, counts)
    bound, rate = BOUND[w.name]
    fc1_s = stage_ms["fc1"] / 1e3
    src_hash = kernel_source_hash()
    traffic = read_traffic(w.name, src_hash)
    if bound == "hbm":
        achieved = work["fc1_bytes"] / fc1_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic}
    else:
        achieved = work["fc1_flops"] / fc1_s / 1e12
        peak = MFMA_PEAK_TFLOPS[rate]
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": traffic}
    roof.update(kernel=FC1_KERNEL[w.name], kernel_ms=stage_ms["fc1"], alg_bytes_per_launch=work["fc1_bytes"],
                alg_flops_per_launch=work["fc1_flops"], kernel_source_sha256_16=src_hash)
    s = ms_med / 1e3
    layer = {"alg_bytes": work["layer_bytes"], "alg_flops": work["layer_flops"],
             "GB_per_s": work["layer_bytes"] / s / 1e9,
             "hbm_frac": work["layer_bytes"] / s / 1e9 / HBM_PEAK_GBS,
             "TFLOP_per_s": work["layer_flops"] / s / 1e12,
             "active_experts": work["active_experts"], "stages_ms": stage_ms}
    if w.act == "mxfp8":
        # the metric's prefill fraction: whole-layer flops against the dense
        # MX-MFMA peak at the FP8 rate, and against the FP4/FP6 rate
        layer["mfma_frac_fp8_peak"] = layer["TFLOP_per_s"] / MFMA_PEAK_TFLOPS["fp8"]
        layer["mfma_frac_fp4_peak"] = layer["TFLOP_per_s"] / MFMA_PEAK_TFLOPS["fp4"]
    elif bound == "mfma":
        layer["mfma_frac_bf16_peak"] = layer["TFLOP_per_s"] / MFMA_PEAK_TFLOPS["bf16"]
    if w.skew:
        top = np.sort(counts)[::-1]
        layer["expert_histogram"] = {"top10_share": float(top[:10].sum() / counts.sum()),
                                     "largest": top[:5].tolist(),
                                     "empty_experts": np.flatnonzero(counts == 0).tolist()}
    line = {
        "metric": "MoE layer tokens/s", "value": w.T / s, "unit": "tokens/s", "ms_per_step": ms_med,
        "ms_per_step_mean": ms_mean, "steps": K, "warmup": args.warmup,
        "dtype": {"bf16": "bf16 x mxfp4 (bf16 MFMA, f32 acc)",
                  "mxfp8": f"mxfp8 x {'mxfp4' if w.wfmt == 'e2m1' else 'mxfp6'} (scaled MFMA, f32 acc)"}[w.act],
        "config": {"workload": w.name, "T": w.T, "H": w.H, "I": w.I, "E": w.E, "k": w.k,
                   "weights": w.wfmt, "activations": w.act, "I_shared": w.I_shared},
        "roofline": roof, "layer": layer,
    }
    return line, (logits, x, y, ids)


def event_median(torch, m, fn, steps, warmup):
    """Median HIP-event time (ms) of fn() over `steps` calls after `warmup`."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = m.HipEvents(steps + 1)
    ev.record(0, stream)
    for i in range(steps):
        fn()
        ev.record(i + 1, stream)
    torch.cuda.synchronize()
    return statistics.median([ev.elapsed_ms(i, i + 1) for i in range(steps)])


def graph_median(torch, m, fn, steps, warmup):
    """Median HIP-event time (ms) of replays of fn() captured in a HIP graph
    (torch.cuda.graph), and the graph (so that its output can be checked)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up outside the capture
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return event_median(torch, m, g.replay, steps, warmup), g


def small_batches(torch, np, m, gen, mw, args, batches=(1, 2, 4, 8)):
    """The decode shapes (H=7168, I=2048, E=384 resident experts, top-8, bf16
    activations) at batches of 1 to 8 tokens, on the default path and on the
    fused small-batch path: the whole layer per call, eager and as a HIP graph
    replay (no launch gaps from the host), and the packed weights of the
    experts the batch routes to (what the call must stream from HBM) per
    second against the HBM peak."""
    base = gen.WORKLOADS[HEADLINE]
    out = {}
    for T in batches:
        w = gen.scaled(base, T=T)
        logits = gen.router_logits(w, args.seed, device="cuda")
        x = gen.hidden_states(w, args.seed, device="cuda")
        y = torch.empty((T, w.H), dtype=torch.bfloat16, device="cuda")
        ids = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
        row = {}
        for path, fused in (("default", False), ("fused_small_batch", True)):
            prob = m.make_problem(T, w.H, w.I, w.E, w.k, w.wfmt, w.act, fused_small_batch=fused)
            ws = torch.empty((m.moe_fused_workspace_bytes(prob),), dtype=torch.uint8, device="cuda")
            # arguments marshalled once (the stream is the current one at each call,
            # so that the same call can be captured)
            fn = m.FusedCall(prob, x, mw, router_logits=logits, y=y, workspace=ws, topk_ids_out=ids)
            ms = event_median(torch, m, fn, args.steps, args.warmup)
            # host time per call (enqueue only): below the GPU time, the calls
            # queue up and the events time the GPU, not the host
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                fn()
            host_us = (time.perf_counter() - t0) / args.steps * 1e6
            torch.cuda.synchronize()
            y_eager = y.clone()
            ms_graph, g = graph_median(torch, m, fn, args.steps, args.warmup)
            torch.cuda.synchronize()
            if not torch.equal(y.view(torch.int16), y_eager.view(torch.int16)):
                raise RuntimeError(f"graph replay differs from the eager call (T={T}, {path})")
            del g
            counts = torch.bincount(ids.flatten().long(), minlength=w.E).cpu().numpy()
            work = algorithmic_work(w, counts)
            wbytes = work["active_experts"] * (work["per_expert_w1_bytes"] + work["per_expert_w2_bytes"])
            gbs = wbytes / (ms / 1e3) / 1e9
            gbs_g = wbytes / (ms_graph / 1e3) / 1e9
            row[path] = {"ms_per_step": ms, "tokens_per_s": T / (ms / 1e3), "weight_GB_per_s": gbs,
                         "hbm_frac": gbs / HBM_PEAK_GBS, "graph_ms_per_step": ms_graph,
                         "graph_hbm_frac": gbs_g / HBM_PEAK_GBS, "host_us_per_call": host_us}
            log(f"# decode shapes T={T} {path}: {ms * 1e3:.1f} us ({ms_graph * 1e3:.1f} us as a graph replay), "
                f"{work['active_experts']} experts, {gbs:.0f} GB/s of weights ({gbs_g:.0f} replayed); "
                f"host {host_us:.1f} us per call")
        row.update(active_experts=work["active_experts"], weight_bytes=wbytes)
        out[str(T)] = row
    return out


# dense GEMMs timed through mx_gemm: (name, M, N, K, weights, activations, roof)
GEMMS = (
    ("w4a8_8192x4096x7168", 8192, 4096, 7168, "e2m1", "mxfp8", "fp8"),
    ("w6a8_2048x8192x5120", 2048, 8192, 5120, "e3m2", "mxfp8", "fp8"),
    ("w4a16_8x4096x7168", 8, 4096, 7168, "e2m1", "bf16", "hbm"),
)


def dense_gemms(torch, m, gen, args):
    """mx_gemm on dense shapes: the prefill FC1 shape of one expert group as
    one GEMM (W4A8), the shared expert's FC1 (W6A8), and a decode-sized GEMV
    (W4A16, weight-streaming bound).  The activations are quantized inside
    the call when they are MXFP8 (part of the timed work)."""
    out = {}
    for name, M, N, K, fmt, act, roof in GEMMS:
        a = gen.normal((M, K), args.seed, 30, device="cuda").to(torch.bfloat16)
        wq, sq = m.mx_quantize(gen.normal((N, K), args.seed, 31, device="cuda", std=0.02), fmt)
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty((max(m.mx_gemm_workspace_bytes(M, N, K, act, fmt), 1),), dtype=torch.uint8, device="cuda")
        fn = lambda: m.mx_gemm(a, wq, sq, fmt, act, c=c, workspace=ws)  # noqa: E731
        ms = event_median(torch, m, fn, args.steps, args.warmup)
        flops = 2.0 * M * N * K
        wbytes = N * K * m.FORMAT_BITS[fmt] / 8 + N * K / 32
        nbytes = wbytes + M * K * 2 + M * N * 2
        d = {"M": M, "N": N, "K": K, "weights": fmt, "activations": act, "ms": ms,
             "TFLOP_per_s": flops / (ms / 1e3) / 1e12, "GB_per_s": nbytes / (ms / 1e3) / 1e9}
        if roof == "hbm":
            d["roofline"] = {"bound": "hbm", "achieved": d["GB_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": d["GB_per_s"] / HBM_PEAK_GBS}
        else:
            d["roofline"] = {"bound": "mfma", "achieved": d["TFLOP_per_s"], "peak": MFMA_PEAK_TFLOPS[roof],
                             "unit": "TFLOP/s", "frac": d["TFLOP_per_s"] / MFMA_PEAK_TFLOPS[roof]}
        out[name] = d
        log(f"# mx_gemm {name}: {ms * 1e3:.1f} us, {d['TFLOP_per_s']:.0f} TFLOP/s, {d['GB_per_s']:.0f} GB/s")
        del a, wq, sq, c, ws
    torch.cuda.empty_cache()
    return out


def cpu_baseline(torch, np, gen, w, seed, logits, x, y_gpu, ntok):
    """Time the CPU oracle (numpy float64, as it stands) on the first `ntok`
    tokens of the workload and compare its output with the GPU's rows.  The
    oracle's own weight quantization is input preparation, done beforehand in
    a pool of fresh ("spawn") worker processes and not timed."""
    from oracle import moe as om
    from oracle.routing import topk_route
    from tests.helpers import ExpertArrays, oracle_weights, pool_workers, shutdown_pool, y_error

    lg = logits[:ntok].cpu().numpy()
    ids, _ = topk_route(lg, w.k)
    experts = sorted(set(int(e) for e in ids.ravel()))
    t0 = time.perf_counter()
    ow = oracle_weights(w, seed, experts, fp32_on="cuda")
    prep = time.perf_counter() - t0
    shutdown_pool()
    arrs = tuple(ExpertArrays({e: ow[e][i] for e in experts}, w.E) for i in range(4))
    xs = x[:ntok].to(torch.float64).cpu().numpy()
    blas = {}
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = {"library": info[0].get("internal_api"), "version": info[0].get("version"),
                    "threads": info[0].get("num_threads")}
    except Exception:
        pass
    cpu_model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    ref = om.moe_forward(xs, lg, *arrs, k=w.k, wfmt=w.wfmt, act=w.act)
    dt = time.perf_counter() - t0
    mr, rr = y_error(y_gpu[:ntok].float().cpu().numpy(), ref["y"])
    ids_ok = bool(np.array_equal(ids, ref["ids"]))
    return ({"value": ntok / dt, "unit": "tokens/s", "cores": blas.get("threads") or 1, "kind": "oracle",
             "sample": f"first {ntok} of the {w.T} tokens of {w.name} ({len(experts)} of its active experts "
                       f"decoded), numpy float64 in one process: {dt:.1f} s (weight quantization by the "
                       f"oracle beforehand, {prep:.0f} s in {pool_workers()} worker processes, not timed)",
             "affinity_cores": affinity, "cpu_model": cpu_model, "blas": blas},
            {"tokens": ntok, "max_rel": mr, "rms_rel": rr, "ids_equal": ids_ok})


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library runs the "
              "layer on one GPU, an expert shard per call, and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from block_scaled_precision_amd import inputs as gen
    from block_scaled_precision_amd import moe_mx as m

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.workload == "small_batches":
        w = gen.WORKLOADS[HEADLINE]
        mw = build_weights(torch, m, gen, w, args.seed)
        print(json.dumps({"small_batches": small_batches(torch, np, m, gen, mw, args)}), flush=True)
        return
    if args.workload == "dense_gemm":
        print(json.dumps({"dense_gemm": dense_gemms(torch, m, gen, args)}), flush=True)
        return
    names = ORDER if args.workload == "all" else (args.workload,)
    head = HEADLINE if HEADLINE in names else names[0]
    lines = {}
    keep = {}
    weights = {}
    for name in names:
        w = gen.WORKLOADS[name]
        key = (w.H, w.I, w.E, w.wfmt, w.I_shared)
        if key not in weights:
            log(f"# weights for {name}: E={w.E} H={w.H} I={w.I} {w.wfmt} I_shared={w.I_shared}")
            weights[key] = build_weights(torch, m, gen, w, args.seed)
        log(f"# bench {name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.k} {w.wfmt}/{w.act} Is={w.I_shared}")
        lines[name], tensors = time_workload(torch, np, m, gen, w, weights[key], args)
        if name == head:
            keep = tensors
            if args.workload == "all":
                small = small_batches(torch, np, m, gen, weights[key], args)
        # free what later workloads do not share
        later = {(gen.WORKLOADS[n].H, gen.WORKLOADS[n].I, gen.WORKLOADS[n].E, gen.WORKLOADS[n].wfmt,
                  gen.WORKLOADS[n].I_shared) for n in names[names.index(name) + 1:]}
        if key not in later:
            del weights[key]
            torch.cuda.empty_cache()

    h = lines[head]
    out = {"metric": "MoE layer tokens/s", "value": h["value"], "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": h["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": h["dtype"],
           "data": "synthetic (seeded N(0,1) logits and x, N(0,0.02) weights quantized on device)",
           "config": h["config"], "roofline": h["roofline"], "layer": h["layer"],
           "ms_per_step_mean": h["ms_per_step_mean"],
           "timing": "per workload: median over the timed steps of HIP-event time per moe_fused call"}
    if len(names) > 1:
        out["workloads"] = lines
    if args.workload == "all":
        out["small_batches"] = small
        out["dense_gemm"] = dense_gemms(torch, m, gen, args)
    if not args.no_cpu_baseline and head == HEADLINE:
        w = gen.WORKLOADS[head]
        logits, x, y, _ = keep
        ntok = min(args.cpu_sample_tokens, w.T)
        log(f"# cpu oracle on {ntok} tokens of {head}")
        cb, par = cpu_baseline(torch, np, gen, w, args.seed, logits, x, y, ntok)
        out["cpu_baseline"] = cb
        out["sampled_parity"] = par
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
