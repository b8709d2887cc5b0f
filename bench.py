"""Throughput of the fused MX mixture-of-experts layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one moe_fused call over one batch: top-k routing of the router
logits, permutation by expert, (MXFP8 quantization of x), FC1 + SiLU(gate)*up,
FC2 + routing-weighted combine (+ shared expert) and the bf16 output.  Inputs
and packed weights are synthetic, seeded and resident in HBM before the timed
region starts.  Prints one JSON line with whole-layer tokens/s, the roofline of
the dominant kernel (timed with HIP events on the library's stream), and the
CPU oracle timed on a bounded sample of the same workload.

Default workload: decode_w4a16 (T=64, H=7168, I=2048, E=384 resident MXFP4
experts, top-8, bf16 activations).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Published MI355X peaks (dense, no sparsity).
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp6": 10100.0, "fp4": 10100.0}

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
    "tiny_w4a16": "k_fc_small<true, 1>",
    "decode_w4a16": "k_fc_small<true, 4>",
    "prefill_w4a8": "k_fc_wide<true>",
    "skew_w4a16": "k_fc_mid<true, 128>",
    "w6a8_shared": "k_fc_tiled<true, 2, 128, false>",
}

# Sources of the GEMM kernels: a committed HBM-traffic summary counts only
# while these are unchanged since it was taken.
KERNEL_SOURCES = tuple(f"block_scaled_precision_amd/csrc/{f}" for f in (
    "copy_ring.h", "gemm.h", "gemm_mid.hip", "gemm_small.hip", "gemm_stream.hip", "gemm_tiled.hip", "gemm_wide.hip",
    "internal.h", "mx_device.h", "tiled_count.h", "wide_count.h"))


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_w4a16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-tokens", type=int, default=None,
                    help="tokens of the workload the CPU oracle runs on (default: per workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale HBM counters)")
    return ap.parse_args()


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


def build_inputs(torch, m, gen, w, seed):
    """Logits, x and all packed weights on the GPU (fp32 weights drawn on the
    GPU per expert and quantized by mx_quantize into place)."""
    dev = "cuda"
    bits = m.FORMAT_BITS[w.wfmt]
    logits = gen.router_logits(w, seed, device=dev)
    x = gen.hidden_states(w, seed, device=dev)
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
    return logits, x, mw


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


def cpu_baseline(torch, np, gen, w, seed, logits, x, y_gpu, ntok):
    """Time the CPU oracle on the first `ntok` tokens of the workload and compare
    its output with the GPU's rows for the same tokens."""
    from oracle import moe as om
    from tests.helpers import ExpertArrays, y_error
    import concurrent.futures as cf
    import multiprocessing as mp

    rows = np.arange(ntok)
    lg = logits[:ntok].cpu().numpy()
    from oracle.routing import topk_route
    ids, _ = topk_route(lg, w.k)
    experts = sorted(set(int(e) for e in ids.ravel()))
    # fp32 weights of those experts from the same seeded generator (on the GPU),
    # quantized by the oracle itself (not part of the timed layer)
    mats = []
    for e in experts:
        mats.append(gen.expert_w1(w, e, seed, device="cuda").cpu().numpy())
        mats.append(gen.expert_w2(w, e, seed, device="cuda").cpu().numpy())
    shared = None
    if w.I_shared:
        mats.append(gen.shared_w1(w, seed, device="cuda").cpu().numpy())
        mats.append(gen.shared_w2(w, seed, device="cuda").cpu().numpy())
    nproc = max(1, min(16, len(os.sched_getaffinity(0))))
    with cf.ProcessPoolExecutor(max_workers=nproc, mp_context=mp.get_context("fork")) as ex:
        q = list(ex.map(om.quantize_weight, mats, [w.wfmt] * len(mats)))
    per = {e: (q[2 * i][0], q[2 * i][1], q[2 * i + 1][0], q[2 * i + 1][1]) for i, e in enumerate(experts)}
    if w.I_shared:
        shared = (q[-2][0], q[-2][1], q[-1][0], q[-1][1])
    arrs = tuple(ExpertArrays({e: v[i] for e, v in per.items()}, w.E) for i in range(4))
    xs = x[:ntok].to(torch.float64).cpu().numpy()
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = None
    t0 = time.perf_counter()
    ref = om.moe_forward(xs, lg, *arrs, k=w.k, wfmt=w.wfmt, act=w.act, shared=shared)
    dt = time.perf_counter() - t0
    mr, rr = y_error(y_gpu[:ntok].float().cpu().numpy(), ref["y"])
    ids_ok = bool(np.array_equal(ids, ref["ids"]))
    return ({"value": ntok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
             "sample": f"first {ntok} tokens of {w.name} ({len(experts)} experts decoded), "
                       f"numpy float64, {dt:.1f} s"},
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
    w = gen.WORKLOADS[args.workload]
    print(f"# bench {w.name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.k} {w.wfmt}/{w.act} Is={w.I_shared}",
          file=sys.stderr, flush=True)
    logits, x, mw = build_inputs(torch, m, gen, w, args.seed)
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared)
    ws = torch.empty((max(m.moe_fused_workspace_bytes(prob), 1),), dtype=torch.uint8, device="cuda")
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(events=None):
        m.moe_fused(prob, x, mw, router_logits=logits, y=y, workspace=ws, topk_ids_out=ids,
                    topk_w_out=wts, stream=stream, stage_events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    ns = m.MOE_NUM_STAGES + 1
    K = args.steps
    # the timed steps run without instrumentation (recording the per-stage
    # events costs about 2% of a decode step); a second, untimed pass of K
    # steps records them for the stage breakdown and the FC1 kernel time
    edge = m.HipEvents(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    edge.record(0, stream)
    for i in range(K):
        step()
    edge.record(1, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = edge.elapsed_ms(0, 1) / K
    stage_ev = [m.HipEvents(ns) for _ in range(K)]
    for i in range(K):
        step(stage_ev[i].handles)
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([stage_ev[i].elapsed_ms(s, s + 1) for i in range(K)]))
                for s, name in enumerate(m.STAGES)}
    print(f"# timed {K} steps: {ms_step:.4f} ms/step (wall {1e3 * wall / K:.4f}); stages "
          + " ".join(f"{k}={v:.4f}" for k, v in stage_ms.items()), file=sys.stderr, flush=True)

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
    roof["kernel"] = FC1_KERNEL[w.name]
    roof["kernel_ms"] = stage_ms["fc1"]
    roof["alg_bytes_per_launch"] = work["fc1_bytes"]
    roof["alg_flops_per_launch"] = work["fc1_flops"]
    roof["kernel_source_sha256_16"] = src_hash

    out = {
        "metric": "MoE layer tokens/s", "value": w.T / (ms_step / 1e3), "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16 x mxfp4 (bf16 MFMA, f32 acc)",
                  "mxfp8": f"mxfp8 x {'mxfp4' if w.wfmt == 'e2m1' else 'mxfp6'} (scaled MFMA, f32 acc)"}[w.act],
        "data": "synthetic (seeded N(0,1) logits and x, N(0,0.02) weights quantized on device)",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "I": w.I, "E": w.E, "k": w.k,
                   "weights": w.wfmt, "activations": w.act, "I_shared": w.I_shared},
        "roofline": roof,
        "layer": {"alg_bytes": work["layer_bytes"], "alg_flops": work["layer_flops"],
                  "GB_per_s": work["layer_bytes"] / (ms_step / 1e3) / 1e9,
                  "hbm_frac": work["layer_bytes"] / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS,
                  "TFLOP_per_s": work["layer_flops"] / (ms_step / 1e3) / 1e12,
                  "active_experts": work["active_experts"], "stages_ms": stage_ms},
    }
    if not args.no_cpu_baseline:
        ntok = args.cpu_sample_tokens or {"tiny_w4a16": 16, "decode_w4a16": 8, "prefill_w4a8": 4,
                                          "skew_w4a16": 8, "w6a8_shared": 4}[w.name]
        print(f"# cpu oracle on {ntok} tokens", file=sys.stderr, flush=True)
        cb, par = cpu_baseline(torch, np, gen, w, args.seed, logits, x, y, ntok)
        out["cpu_baseline"] = cb
        out["sampled_parity"] = par
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
