"""Throughput of the DeepSeekMoE layer forward pass on one MI355X.

One step = one full layer forward (router, dispatch, grouped expert GEMMs,
combine) over the 16B-shaped workload: T=16384 tokens, d=2048, 64 routed
experts (inner 1408, top-6, softmax gate) + 2 shared experts, bf16 with an
fp32 router, seeded synthetic inputs resident in HBM before timing starts.

Prints one JSON line with tokens/s, activated TFLOP/s and the fraction of
the bf16 matrix peak, per-stage times from HIP events recorded on the
layer's stream during the timed steps, a roofline entry for the dominant
kernel, the FP8 variant of the same layer (E4M3 expert GEMMs, its own
stage times and roofline against the fp8 matrix peak), the layer backward on
the same workload (stage times, matrix TFLOP/s, the roofline of its slowest
GEMM stage), the other layer shapes (2B-shaped: tokens/s and fraction of the
bf16 peak; V3-shaped: per-call median against the HBM roofline; the skewed
128-token batch: the same with a cold cache), and the CPU oracle timed on a
bounded token sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("MoE layer fwd tokens/s + activated TFLOP/s (% bf16 MFMA peak), "
          "16B-shape, 1 GPU")
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 matrix peak (TFLOP/s)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (GB/s)
PEAK_FP8_TFLOPS = 5033.2       # MI355X dense fp8 matrix peak (TFLOP/s)
DOMINANT = "gemm_gateup"
# The dominant kernel of each variant: (name prefix in a trace, sources,
# committed traffic summary).
GATEUP = {
    "bf16": ("gemm_bf16_kernel<0", ("common.h", "gemm_common.h", "gemm_bf16.hip"),
             os.path.join(ROOT, "profiles", "traffic_gemm_gateup_16b.json")),
    "fp8": ("gemm_fp8_kernel<0", ("common.h", "gemm_common.h", "gemm_fp8.hip"),
            os.path.join(ROOT, "profiles", "traffic_gemm_fp8_gateup_16b.json")),
    # the backward's two slowest GEMM stages (either can be the longer one):
    # the recomputed routed gate/up with the SwiGLU backward, routed dW1/dW3
    "bwd_gateup": ("gemm_bf16_kernel<3", ("common.h", "gemm_common.h", "gemm_bf16.hip"),
                   os.path.join(ROOT, "profiles", "traffic_gemm_gateup_bwd_16b.json")),
    "bwd_dw13": ("gemm_bwd_kernel<3, false>", ("common.h", "gemm_common.h", "gemm_bwd.hip"),
                 os.path.join(ROOT, "profiles", "traffic_gemm_bwd_dw13_routed_16b.json")),
}
# The backward stages whose launch a committed traffic summary covers.
BWD_TRAFFIC = {"gateup_bwd_routed": "bwd_gateup", "dw13_routed": "bwd_dw13"}


def gateup_flops(cfg) -> float:
    """FLOPs of the gate/up launch: 2 d (2 inner) per routed (token, slot) and
    2 d (2 K_s I_s) per token for the shared experts."""
    return 2.0 * cfg.d * 2 * (cfg.T * cfg.top_k * cfg.inner +
                              cfg.T * cfg.n_shared * cfg.shared_inner)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(kind: str = "bf16") -> str:
    """Hash of a dominant kernel's sources (its file and the headers it uses)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_layer_mk_amd", "csrc")
    for f in GATEUP[kind][1]:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kind: str = "bf16"):
    """HBM bytes per launch of a dominant kernel from the committed rocprofv3
    counter summary, or None if absent or taken on other sources."""
    path = GATEUP[kind][2]
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(kind):
        return None
    return t.get("bytes_per_launch")


def summarize_traffic(fetch_csv, write_csv, copy_mb):
    """Write the traffic summaries of the dominant kernels (the gate/up launch
    of the bf16 and of the FP8 forward; the backward's routed gate/up and
    routed dW1/dW3 launches) from two rocprofv3 --pmc counter files
    (FETCH_SIZE run, WRITE_SIZE run, both of a bench run with
    --copy-calibration-mb copy_mb).  Each counter is scaled by what it reads
    for the plain device copy of copy_mb MiB; of the launches of a kernel the
    one with the largest grid is the one summarised (the forward gate/up
    launch holds the routed and shared tiles; the backward's routed launches
    are larger than its shared ones)."""
    import csv
    import collections

    def per_kernel(path, counter):
        acc = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                acc[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    vals = {"fetch": per_kernel(fetch_csv, "FETCH_SIZE"),
            "write": per_kernel(write_csv, "WRITE_SIZE")}
    whats = {"bwd_gateup": "routed gate/up + SwiGLU backward launch",
             "bwd_dw13": "routed dW1/dW3 launch"}
    for kind, (prefix, _, path) in GATEUP.items():
        what = whats.get(kind, "gate/up launch (routed + shared)")
        out = {"source_hash": source_hash(kind), "kernel": prefix.rstrip(">") + ">, " + what,
               "copy_calibration_mib": copy_mb}
        for name in ("fetch", "write"):
            v_all = vals[name]
            copy = [v for (k, g), v in v_all.items() if "copyBuffer" in k]
            gemm = [(g, v) for (k, g), v in v_all.items() if prefix in k]
            if not copy or not gemm:
                print(f"{kind}: copy or gate/up kernel missing in the {name} counters",
                      file=sys.stderr)
                break
            scale = (copy_mb * 1024.0) / max(copy)            # KiB per counter KiB
            g, v = max(gemm)
            out[f"{name}_kib_raw"] = v
            out[f"{name}_scale"] = scale
            out[f"{name}_bytes"] = v * scale * 1024.0
        else:
            out["bytes_per_launch"] = out["fetch_bytes"] + out["write_bytes"]
            os.makedirs(os.path.dirname(path), exist_ok=True)
            with open(path, "w") as f:
                json.dump(out, f, indent=1)
            print(json.dumps(out))


def cpu_baseline(cfg, host, n_tokens, reps):
    """Time the fp64 CPU oracle on the first n_tokens tokens, reps times."""
    import numpy as np
    import threadpoolctl
    import oracle
    w = [t.float().numpy() for t in host["routed"]]
    ws = [t.float().numpy() for t in host["shared"]] if host["shared"] is not None else None
    x = host["x"][:n_tokens].float().numpy()
    wg = host["w_gate"].numpy()
    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info] or [1])
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.moe_forward(x, wg, tuple(w), tuple(ws) if ws else None, cfg.top_k,
                           n_shared=cfg.n_shared, score=cfg.score)
    dt = time.perf_counter() - t0
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    fpt = oracle.expert_flops_per_token(cfg.d, cfg.top_k, cfg.inner, cfg.n_shared,
                                        cfg.shared_inner) + 2 * cfg.d * cfg.n_routed
    return {"value": n_tokens * reps / dt, "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", "seconds": round(dt, 3), "cpu_model": model,
            "gflops": round(fpt * n_tokens * reps / dt / 1e9, 1),
            "sample": f"{reps} x the first {n_tokens} of {cfg.T} tokens of the same workload "
                      f"(numpy fp64 oracle, BLAS threads={cores})"}


def per_call_ms(step, reps, cold_cache, dev):
    """Each of ``reps`` calls timed alone between two events on the current
    stream; with ``cold_cache`` a 1 GiB buffer is overwritten (untimed) before
    every call, evicting the weights from L2 and the 256 MB MALL."""
    import torch
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if cold_cache else None
    out = []
    for _ in range(reps):
        if scratch is not None:
            scratch.fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        e1.synchronize()
        out.append(e0.elapsed_time(e1))
    return out


def layer_hbm_bytes(cfg, counts):
    """Algorithmic HBM bytes of one forward: the weights of every routed expert
    that receives a token and of the shared experts, x read, out written and
    the fp32 gate read."""
    b = 2
    nonempty = int((counts > 0).sum())
    w = 3 * cfg.d * (nonempty * cfg.inner + cfg.n_shared * cfg.shared_inner) * b
    return w + 2 * cfg.T * cfg.d * b + cfg.n_routed * cfg.d * 4, nonempty


def time_fp8(moe, cfg, d, steps, warmup, fpt):
    """The FP8 variant of the same layer (E4M3 expert GEMMs with power-of-two
    block scales): weights quantised once beforehand (the layer's weight
    format), then ``steps`` timed forwards, stage times from HIP events."""
    import torch
    q = {k: [moe.quantize_fp8_blocks(w) for w in d[k]] for k in ("routed", "shared")}
    codes = {k: tuple(c for c, _ in v) for k, v in q.items()}
    scales = {k: tuple(s for _, s in v) for k, v in q.items()}
    desc = moe.make_desc(cfg.T, cfg.d, cfg.n_routed, cfg.top_k, cfg.inner,
                         cfg.n_shared, cfg.shared_inner, n_groups=cfg.n_groups,
                         topk_groups=cfg.topk_groups, score=cfg.score,
                         norm_topk=cfg.norm_topk, routed_scale=cfg.routed_scale,
                         dtype="fp8")
    ws = torch.empty(moe.workspace_size(desc), dtype=torch.uint8, device=d["x"].device)
    out = torch.empty_like(d["x"])
    names = moe.trace_stage_names()
    nst = len(names)
    events = [moe.HipEvents(nst + 1) for _ in range(steps)]

    def step(ev=None):
        moe.moe_layer_forward(d["x"], d["w_gate"], codes["routed"], codes["shared"], cfg.top_k,
                              score=cfg.score, norm_topk=cfg.norm_topk,
                              n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                              select_bias=d["select_bias"], logit_bias=d["logit_bias"],
                              routed_scale=cfg.routed_scale, out=out, workspace=ws,
                              expert_scales=scales["routed"], shared_scales=scales["shared"],
                              trace_events=None if ev is None else ev.handles)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    for i in range(steps):   # stage breakdown: a traced pass (stages in order)
        step(events[i])
    torch.cuda.synchronize()
    stage_ms = {n: sum(ev.elapsed_ms(i, i + 1) for ev in events) / steps
                for i, n in enumerate(names)}
    for ev in events:
        ev.close()
    tflops = fpt * cfg.T / (ms / 1e3) / 1e12
    dom_flops = gateup_flops(cfg)
    dom_ms = stage_ms[DOMINANT]
    achieved = dom_flops / (dom_ms / 1e3) / 1e12
    return {
        "ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.T / (ms / 1e3), 1),
        "activated_tflops": round(tflops, 1),
        "frac_fp8_peak": round(tflops / PEAK_FP8_TFLOPS, 4),
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "roofline": {"kernel": "gemm_fp8_kernel<GATEUP> (routed + shared launch)",
                     "bound": "mfma",
                     "achieved": round(achieved, 1), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "traffic": measured_traffic("fp8"), "flops_per_launch": dom_flops,
                     "avg_launch_ms": round(dom_ms, 4)},
        "recipe": "E4M3 codes; token rows and SwiGLU activations per 1x128, weights per "
                  "128x128 block, power-of-two scales; fp32 accumulation across instructions",
    }


# The other layer shapes, reported beside the headline (key: workload, timing).
OTHER_SHAPES = (
    ("deepseekmoe_2b", "deepseekmoe-2b", False),       # MFMA-bound, back-to-back steps
    ("deepseek_v3", "deepseek-v3", False),             # weight streaming, warm calls
    ("skewed_16b_small", "skewed-16b-small", True),    # weight streaming, cold cache
)


def time_shape(moe, cfg, dev, steps, warmup, reps, cold_cache):
    """One more workload: back-to-back steps (tokens/s, activated TFLOP/s and
    its fraction of the bf16 peak) and calls timed one by one (median; with
    ``cold_cache`` L2 and MALL are flushed before each), with the whole layer
    against the HBM roofline (weights of the experts that receive tokens)."""
    import numpy as np
    import torch
    import oracle
    import workloads
    log(f"[bench] {cfg.name}: generating")
    host = workloads.make_inputs(cfg).torch_tensors("cpu")
    d = {k: (tuple(t.to(dev) for t in v) if isinstance(v, tuple)
             else (v.to(dev) if v is not None else None)) for k, v in host.items()}
    del host
    desc = moe.make_desc(cfg.T, cfg.d, cfg.n_routed, cfg.top_k, cfg.inner,
                         cfg.n_shared, cfg.shared_inner, n_groups=cfg.n_groups,
                         topk_groups=cfg.topk_groups, score=cfg.score,
                         norm_topk=cfg.norm_topk, routed_scale=cfg.routed_scale,
                         dtype=cfg.dtype)
    ws = torch.empty(moe.workspace_size(desc), dtype=torch.uint8, device=dev)
    out = torch.empty_like(d["x"])
    counts = torch.empty(cfg.n_routed, dtype=torch.int32, device=dev)

    def step(routing=False):
        return moe.moe_layer_forward(
            d["x"], d["w_gate"], d["routed"], d["shared"], cfg.top_k, score=cfg.score,
            norm_topk=cfg.norm_topk, n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
            select_bias=d["select_bias"], logit_bias=d["logit_bias"],
            routed_scale=cfg.routed_scale, out=out, workspace=ws, return_routing=routing)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name}: timing")
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    _, rt = step(routing=True)
    counts = rt["expert_counts"].cpu().numpy()
    calls = per_call_ms(step, reps, cold_cache, dev)
    med = float(np.median(calls))
    hbm, nonempty = layer_hbm_bytes(cfg, counts)
    fpt = oracle.expert_flops_per_token(cfg.d, cfg.top_k, cfg.inner, cfg.n_shared,
                                        cfg.shared_inner)
    tfl = fpt * cfg.T / (ms / 1e3) / 1e12
    res = {"workload": f"T={cfg.T}, d={cfg.d}, {cfg.n_routed} routed (inner {cfg.inner}, "
                       f"top-{cfg.top_k}) + {cfg.n_shared} shared",
           "ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.T / (ms / 1e3), 1),
           "activated_tflops": round(tfl, 1),
           "frac_bf16_peak": round(tfl / PEAK_BF16_TFLOPS, 4),
           "per_call_median_ms": round(med, 4), "cold_cache": bool(cold_cache),
           "hbm_roofline": {"bytes": hbm, "nonempty_experts": nonempty,
                            "achieved_gbs": round(hbm / (med / 1e3) / 1e9, 1),
                            "peak_gbs": PEAK_HBM_GBS,
                            "frac": round(hbm / (med / 1e3) / 1e9 / PEAK_HBM_GBS, 4)}}
    del d, ws, out
    torch.cuda.empty_cache()
    return res


BWD_KERNEL = {
    "dh_routed": "gemm_bwd_kernel<0> (routed dy W2)",
    "dh_shared": "gemm_bwd_kernel<0> (shared dy W2)",
    "gateup_bwd_routed": "gemm_bf16_kernel<GATEUP_BWD> (routed)",
    "gateup_bwd_shared": "gemm_bf16_kernel<GATEUP_BWD> (shared)",
    "dx_routed": "gemm_bwd_kernel<1> (routed dA [W1; W3])",
    "dx_shared": "gemm_bwd_kernel<1> (shared dA [W1; W3])",
    "dw2_routed": "gemm_bwd_kernel<2> (routed dW2)",
    "dw13_routed": "gemm_bwd_kernel<3> (routed dW1, dW3)",
    "dw2_shared": "gemm_bwd_kernel<2> (shared dW2)",
    "dw13_shared": "gemm_bwd_kernel<3> (shared dW1, dW3)",
}


def backward_stage_flops(cfg):
    """Matrix FLOPs of each GEMM stage of the backward (the recomputed
    gate/up included): R = T K routed rows, S = K_s I_s shared columns."""
    R, T, d, I = cfg.T * cfg.top_k, cfg.T, cfg.d, cfg.inner
    S = cfg.n_shared * cfg.shared_inner
    return {"dh_routed": 2.0 * R * d * I, "dh_shared": 2.0 * T * d * S,
            "gateup_bwd_routed": 4.0 * R * d * I, "gateup_bwd_shared": 4.0 * T * d * S,
            "dx_routed": 4.0 * R * d * I, "dx_shared": 4.0 * T * d * S,
            "dw2_routed": 2.0 * R * d * I, "dw13_routed": 4.0 * R * d * I,
            "dw2_shared": 2.0 * T * d * S, "dw13_shared": 4.0 * T * d * S}


def time_backward(moe, cfg, d, steps, warmup):
    """The layer backward on the same workload: dout N(0, 1) in bf16, every
    gradient written each step; stage times from HIP events on the stream."""
    import torch
    g = torch.Generator(device=d["x"].device).manual_seed(0)
    dout = torch.randn(d["x"].shape, generator=g, device=d["x"].device).to(torch.bfloat16)
    desc = moe.make_desc(cfg.T, cfg.d, cfg.n_routed, cfg.top_k, cfg.inner,
                         cfg.n_shared, cfg.shared_inner, n_groups=cfg.n_groups,
                         topk_groups=cfg.topk_groups, score=cfg.score,
                         norm_topk=cfg.norm_topk, routed_scale=cfg.routed_scale)
    ws = torch.empty(moe.backward_workspace_size(desc), dtype=torch.uint8,
                     device=d["x"].device)
    names = moe.backward_stage_names()
    nst = len(names)
    events = [moe.HipEvents(nst + 1) for _ in range(steps)]
    grads = None

    def step(ev=None):
        nonlocal grads
        grads = moe.moe_layer_backward(
            d["x"], d["w_gate"], d["routed"], d["shared"], cfg.top_k, dout,
            score=cfg.score, norm_topk=cfg.norm_topk, n_groups=cfg.n_groups,
            topk_groups=cfg.topk_groups, select_bias=d["select_bias"],
            logit_bias=d["logit_bias"], routed_scale=cfg.routed_scale, workspace=ws,
            grads=grads, trace_events=None if ev is None else ev.handles)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    for i in range(steps):   # stage breakdown: a traced pass (stages in order)
        step(events[i])
    torch.cuda.synchronize()
    stage_ms = {n: sum(ev.elapsed_ms(i, i + 1) for ev in events) / steps
                for i, n in enumerate(names)}
    for ev in events:
        ev.close()
    flops = backward_stage_flops(cfg)
    total = sum(flops.values())
    dom = max(flops, key=lambda n: stage_ms[n])
    ach = flops[dom] / (stage_ms[dom] / 1e3) / 1e12
    return {
        "ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.T / (ms / 1e3), 1),
        "expert_tflop_per_step": round(total / 1e12, 3),
        "tflops": round(total / (ms / 1e3) / 1e12, 1),
        "frac_bf16_peak": round(total / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stage_tflops": {k: round(flops[k] / (stage_ms[k] / 1e3) / 1e12, 1)
                         for k in flops if stage_ms[k] > 0},
        "roofline": {"kernel": BWD_KERNEL[dom], "bound": "mfma", "achieved": round(ach, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                     "traffic": (measured_traffic(BWD_TRAFFIC[dom]) if dom in BWD_TRAFFIC
                                 else None),
                     "flops_per_launch": flops[dom], "avg_launch_ms": round(stage_ms[dom], 4)},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="deepseekmoe-16b")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="oracle sample size (0: all tokens of the workload)")
    ap.add_argument("--cpu-reps", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-cache", action="store_true",
                    help="weight-streaming report: overwrite a 1 GiB buffer before "
                         "each timed call so that no weights stay in L2 / MALL")
    ap.add_argument("--reps", type=int, default=50,
                    help="calls timed one by one for the per-call statistics")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the layer backward on the same workload")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 (E4M3) variant of the same workload")
    ap.add_argument("--no-other-shapes", action="store_true",
                    help="skip the 2B-shaped, V3-shaped and skewed small-batch layers "
                         "reported beside the 16B-shaped headline")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (for "
                         "scaling HBM byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the dominant kernel's traffic summary from two "
                         "rocprofv3 --pmc counter files and exit")
    args = ap.parse_args()
    if args.traffic_from:
        summarize_traffic(*args.traffic_from, args.copy_calibration_mb or 1024)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import oracle
    import workloads
    import mixture_experts_layer_mk_amd as moe

    cfg = workloads.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    log(f"[bench] generating {cfg.name}")
    inp = workloads.make_inputs(cfg)
    host = inp.torch_tensors("cpu")
    d = {k: (tuple(t.to(dev) for t in v) if isinstance(v, tuple)
             else (v.to(dev) if v is not None else None)) for k, v in host.items()}
    desc = moe.make_desc(cfg.T, cfg.d, cfg.n_routed, cfg.top_k, cfg.inner,
                         cfg.n_shared, cfg.shared_inner, n_groups=cfg.n_groups,
                         topk_groups=cfg.topk_groups, score=cfg.score,
                         norm_topk=cfg.norm_topk, routed_scale=cfg.routed_scale,
                         dtype=cfg.dtype)
    ws = torch.empty(moe.workspace_size(desc), dtype=torch.uint8, device=dev)
    out = torch.empty_like(d["x"])
    names = moe.trace_stage_names()
    nst = len(names)
    events = [moe.HipEvents(nst + 1) for _ in range(args.steps)]

    def step(ev=None):
        moe.moe_layer_forward(d["x"], d["w_gate"], d["routed"], d["shared"], cfg.top_k,
                              score=cfg.score, norm_topk=cfg.norm_topk,
                              n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                              select_bias=d["select_bias"], logit_bias=d["logit_bias"],
                              routed_scale=cfg.routed_scale, out=out, workspace=ws,
                              trace_events=None if ev is None else ev.handles)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # Stage breakdown from a traced pass of as many steps: a traced call runs
    # the same launches as an untraced one, with events between them.
    log(f"[bench] traced pass {args.steps} steps")
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    stage_ms = {n: 0.0 for n in names}
    total_ev = 0.0
    for ev in events:
        for i, n in enumerate(names):
            stage_ms[n] += ev.elapsed_ms(i, i + 1) / args.steps
        total_ev += ev.elapsed_ms(0, nst) / args.steps
    for ev in events:
        ev.close()
    ms = wall * 1e3 / args.steps
    tok_s = cfg.T / (ms / 1e3)
    fpt = oracle.expert_flops_per_token(cfg.d, cfg.top_k, cfg.inner, cfg.n_shared,
                                        cfg.shared_inner)
    act_tflops = fpt * cfg.T / (ms / 1e3) / 1e12
    router_gflop = 2 * cfg.T * cfg.d * cfg.n_routed / 1e9

    # dominant kernel: the gate/up GEMM launch (routed and shared tiles),
    # 2 * d * 2 * (T*K * inner + T * K_s * I_s) flops
    dom_flops = gateup_flops(cfg)
    dom_ms = stage_ms[DOMINANT]
    achieved = dom_flops / (dom_ms / 1e3) / 1e12
    roofline = {"kernel": "gemm_bf16_kernel<GATEUP> (routed + shared launch)", "bound": "mfma",
                "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic("bf16"),
                "flops_per_launch": dom_flops, "avg_launch_ms": round(dom_ms, 4)}

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    # The step after a training forward: the auxiliary-loss-free bias update
    # on this forward's expert counts (one small kernel), timed on its own.
    _, rt = moe.moe_layer_forward(d["x"], d["w_gate"], d["routed"], d["shared"], cfg.top_k,
                                  score=cfg.score, norm_topk=cfg.norm_topk,
                                  n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                                  select_bias=d["select_bias"], logit_bias=d["logit_bias"],
                                  routed_scale=cfg.routed_scale, workspace=ws,
                                  return_routing=True)
    sb = torch.zeros(cfg.n_routed, dtype=torch.float32, device=dev)
    rel = torch.empty_like(sb)
    for _ in range(3):
        moe.moe_bias_update(rt["expert_counts"], 1e-3, sb, rel)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(50):
        moe.moe_bias_update(rt["expert_counts"], 1e-3, sb, rel)
    e1.record()
    torch.cuda.synchronize()
    bias_us = e0.elapsed_time(e1) / 50 * 1e3
    max_rel_load = float(rel.max())

    # Per-call statistics and the whole layer against the HBM roofline: the
    # weights of the experts that receive tokens, x and out.  Layers with few
    # rows per expert stream their weights, and that is their roofline.
    import numpy as np
    counts = rt["expert_counts"].cpu().numpy()
    hbm_bytes, nonempty = layer_hbm_bytes(cfg, counts)
    log(f"[bench] {args.reps} calls timed one by one (cold cache: {args.cold_cache})")
    calls = per_call_ms(step, args.reps, args.cold_cache, dev)
    med = float(np.median(calls))
    p10, p90 = (float(v) for v in np.percentile(calls, [10, 90]))
    per_call = {"median_ms": round(med, 4), "p10_ms": round(p10, 4), "p90_ms": round(p90, 4),
                "reps": args.reps, "cold_cache": bool(args.cold_cache)}
    layer_gbs = hbm_bytes / (med / 1e3) / 1e9
    layer_hbm = {"bytes": hbm_bytes, "nonempty_experts": nonempty,
                 "achieved_gbs": round(layer_gbs, 1), "peak_gbs": PEAK_HBM_GBS,
                 "frac": round(layer_gbs / PEAK_HBM_GBS, 4)}
    streaming = cfg.T * cfg.top_k / cfg.n_routed < 512
    if streaming:
        roofline = {"kernel": "whole layer forward (weight streaming)", "bound": "hbm",
                    "achieved": round(layer_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(layer_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                    "bytes_per_launch": hbm_bytes, "avg_launch_ms": round(med, 4)}
        ms = med
        tok_s = cfg.T / (ms / 1e3)
        act_tflops = fpt * cfg.T / (ms / 1e3) / 1e12

    # Attainable bf16 matrix rate on this GPU: the vendor GEMM (torch.matmul,
    # hipBLASLt) on a square 8192^3 problem, timed with events.
    a8 = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b8 = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        a8 @ b8
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        a8 @ b8
    e1.record()
    torch.cuda.synchronize()
    attain = 2.0 * 8192 ** 3 / (e0.elapsed_time(e1) / 10 / 1e3) / 1e12
    del a8, b8

    # Achieved rates of the stages around the GEMMs: the router's logits
    # (fp32-accurate, 2 T d E FLOPs; x, the gate and the choice as bytes) and
    # the permute's row maps (the choice read, two int32 maps written).
    def rate(nbytes, ms_):
        return round(nbytes / (ms_ / 1e3) / 1e9, 1) if ms_ > 0 else None
    TKn = cfg.T * cfg.top_k
    xb = 2 if cfg.dtype == "bf16" else 4
    router_bytes = cfg.T * cfg.d * xb + cfg.n_routed * cfg.d * 4 + TKn * 8
    stage_rates = {
        "router": {"tflops_fp32_equiv": round(2.0 * cfg.T * cfg.d * cfg.n_routed /
                                              (stage_ms["router"] / 1e3) / 1e12, 2),
                   "gbs": rate(router_bytes, stage_ms["router"])},
        "permute": {"gbs": rate(TKn * 4 * 3, stage_ms["permute"])},
        # S (fp32) or x read, the fp16 Y rows and their scales read, out written
        "combine": {"gbs": rate((cfg.T * cfg.d * 4 if cfg.n_shared else cfg.T * cfg.d * xb) +
                                TKn * cfg.d * 2 + TKn * (cfg.d // 64) * 4 +
                                cfg.T * cfg.d * xb, stage_ms["combine"])},
    }

    fp8 = None
    if not args.no_fp8 and cfg.dtype == "bf16" and not args.cold_cache:
        log(f"[bench] fp8 variant: {args.steps} steps")
        fp8 = time_fp8(moe, cfg, d, args.steps, args.warmup, fpt)

    bwd = None
    if not args.no_backward and cfg.dtype == "bf16" and not args.cold_cache:
        log(f"[bench] backward: {args.steps} steps")
        bwd = time_backward(moe, cfg, d, args.steps, args.warmup)

    others = {}
    if not args.no_other_shapes and args.config == "deepseekmoe-16b" and not args.cold_cache:
        for key, name, cold in OTHER_SHAPES:
            others[key] = time_shape(moe, workloads.CONFIGS[name], dev, args.steps,
                                     args.warmup, args.reps, cold)

    cpu = None
    if not args.no_cpu_baseline:
        n = min(args.cpu_tokens or (min(cfg.T, 512) if streaming else cfg.T), cfg.T)
        log(f"[bench] cpu baseline: {args.cpu_reps} x {n} tokens")
        cpu = cpu_baseline(cfg, host, n, args.cpu_reps)

    res = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": (f"{cfg.name} MoE layer: T={cfg.T}, d={cfg.d}, "
                                f"{cfg.n_routed} routed (inner {cfg.inner}, top-{cfg.top_k}, "
                                f"{cfg.score}"
                                + (f", {cfg.n_groups} groups keep {cfg.topk_groups}, selection bias"
                                   if cfg.n_groups > 1 else "")
                                + (f", Zipf({cfg.zipf_s}) logit bias" if cfg.zipf_s else "")
                                + f") + {cfg.n_shared} shared (inner {cfg.shared_inner})"
                                + (", cold cache" if args.cold_cache else "")),
                   "tokens": cfg.T, "parallelism": "single-gpu"},
        "activated_tflops": round(act_tflops, 1),
        "frac_bf16_peak": round(act_tflops / PEAK_BF16_TFLOPS, 4),
        "router_gflop": round(router_gflop, 2),
        "stages_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stage_rates": stage_rates,
        "events_ms_per_step": round(total_ev, 4),
        "roofline": roofline,
        "per_call": per_call,
        "layer_hbm": layer_hbm,
        "bias_update": {"us_per_call": round(bias_us, 2), "max_relative_load": round(max_rel_load, 4)},
        "attainable_bf16_tflops": {"value": round(attain, 1),
                                   "how": "vendor GEMM (torch.matmul / hipBLASLt), bf16 8192^3"},
        "fp8": fp8,
        "backward": bwd,
        "other_shapes": others or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
