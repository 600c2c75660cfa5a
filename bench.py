"""Training-throughput benchmark: GPT-2 training steps (forward + backward +
AdamW) through the HIP C-ABI library on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 124m|350m|1.6b]
                    [--accum M] [--max-grad-norm X] [--graph] [--arch relu2,qk_norm,rope]

(--accum / --max-grad-norm time updates over M accumulated micro-batches with
global-norm clipping; --graph replays each step from one captured HIP graph;
--arch turns on architecture variants of the block; the defaults time the
plain step of the headline metric.)

Prints one JSON line.  value = tokens/s of whole training steps (inputs
already resident in HBM), MFU against the bf16 dense MFMA peak, the roofline
position of the step's dominant kernel (its average launch duration measured
with HIP events on the library stream during the timed steps), and the CPU
oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "train tokens/sec + MFU, GPT-2 124M B=24 T=1024 bf16, 1 MI355X"
PEAK_BF16 = 2.5e15        # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12         # MI355X HBM3E, bytes/s
CPU_ROWS = 4              # batch rows of the CPU-oracle sample

CONFIGS = {
    "124m": dict(V=50257, Vp=50304, maxT=1024, L=12, H=12, C=768, B=24, T=1024, lr=6e-4, wd=0.1),
    "350m": dict(V=50257, Vp=50304, maxT=1024, L=24, H=16, C=1024, B=16, T=1024, lr=6e-4, wd=0.1),
    "1.6b": dict(V=50257, Vp=50304, maxT=1024, L=48, H=25, C=1600, B=8, T=1024, lr=2e-4, wd=0.1),
}

# kernel sites the library can time (include/gpt2.h); each is one kernel.  The
# GEMMs and the attention products are bounded by the matrix cores, the rest
# by HBM bandwidth.
GEMM_SITES = ["qkv", "attproj", "fc", "fcproj", "logits", "fcproj_dx", "fcproj_dw", "fc_dx", "fc_dw",
              "attproj_dx", "attproj_dw", "qkv_dx", "qkv_dw", "cls_dx", "cls_dw"]
MFMA_SITES = set(GEMM_SITES) | {"attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq"}


def flops_per_token(c) -> float:
    """6 N + 12 L C T with N the unpadded parameter count (model FLOPs)."""
    V, T, L, C = c["V"], c["maxT"], c["L"], c["C"]
    N = V * C + T * C + L * (12 * C * C + 13 * C) + 2 * C
    return 6.0 * N + 12.0 * L * C * c["T"]


# kernel that runs at each site for the 124M shapes in bf16 (the name rocprofv3
# reports, up to its template arguments)
KERNEL_OF = {
    "attn_fwd": "attn_fwd_mfma_kernel", "attn_bwd_dkdv": "attn_bwd_dkdv_mfma_kernel",
    "attn_bwd_dq": "attn_bwd_dq_mfma_kernel", "attn_bwd_dot": "attn_bwd_dot_kernel",
    "softmax_xent": "softmax_xent_bf16_kernel", "ln_fwd": "ln_fwd_half_kernel", "ln_bwd": "ln_bwd_kernel",
    "encoder_fwd": "encoder_fwd_kernel", "adamw": "adamw_fused_kernel", "weight_transpose": "transpose_bf16_kernel",
    "grad_norm": "grad_sumsq_kernel", "qk_fwd": "qk_fwd_kernel", "qk_bwd": "qk_bwd_kernel",
    "fp8_quant": "quantize_kernel",
}
for _s in GEMM_SITES:
    KERNEL_OF[_s] = "gemm_bf16_dma_kernel"


def roofline_of(site, r):
    """Roofline position of one timed site: algorithmic work per launch over
    the average launch duration, against the MI355X dense bf16 or HBM peak."""
    avg_ms = r["total_ms"] / max(r["launches"], 1)
    if site in MFMA_SITES:
        achieved = r["flops_per_launch"] / (avg_ms / 1e3) / 1e12
        return {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": achieved / (PEAK_BF16 / 1e12), "algorithmic_per_launch": r["flops_per_launch"],
                "avg_ms": avg_ms}
    achieved = r["bytes_per_launch"] / (avg_ms / 1e3) / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": achieved / (PEAK_HBM / 1e9), "algorithmic_per_launch": r["bytes_per_launch"], "avg_ms": avg_ms}


def measured_traffic(site, config):
    """HBM bytes per launch of the site's kernel from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel), or
    None when there is none for this site and workload, or when the kernel's
    source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{site}_{config}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    srcs = [s.strip() for s in kv.get("source", "").split(",") if s.strip()]
    shas = [s.strip() for s in kv.get("source_sha256", "").split(",")]
    if not srcs or len(srcs) != len(shas):
        return None
    for src, sha in zip(srcs, shas):
        path_src = os.path.join(ROOT, src)
        if not os.path.isfile(path_src):
            return None
        with open(path_src, "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != sha:
                return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(c, seed):
    """The CPU oracle (float32 numpy), as it stands, on one sequence of the
    same workload: one forward + backward + AdamW step on CPU_ROWS rows of
    T=1024 tokens (a bounded sample of the B=24 batch)."""
    import oracle as O
    from gpt_transformer_lm_amd import synthetic as S
    cores = len(os.sched_getaffinity(0))
    oc = O.OracleConfig(vocab_size=c["V"], max_seq_len=c["maxT"], num_layers=c["L"], num_heads=c["H"],
                        channels=c["C"])
    params = S.random_params(c["V"], c["V"], c["maxT"], c["L"], c["C"], seed=seed, perturbed=False)
    tok, tgt = S.zipf_batch(CPU_ROWS, c["T"], seed=seed + 1)
    t0 = time.perf_counter()
    O.gpt2_step(params, tok, tgt, oc, None, c["lr"], 0.9, 0.999, 1e-8, c["wd"], 1)
    dt = time.perf_counter() - t0
    return {"value": CPU_ROWS * c["T"] / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{CPU_ROWS} sequences x {c['T']} tokens ({CPU_ROWS} of the {c['B']} rows of a batch): one "
                      f"float32 numpy forward+backward+AdamW step of the same model, {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="124m", choices=sorted(CONFIGS))
    ap.add_argument("--seed", type=int, default=1234)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--site", default=None, help="kernel site to report in roofline (default: the slowest)")
    ap.add_argument("--accum", type=int, default=1,
                    help="micro-batches of B x T accumulated per update (gradient of their mean loss)")
    ap.add_argument("--max-grad-norm", type=float, default=0.0,
                    help="global-norm gradient clipping threshold (0: off)")
    ap.add_argument("--arch", default="",
                    help="comma-separated architecture variants: relu2, qk_norm, rope (default: GPT-2 as published)")
    ap.add_argument("--fp8", action="store_true",
                    help="FP8 products for the QKV projection, the MLP and the head (GPT2_BF16_FP8)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each timed step from one captured HIP graph (plain step only)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a kernel of known traffic, "
                         "to calibrate hardware byte counters against)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from gpt_transformer_lm_amd import lib
    from gpt_transformer_lm_amd import synthetic as S

    c = CONFIGS[args.config]
    B, T = c["B"], c["T"]
    flag_of = {"relu2": lib.GPT2_ARCH_RELU2, "qk_norm": lib.GPT2_ARCH_QK_NORM, "rope": lib.GPT2_ARCH_ROPE}
    arch = [a for a in args.arch.split(",") if a]
    if any(a not in flag_of for a in arch):
        print(f"--arch takes {sorted(flag_of)}", file=sys.stderr)
        sys.exit(2)
    cfg = lib.make_config(c["V"], c["Vp"], c["maxT"], c["L"], c["H"], c["C"], B, T,
                          lib.GPT2_BF16_FP8 if args.fp8 else lib.GPT2_BF16, sum(flag_of[a] for a in set(arch)))
    torch.cuda.init()
    K = max(args.accum, 1)
    plain = K == 1 and args.max_grad_norm <= 0
    if args.graph and not plain:
        print("--graph replays the plain step (no --accum / --max-grad-norm)", file=sys.stderr)
        sys.exit(2)
    # a captured graph needs a stream other than the null stream
    stream = torch.cuda.Stream() if args.graph else torch.cuda.current_stream()
    torch.cuda.set_stream(stream)
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    model = lib.Model(cfg, seed=args.seed, stream=stream)
    nsteps = args.warmup + args.steps
    batches = []
    for s in range(nsteps * K + 1):
        x, y = S.zipf_batch(B, T, seed=args.seed * 1000 + s)
        batches.append((torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()))
    torch.cuda.synchronize()

    # The timed steps read no loss back (nothing waits on the host inside a
    # step); the loss of the first and the last timed step is read afterwards.
    def step(i, t):
        if plain:
            x, y = batches[i]
            model.forward(x, y, read_loss=False)
            model.backward()
            model.adamw_step(c["lr"], 0.9, 0.999, 1e-8, c["wd"], t)
            return None
        # K micro-batches, each forward with loss scale 1/K, gradients accumulated,
        # then the clipped update (norm and factor stay on the device)
        for j in range(K):
            x, y = batches[i * K + j]
            model.forward_scaled(x, y, 1.0 / K)
            if j == 0:
                model.backward()
            else:
                model.backward_accumulate()
        model.adamw_step_clipped(c["lr"], 0.9, 0.999, 1e-8, c["wd"], t, args.max_grad_norm, want_norm=False)
        return None

    # warmup; the last warmup step also times every kernel site once to find the dominant kernel
    t = 0
    for i in range(args.warmup):
        if i == args.warmup - 1:
            for s in lib.SITES:
                model.timing_enable(s, True)
        t += 1
        step(i, t)
    site_ms, sites = {}, {}
    if args.warmup > 0:
        for s in lib.SITES:
            r = model.timing_read(s)
            model.timing_enable(s, False)
            if r["launches"] == 0:
                continue
            site_ms[s] = r["total_ms"]
            sites[s] = dict(roofline_of(s, r), ms=r["total_ms"], launches=r["launches"])
    dom = args.site or (max(site_ms, key=site_ms.get) if site_ms else "fc")
    if args.graph:
        # the timing events sit outside the graph: the dominant kernel's launch
        # time comes from the last warmup step, then the step is captured
        tok_buf = torch.zeros((B, T), dtype=torch.int32, device="cuda")
        tgt_buf = torch.zeros((B, T), dtype=torch.int32, device="cuda")
        model.graph_capture(tok_buf, tgt_buf)

        def step(i, t):
            x, y = batches[i]
            tok_buf.copy_(x)
            tgt_buf.copy_(y)
            model.graph_step(c["lr"], 0.9, 0.999, 1e-8, c["wd"], t, read_loss=False)
    else:
        model.timing_enable(dom, True)

    torch.cuda.synchronize()
    loss_before = model.get_mean_loss() if args.warmup > 0 else None   # last warmup step
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        t += 1
        step(args.warmup + i, t)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    elapsed = wall
    dom_t = sites[dom] if args.graph else model.timing_read(dom)
    loss_last = model.get_mean_loss() if args.steps > 0 else None
    model.close()

    tok_s = K * B * T * args.steps / elapsed
    ftok = flops_per_token(c)
    mfu = tok_s * ftok / PEAK_BF16
    roof = roofline_of(dom, dom_t) if not args.graph else {k: dom_t[k] for k in (
        "bound", "achieved", "peak", "unit", "frac", "algorithmic_per_launch", "avg_ms")}
    roof["traffic"] = measured_traffic(dom, args.config)
    roof.update({"kernel_site": dom, "kernel": KERNEL_OF.get(dom, dom), "avg_launch_ms": roof.pop("avg_ms"),
                 "launches": dom_t["launches"],
                 "timed_in": "the last warmup step (eager)" if args.graph else "the timed steps"})

    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+fp8" if args.fp8 else "bf16",
        "data": "synthetic Zipf(1.1)/EoT token ids, seeded random GPT-2 init",
        "config": {"workload": f"GPT-2 {args.config} training step (fwd+bwd+AdamW, fp32 master), "
                               f"B={B}, T={T}, vocab 50257 padded to 50304"
                               + ("" if plain else f", {K} accumulated micro-batches per update, global-norm "
                                                   f"clipping at {args.max_grad_norm}")
                               + (", each step one HIP graph replay" if args.graph else "")
                               + (f", variants {'+'.join(sorted(set(arch)))}" if arch else "")
                               + (", FP8 (E4M3/E5M2) QKV, MLP and head products" if args.fp8 else ""),
                   "global_batch": K * B, "seq_len": T, "parallelism": "single GPU"},
        "mfu": mfu,
        "model_flops_per_token": ftok,
        "loss_before_after": [loss_before, loss_last],
        "site_ms_one_step": site_ms,
        "site_roofline_one_step": {k: {"ms": round(v["ms"], 4), "n": v["launches"], "frac": round(v["frac"], 4),
                                       "bound": v["bound"]} for k, v in sites.items()},
        "gpu_event_ms_per_step": gpu_ms / args.steps,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(c, args.seed)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
