#!/usr/bin/env python3
"""Benchmark of the MoE expert-parallel layer on one MI355X.

One step = one fused layer forward (moe_ep_layer_forward_timed: dispatch ->
bridge -> grouped gate_up GEMM with SwiGLU -> down GEMM -> weighted combine)
over one batch of synthetic inputs already resident in HBM.  The default
workload is the high-throughput prefill share: 8 source ranks x 4096 tokens,
H=7168, I=2048, 256 experts of which 32 are local, top-8, Zipf(1.1) expert
popularity, FLAT receive layout.

Prints ONE JSON line: whole-job tokens/s, per-stage times from HIP events
recorded by the library at the stage boundaries inside the timed steps, the
roofline of the dominant kernel (the gate_up GEMM, bf16 MFMA), and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s on 1 GPU; grouped-GEMM MFMA util; dispatch/combine GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_units(cfg, ids, mask=None):
    """Local picks P, tokens with a local pick R (host count from the routing inputs); tokens of a
    source rank whose mask entry is 0 have none."""
    import numpy as np
    o = cfg.rank * cfg.num_local_experts
    loc = (ids >= o) & (ids < o + cfg.num_local_experts)
    if mask is not None:
        loc &= np.repeat(mask != 0, cfg.max_tokens_per_rank)[: cfg.num_tokens, None]
    return int(loc.sum()), int(loc.any(axis=1).sum())


def experts_with_rows(cfg, ids, mask=None) -> int:
    """Local experts with at least one local pick (the experts whose weights the GEMMs read)."""
    import numpy as np
    o = cfg.rank * cfg.num_local_experts
    loc = (ids >= o) & (ids < o + cfg.num_local_experts)
    if mask is not None:
        loc &= np.repeat(mask != 0, cfg.max_tokens_per_rank)[: cfg.num_tokens, None]
    return int(np.unique(ids[loc]).size)


def gate_up_roofline(cfg, P: int, L_rows: int, t_ms: float, fp8: bool, traffic) -> dict:
    """Roofline of the gate_up GEMM launch that took t_ms: bound by the MFMA peak or by HBM, whichever
    its arithmetic intensity puts it under (flop per algorithmic byte: the weights of the L_rows local
    experts with rows, read once, the P gathered A rows and the P h rows written).  With few rows per
    expert the GEMM streams weights."""
    H, I = cfg.hidden, cfg.intermediate
    flops = 4.0 * P * I * H
    k_row = H + ((H // 128 + 3) // 4 * 4) if fp8 else 2 * H  # one K-long row (+ FP8 scales), bytes
    nbytes = L_rows * 2 * I * k_row + P * k_row + P * I * 2
    peak_f = FP8_MFMA_PEAK_TFLOPS if fp8 else BF16_MFMA_PEAK_TFLOPS
    if fp8:
        kname = "k_gemm_fp8_gate_up (FP8 grouped gate_up GEMM + SwiGLU)"
    elif cfg.num_tokens * cfg.top_k >= 512 * cfg.num_experts:  # the library's 256-row tiles from 512 mean rows
        kname = "k_grouped_gemm16<true> (grouped gate_up GEMM + SwiGLU, 256-row tiles)"
    else:
        kname = "k_grouped_gemm<true> (grouped gate_up GEMM + SwiGLU, 64-row tiles)"
    if flops / nbytes >= peak_f * 1e12 / (HBM_PEAK_GBS * 1e9):
        achieved = flops / (t_ms * 1e-3) / 1e12
        return {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 1), "peak": peak_f,
                "unit": "TFLOP/s", "frac": round(achieved / peak_f, 4), "traffic": traffic}
    achieved = nbytes / (t_ms * 1e-3) / 1e9
    return {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "algorithmic_bytes": nbytes}


def algorithmic_bytes(cfg, P: int, R: int, fp8: bool = False) -> tuple[int, int]:
    """(dispatch bytes, combine bytes) the method must move, per layer forward.  With FP8 dispatch a
    received row is H code bytes plus its padded scale bytes instead of 2H."""
    N, K, H = cfg.num_tokens, cfg.top_k, cfg.hidden
    row = 2 * H
    recv_row = H + ((H // 128 + 3) // 4 * 4) if fp8 else row
    ids = N * K * 8
    if cfg.layout == "EXPERT_MAJOR":
        dispatch = ids + R * row + P * recv_row + N * K * 4 + P * 4
        combine = P * row + N * row + N * K * (4 + 4)
    elif cfg.layout == "RANK_MAJOR":
        dispatch = ids + R * row + R * recv_row + N * K * 8
        combine = P * row + N * row + R * K * (4 + 4) + N * 4
    else:
        dispatch = ids + R * row + R * recv_row + R * K * 8 + R * 4
        combine = P * row + N * row + R * K * (4 + 4) + N * 4
    return dispatch, combine


def _traffic_source(fp8: bool):
    """The committed HBM-traffic summary for the gate_up kernel and the sources that kernel is built from."""
    csrc = os.path.join(ROOT, "combine_topk_ids_amd", "csrc")
    if fp8:
        return (os.path.join(ROOT, "profiles", "hbm_traffic_prefill_flat_zipf_fp8.md"),
                [os.path.join(csrc, f) for f in ("gemm_fp8.hip", "common.h")])
    return (os.path.join(ROOT, "profiles", "hbm_traffic_prefill_flat_zipf.md"),
            [os.path.join(csrc, f) for f in ("gemm.hip", "common.h")])


def measured_gate_up_traffic(workload: str, fp8: bool = False):
    """HBM bytes per gate_up launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary,
    or None if that summary is for another workload or for a different kernel source."""
    import hashlib
    path, sources = _traffic_source(fp8)
    if workload != "prefill_flat_zipf" or not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in sources:
        with open(f, "rb") as fh:
            h.update(fh.read())
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":")[0] in ("gate_up_traffic_bytes_per_launch", "gemm_source_sha256"):
                k, v = line.split(":", 1)
                vals[k] = v.strip()
    if vals.get("gemm_source_sha256") != h.hexdigest():
        return None
    return float(vals["gate_up_traffic_bytes_per_launch"])


def device_copy_gbps(torch, nbytes: int = 2 << 30, reps: int = 5) -> float:
    """Read+write GB/s of a plain device-to-device copy of nbytes (context for the HBM figures)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    return 2.0 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9


def router_time_us(torch, m, cfg, reps: int) -> tuple[float, int]:
    """Average time of the router (top_k of N x E fp32 scores + softmax) on N(0,1) scores of the
    workload's shape, outside the layer's timed steps; and its algorithmic bytes."""
    N, E, K = cfg.num_tokens, cfg.num_experts, cfg.top_k
    g = torch.Generator(device="cuda").manual_seed(7)
    scores = torch.randn((N, E), generator=g, device="cuda", dtype=torch.float32)
    ids = torch.empty((N, K), dtype=torch.int64, device="cuda")
    w = torch.empty((N, K), dtype=torch.float32, device="cuda")
    m.moe_ep_router_topk(scores, K, ids, w)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        m.moe_ep_router_topk(scores, K, ids, w)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / reps, N * E * 4 + N * K * (8 + 4)


def cpu_baseline(cfg, d, sample: int, mask=None) -> dict:
    import numpy as np
    import oracle
    n = cfg.num_tokens
    step = max(1, n // sample)
    toks = np.arange(0, n, step)[:sample]
    p = oracle.params(cfg, active_ranks=mask)
    t0 = time.perf_counter()
    oracle.forward_tokens(p, d["hidden_states"], d["topk_ids"], d["topk_weights"], d["w_gate_up"], d["w_down"],
                          toks, threads=1)
    dt = time.perf_counter() - t0
    # the same oracle over all the host cores this process may use (at most 16, the box's share):
    # independent instances over disjoint token ranges, on a sample as many times larger
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    step_all = max(1, n // (sample * threads))
    toks_all = np.arange(0, n, step_all)[: sample * threads]
    t1 = time.perf_counter()
    oracle.forward_tokens(p, d["hidden_states"], d["topk_ids"], d["topk_weights"], d["w_gate_up"], d["w_down"],
                          toks_all, threads=threads)
    dt_all = time.perf_counter() - t1
    return {"value": round(len(toks) / dt, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(toks)} of {n} tokens (every {step}th), full per-token layer output, single-threaded C "
                      f"oracle, {dt:.1f} s",
            "host": host_cpu(),
            "all_cores": {"value": round(len(toks_all) / dt_all, 3), "unit": "tokens/s", "cores": threads,
                          "sample": f"{len(toks_all)} of {n} tokens (every {step_all}th), {threads} oracle "
                                    f"instances over disjoint token ranges, {dt_all:.1f} s"}}


def host_cpu() -> str:
    """CPU model name and the number of cores this process may use (for the oracle's baseline)."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {len(os.sched_getaffinity(0))} cores available"


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: at least 5 and at least 0.25 s of steps)")
    ap.add_argument("--workload", default="prefill_flat_zipf")
    ap.add_argument("--cpu-sample", type=int, default=768,
                    help="tokens the CPU oracle baseline runs on (about 10-30 s of single-core work)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8", action="store_true",
                    help="FP8 dispatch + FP8 gate_up GEMM (moe_ep_layer_forward_fp8); W1 quantised once, untimed")
    ap.add_argument("--inactive-ranks", default="",
                    help="comma-separated source ranks marked inactive in the active_ranks mask")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs one GPU's share of the layer on exactly one GPU; --gpus {args.gpus} "
              f"(WORLD_SIZE {world}) is not supported by this build", file=sys.stderr, flush=True)
        return 2

    import numpy as np
    import torch

    import combine_topk_ids_amd as m
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = synth.get_config(args.workload)
    log(f"workload {cfg}")
    t0 = time.perf_counter()
    d = synth.make_inputs(cfg)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    inactive = [int(r) for r in args.inactive_ranks.split(",") if r.strip()]
    mask_h = None
    if inactive:
        mask_h = np.ones(cfg.world, np.int32)
        mask_h[inactive] = 0
    P, R = algorithmic_units(cfg, d["topk_ids"], mask_h)
    L_rows = experts_with_rows(cfg, d["topk_ids"], mask_h)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    x = dev(d["hidden_states"])
    ids = torch.from_numpy(d["topk_ids"]).cuda()
    w = torch.from_numpy(d["topk_weights"]).cuda()
    identity = cfg.intermediate == 0
    w1 = None if identity else dev(d["w_gate_up"])
    w2 = None if identity else dev(d["w_down"])
    p = m.params(cfg.num_experts, cfg.num_local_experts, cfg.rank, cfg.max_tokens_per_rank, cfg.num_tokens,
                 cfg.hidden, cfg.intermediate, cfg.top_k, cfg.layout)
    ws = torch.zeros(m.moe_ep_workspace_size(p), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    mask = None if mask_h is None else torch.from_numpy(mask_h).cuda()
    if args.fp8:
        if identity:
            log("--fp8 needs an expert GEMM (intermediate > 0)")
            return 2
        L2I = cfg.num_local_experts * 2 * cfg.intermediate
        w1q = torch.empty((L2I, cfg.hidden), dtype=torch.uint8, device="cuda")
        w1s = torch.empty((L2I, m.moe_ep_fp8_scale_stride(cfg.hidden)), dtype=torch.uint8, device="cuda")
        m.moe_ep_quantize_fp8(w1.view(L2I, cfg.hidden), w1q, w1s)

        def forward(evs):
            m.moe_ep_layer_forward_fp8(p, x, ids, w, w1q, w1s, w2, out, ws, events=evs, active_ranks=mask)
    else:
        def forward(evs):
            m.moe_ep_layer_forward_timed(p, x, ids, w, w1, w2, out, ws, evs, active_ranks=mask)
    torch.cuda.synchronize()

    if args.warmup is None:
        t1 = time.perf_counter()
        forward([None] * 6)
        torch.cuda.synchronize()
        one = max(time.perf_counter() - t1, 1e-6)
        args.warmup = max(5, int(np.ceil(0.25 / one)))
        done = 1
    else:
        done = 0
    for _ in range(args.warmup - done):
        forward([None] * 6)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # torch creates an event's HIP handle on its first record(); record each once here so the
    # library can re-record the handles at the stage boundaries inside the timed steps.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for ev in events:
        for e in ev:
            e.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        forward(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall * 1e3:.2f} ms")
    if not torch.isfinite(out.float()).all():
        log("non-finite values in the output")
        return 1
    # Cold-cache check, outside the timed steps: a few more layers, each after a 1 GiB scratch write
    # that evicts the 256 MB Infinity Cache (and L2), timed by their own stage events.
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    cold = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(min(args.steps, 10))]
    for ev in cold:
        for e in ev:
            e.record()
    torch.cuda.synchronize()
    for ev in cold:
        scratch.fill_(1)
        forward(ev)
    torch.cuda.synchronize()
    layer_cold_ms = float(np.median([ev[0].elapsed_time(ev[5]) for ev in cold]))
    del scratch
    copy_gbps = device_copy_gbps(torch)
    router_us, router_bytes = router_time_us(torch, m, cfg, args.steps)

    def avg_ms(a: int, b: int) -> float:
        return float(np.mean([ev[a].elapsed_time(ev[b]) for ev in events]))

    layer_ms = np.array([ev[0].elapsed_time(ev[5]) for ev in events])

    t_dispatch = avg_ms(0, 1)
    t_bridge = avg_ms(1, 2)
    t_gate_up = avg_ms(2, 3)
    t_down = avg_ms(3, 4)
    t_combine = avg_ms(4, 5)
    t_layer = avg_ms(0, 5)
    H, I, N = cfg.hidden, cfg.intermediate, cfg.num_tokens
    disp_bytes, comb_bytes = algorithmic_bytes(cfg, P, R, args.fp8)
    stages = {
        "layer_us": round(t_layer * 1e3, 2),
        "layer_us_median": round(float(np.median(layer_ms)) * 1e3, 2),
        "layer_us_min": round(float(layer_ms.min()) * 1e3, 2),
        "layer_us_cold_cache_median": round(layer_cold_ms * 1e3, 2),
        "dispatch_us": round(t_dispatch * 1e3, 2),
        "bridge_us": round(t_bridge * 1e3, 2),
        "gate_up_gemm_us": round(t_gate_up * 1e3, 2),
        "down_gemm_us": round(t_down * 1e3, 2),
        "combine_us": round(t_combine * 1e3, 2),
        "local_picks": P,
        "tokens_with_local_pick": R,
        "dispatch_GBps": round(disp_bytes / (t_dispatch * 1e-3) / 1e9, 1),
        "combine_GBps": round(comb_bytes / (t_combine * 1e-3) / 1e9, 1),
        "dispatch_combine_hbm_frac": round((disp_bytes + comb_bytes) / ((t_dispatch + t_combine) * 1e-3) / 1e9
                                           / HBM_PEAK_GBS, 4),
        "context_device_copy_GBps": round(copy_gbps, 1),
        "router_us": round(router_us, 2),
        "router_GBps": round(router_bytes / (router_us * 1e-6) / 1e9, 1),
    }
    roofline = None
    if not identity:
        gemm_flops = 6.0 * P * I * H
        t_gemm = (t_gate_up + t_down) * 1e-3
        stages["gemm_TFLOPs"] = round(gemm_flops / t_gemm / 1e12, 1)
        # both GEMMs against their own peaks: the time they would take at peak / the time they took
        # (with --fp8 the gate_up GEMM runs at the FP8 peak, the down GEMM at the bf16 one)
        gu_peak = FP8_MFMA_PEAK_TFLOPS if args.fp8 else BF16_MFMA_PEAK_TFLOPS
        t_peak = (4.0 * P * I * H / gu_peak + 2.0 * P * I * H / BF16_MFMA_PEAK_TFLOPS) / 1e12
        stages["gemm_mfma_frac"] = round(t_peak / t_gemm, 4)
        roofline = gate_up_roofline(cfg, P, L_rows, t_gate_up, args.fp8,
                                    measured_gate_up_traffic(cfg.name, fp8=args.fp8))
    else:
        achieved = (disp_bytes + comb_bytes) / ((t_dispatch + t_combine) * 1e-3) / 1e9
        roofline = {"kernel": "dispatch + combine", "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": None}

    result = {
        "metric": METRIC,
        "value": round(N * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 e4m3 dispatch + gate_up, bf16 down" if args.fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "layout": cfg.layout, "num_tokens": N, "world": cfg.world,
                   "max_tokens_per_rank": cfg.max_tokens_per_rank, "num_experts": cfg.num_experts,
                   "num_local_experts": cfg.num_local_experts, "rank": cfg.rank, "top_k": cfg.top_k,
                   "hidden": H, "intermediate": I, "routing": f"zipf({cfg.zipf_s})" if cfg.zipf_s else "uniform",
                   "parallelism": "one GPU's expert-parallel share",
                   **({"inactive_ranks": inactive} if inactive else {})},
        "stages": stages,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline and not args.fp8:
        log("timing the CPU oracle on a token sample")
        result["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_sample, mask_h)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
