#!/usr/bin/env python3
"""Benchmark of the MoE expert-parallel layer on one MI355X.

One step = one fused layer forward (moe_ep_layer_forward_timed: dispatch ->
bridge -> grouped gate_up GEMM with SwiGLU -> down GEMM -> weighted combine)
over one batch of synthetic inputs already resident in HBM.  The default
workload is the high-throughput prefill share: 8 source ranks x 4096 tokens,
H=7168, I=2048, 256 experts of which 32 are local, top-8, Zipf(1.1) expert
popularity, FLAT receive layout.

Prints ONE JSON line: whole-job tokens/s over the timed steps (the layer alone),
per-stage times from HIP events that the library records at the stage
boundaries in as many further steps, the roofline of the dominant kernel (the
gate_up GEMM, bf16 MFMA), and the CPU oracle timed on a bounded sample of the
same workload.  The steps alternate between two identical input / weight sets.
The same line carries the other workloads of the layer (low-latency decode in
EXPERT_MAJOR, RANK_MAJOR, the identity-expert bandwidth share) under
"other_workloads": per-stage times with the Infinity Cache flushed before every
step, the layer timed without the stage events inside it, rates and roofline
fractions, and the single-threaded oracle over all of their tokens.
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


def down_roofline(cfg, P: int, L_rows: int, t_ms: float) -> dict:
    """Roofline of the down GEMM launch that took t_ms (bf16): MFMA-bound or HBM-bound by its
    arithmetic intensity over its algorithmic bytes (W2 of the local experts with rows, read once;
    the P h rows read; the P y rows written)."""
    H, I = cfg.hidden, cfg.intermediate
    flops = 2.0 * P * I * H
    nbytes = L_rows * H * I * 2 + P * I * 2 + P * H * 2
    if flops / nbytes >= BF16_MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        achieved = flops / (t_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_MFMA_PEAK_TFLOPS, 4)}
    achieved = nbytes / (t_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes": nbytes}


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


def vendor_dense_gemm(torch, rows: int, H: int, I: int, reps: int = 10) -> dict:
    """Context for the grouped GEMMs: the vendor library's dense bf16 GEMMs (torch's linear) of the
    same shapes, one matrix of `rows` rows (the local picks) against one expert's weights, no gather,
    no grouping, no SwiGLU; time per GEMM and fraction of the published bf16 peak."""
    import torch.nn.functional as F
    g = torch.Generator(device="cuda").manual_seed(11)
    out = {}
    for name, k, n in (("gate_up", H, 2 * I), ("down", I, H)):
        a = torch.randn(rows, k, device="cuda", dtype=torch.bfloat16, generator=g)
        w = torch.randn(n, k, device="cuda", dtype=torch.bfloat16, generator=g)
        for _ in range(3):
            c = F.linear(a, w)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            c = F.linear(a, w)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / reps
        out[f"{name}_us"] = round(us, 1)
        out[f"{name}_frac"] = round(2.0 * rows * k * n / (us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)
        del a, w, c
    flop = 2.0 * rows * H * 2 * I + 2.0 * rows * I * H
    out["both_frac"] = round(flop / ((out["gate_up_us"] + out["down_us"]) * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)
    out["rows"] = rows
    torch.cuda.empty_cache()
    return out


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


class Workload:
    """One workload on the GPU: inputs (nsets identical copies, so consecutive steps can read
    different buffers), workspace, output, and the layer forward through the C ABI."""

    def __init__(self, torch, m, cfg, d, nsets: int = 1, fp8: bool = False, mask_h=None, fused_combine=False):
        import numpy as np
        self.cfg, self.fp8, self.fused_combine = cfg, fp8, fused_combine
        self.P, self.R = algorithmic_units(cfg, d["topk_ids"], mask_h)
        self.L_rows = experts_with_rows(cfg, d["topk_ids"], mask_h)
        self.identity = cfg.intermediate == 0

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

        self.sets = []
        for _ in range(nsets):
            st = {"x": dev(d["hidden_states"]), "ids": torch.from_numpy(d["topk_ids"]).cuda(),
                  "w": torch.from_numpy(d["topk_weights"]).cuda(),
                  "w1": None if self.identity else dev(d["w_gate_up"]),
                  "w2": None if self.identity else dev(d["w_down"])}
            if fp8:
                L2I = cfg.num_local_experts * 2 * cfg.intermediate
                st["w1q"] = torch.empty((L2I, cfg.hidden), dtype=torch.uint8, device="cuda")
                st["w1s"] = torch.empty((L2I, m.moe_ep_fp8_scale_stride(cfg.hidden)), dtype=torch.uint8,
                                        device="cuda")
                m.moe_ep_quantize_fp8(st["w1"].view(L2I, cfg.hidden), st["w1q"], st["w1s"])
                st["w1"] = None
            self.sets.append(st)
        self.p = m.params(cfg.num_experts, cfg.num_local_experts, cfg.rank, cfg.max_tokens_per_rank, cfg.num_tokens,
                          cfg.hidden, cfg.intermediate, cfg.top_k, cfg.layout)
        self.ws = torch.zeros(m.moe_ep_workspace_size(self.p), dtype=torch.uint8, device="cuda")
        self.out = torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
        self.mask = None if mask_h is None else torch.from_numpy(mask_h).cuda()
        self.m = m
        torch.cuda.synchronize()

    def forward(self, evs, i: int = 0):
        st, m = self.sets[i % len(self.sets)], self.m
        if self.fp8:
            m.moe_ep_layer_forward_fp8(self.p, st["x"], st["ids"], st["w"], st["w1q"], st["w1s"], st["w2"], self.out,
                                       self.ws, events=evs, active_ranks=self.mask)
        elif self.fused_combine:
            m.moe_ep_layer_forward_fused_combine(self.p, st["x"], st["ids"], st["w"], st["w1"], st["w2"], self.out,
                                                 self.ws, events=evs, active_ranks=self.mask)
        else:
            m.moe_ep_layer_forward_timed(self.p, st["x"], st["ids"], st["w"], st["w1"], st["w2"], self.out, self.ws,
                                         evs, active_ranks=self.mask)


def flush_caches(scratch) -> None:
    """Evict L2 and the 256 MB Infinity Cache by reading a 1 GiB buffer (a read leaves no dirty
    lines whose write-back would overlap the next timed kernels, as a scratch write would)."""
    scratch.sum()


def recorded_events(torch, n: int):
    """n lists of 6 timing events, each recorded once (torch creates an event's HIP handle on its
    first record(); the library re-records the handles at the stage boundaries)."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(n)]
    for ev in evs:
        for e in ev:
            e.record()
    torch.cuda.synchronize()
    return evs


def stage_report(cfg, wl, events, fp8: bool = False) -> tuple[dict, dict | None]:
    """Per-stage times from the library's stage events (averaged over the steps), rates and roofline
    fractions: dispatch and combine against HBM, the GEMMs against their own bound."""
    import numpy as np

    def avg_ms(a: int, b: int) -> float:
        return float(np.mean([ev[a].elapsed_time(ev[b]) for ev in events]))

    layer_ms = np.array([ev[0].elapsed_time(ev[5]) for ev in events])
    t_dispatch, t_bridge, t_gate_up = avg_ms(0, 1), avg_ms(1, 2), avg_ms(2, 3)
    t_down, t_combine, t_layer = avg_ms(3, 4), avg_ms(4, 5), avg_ms(0, 5)
    P, R = wl.P, wl.R
    disp_bytes, comb_bytes = algorithmic_bytes(cfg, P, R, fp8)
    stages = {
        "layer_us": round(t_layer * 1e3, 2),
        "layer_us_median": round(float(np.median(layer_ms)) * 1e3, 2),
        "layer_us_min": round(float(layer_ms.min()) * 1e3, 2),
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
    }
    H, I = cfg.hidden, cfg.intermediate
    if wl.identity:
        achieved = (disp_bytes + comb_bytes) / ((t_dispatch + t_combine) * 1e-3) / 1e9
        return stages, {"kernel": "dispatch + combine", "bound": "hbm", "achieved": round(achieved, 1),
                        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                        "traffic": None}
    gemm_flops = 6.0 * P * I * H
    t_gemm = (t_gate_up + t_down) * 1e-3
    stages["gemm_TFLOPs"] = round(gemm_flops / t_gemm / 1e12, 1)
    # both GEMMs against their own peaks: the time they would take at peak / the time they took
    # (with FP8 the gate_up GEMM runs at the FP8 peak, the down GEMM at the bf16 one)
    gu_peak = FP8_MFMA_PEAK_TFLOPS if fp8 else BF16_MFMA_PEAK_TFLOPS
    t_peak = (4.0 * P * I * H / gu_peak + 2.0 * P * I * H / BF16_MFMA_PEAK_TFLOPS) / 1e12
    stages["gemm_mfma_frac"] = round(t_peak / t_gemm, 4)
    stages["down_gemm_roofline"] = down_roofline(cfg, P, wl.L_rows, t_down)
    roofline = gate_up_roofline(cfg, P, wl.L_rows, t_gate_up, fp8, measured_gate_up_traffic(cfg.name, fp8=fp8))
    return stages, roofline


def oracle_full_time_s(cfg, d) -> float:
    """Wall time of the single-threaded CPU oracle over every token of the workload."""
    import numpy as np
    import oracle
    p = oracle.params(cfg)
    ident = cfg.intermediate == 0
    t0 = time.perf_counter()
    oracle.forward_tokens(p, d["hidden_states"], d["topk_ids"], d["topk_weights"],
                          None if ident else d["w_gate_up"], None if ident else d["w_down"],
                          np.arange(cfg.num_tokens), threads=1)
    return time.perf_counter() - t0


def other_workload(torch, m, synth, name: str, steps: int, with_oracle: bool) -> dict:
    """A secondary workload's figures: stage times with the 256 MB Infinity Cache flushed before
    every step (a 1 GiB read outside the stage events), the same warm, the layer alone (no stage
    events inside it; tokens/s comes from this one), and (optionally) the single-threaded oracle over
    all of its tokens."""
    import numpy as np
    cfg = synth.get_config(name)
    d = synth.make_inputs(cfg)
    wl = Workload(torch, m, cfg, d)
    for _ in range(5):
        wl.forward([None] * 6)
    warm = recorded_events(torch, steps)
    for ev in warm:
        wl.forward(ev)
    torch.cuda.synchronize()
    scratch = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    cold = recorded_events(torch, steps)
    for ev in cold:
        flush_caches(scratch)
        wl.forward(ev)
    torch.cuda.synchronize()
    # the layer alone, timed by two events around it: each of the library's four stage events inside
    # the layer costs a few microseconds of GPU time, which matters on layers of a few hundred
    # microseconds
    plain = {}
    for flush in (True, False):
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        for a, b in pairs:
            a.record()
            b.record()
        torch.cuda.synchronize()
        for a, b in pairs:
            if flush:
                flush_caches(scratch)
            a.record()
            wl.forward([None] * 6)
            b.record()
        torch.cuda.synchronize()
        plain[flush] = float(np.median([a.elapsed_time(b) for a, b in pairs])) * 1e3
    del scratch
    stages, roofline = stage_report(cfg, wl, cold)
    warm_stages, _ = stage_report(cfg, wl, warm)
    stages["layer_us_median_no_stage_events"] = round(plain[True], 2)
    res = {"config": {"layout": cfg.layout, "num_tokens": cfg.num_tokens, "world": cfg.world,
                      "num_experts": cfg.num_experts, "num_local_experts": cfg.num_local_experts, "top_k": cfg.top_k,
                      "hidden": cfg.hidden, "intermediate": cfg.intermediate,
                      "routing": f"zipf({cfg.zipf_s})" if cfg.zipf_s else "uniform"},
           "timing": f"{steps} steps, Infinity Cache flushed before each (outside the timed events); tokens/s from "
                     "the layer timed without the stage events inside it",
           "tokens_per_s": round(cfg.num_tokens / (plain[True] * 1e-6), 1),
           "stages": stages, "gate_up_roofline" if not wl.identity else "roofline": roofline,
           "warm": {**{k: warm_stages[k] for k in ("layer_us_median", "dispatch_us", "bridge_us", "gate_up_gemm_us",
                                                  "down_gemm_us", "combine_us", "dispatch_combine_hbm_frac")},
                    "layer_us_median_no_stage_events": round(plain[False], 2)}}
    del wl
    torch.cuda.empty_cache()
    if with_oracle:
        res["oracle_single_thread_s"] = round(oracle_full_time_s(cfg, d), 3)
    log(f"{name}: layer {stages['layer_us_median']:.1f} us (cold), {warm_stages['layer_us_median']:.1f} us (warm); "
        f"without stage events {plain[True]:.1f} / {plain[False]:.1f} us")
    return res


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
    ap.add_argument("--no-others", action="store_true",
                    help="skip the secondary workloads (decode, rank-major, bandwidth) in the JSON line")
    ap.add_argument("--fp8", action="store_true",
                    help="FP8 dispatch + FP8 gate_up GEMM (moe_ep_layer_forward_fp8); W1 quantised once, untimed")
    ap.add_argument("--fused-combine", action="store_true",
                    help="the combine fused into the down GEMM (moe_ep_layer_forward_fused_combine; RANK_MAJOR / FLAT)")
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
    identity = cfg.intermediate == 0
    if args.fp8 and identity:
        log("--fp8 needs an expert GEMM (intermediate > 0)")
        return 2
    # two identical input / weight sets, used alternately, so that no step reads what the step
    # before it left in the caches
    wl = Workload(torch, m, cfg, d, nsets=2, fp8=args.fp8, mask_h=mask_h, fused_combine=args.fused_combine)
    P, R = wl.P, wl.R

    if args.warmup is None:
        t1 = time.perf_counter()
        wl.forward([None] * 6)
        torch.cuda.synchronize()
        one = max(time.perf_counter() - t1, 1e-6)
        args.warmup = max(5, int(np.ceil(0.25 / one)))
        done = 1
    else:
        done = 0
    for i in range(args.warmup - done):
        wl.forward([None] * 6, i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # the timed steps: the layer alone, with no stage events inside it
    t0 = time.perf_counter()
    for i in range(args.steps):
        wl.forward([None] * 6, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall * 1e3:.2f} ms")
    # the same steps again with the library's stage events, for the per-stage times
    events = recorded_events(torch, args.steps)
    for i in range(args.steps):
        wl.forward(events[i], i)
    torch.cuda.synchronize()
    if not torch.isfinite(wl.out.float()).all():
        log("non-finite values in the output")
        return 1
    # Cold-cache check, outside the timed steps: a few more layers, each after a 1 GiB read that
    # evicts the 256 MB Infinity Cache (and L2), timed by their own stage events.
    scratch = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    cold = recorded_events(torch, min(args.steps, 10))
    for ev in cold:
        flush_caches(scratch)
        wl.forward(ev)
    torch.cuda.synchronize()
    layer_cold_ms = float(np.median([ev[0].elapsed_time(ev[5]) for ev in cold]))
    del scratch
    copy_gbps = device_copy_gbps(torch)
    router_us, router_bytes = router_time_us(torch, m, cfg, args.steps)

    stages, roofline = stage_report(cfg, wl, events, args.fp8)
    stages["layer_us_cold_cache_median"] = round(layer_cold_ms * 1e3, 2)
    stages["context_device_copy_GBps"] = round(copy_gbps, 1)
    stages["router_us"] = round(router_us, 2)
    stages["router_GBps"] = round(router_bytes / (router_us * 1e-6) / 1e9, 1)
    H, I, N = cfg.hidden, cfg.intermediate, cfg.num_tokens
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
        **({"variant": "combine fused into the down GEMM (bf16 atomics)"} if args.fused_combine else {}),
        "data": "synthetic",
        "config": {"workload": cfg.name, "layout": cfg.layout, "num_tokens": N, "world": cfg.world,
                   "max_tokens_per_rank": cfg.max_tokens_per_rank, "num_experts": cfg.num_experts,
                   "num_local_experts": cfg.num_local_experts, "rank": cfg.rank, "top_k": cfg.top_k,
                   "hidden": H, "intermediate": I, "routing": f"zipf({cfg.zipf_s})" if cfg.zipf_s else "uniform",
                   "parallelism": "one GPU's expert-parallel share", "input_sets": 2,
                   **({"inactive_ranks": inactive} if inactive else {})},
        "stages": stages,
        "roofline": roofline,
    }
    rows_local = int(stages.get("local_picks", 0))
    del wl
    torch.cuda.empty_cache()
    if not args.fp8 and rows_local > 0 and I > 0:
        stages["context_vendor_dense_gemm"] = vendor_dense_gemm(torch, rows_local, H, I, args.steps)
    others = {}
    if (not args.no_others and not args.fp8 and not inactive and not args.fused_combine
            and cfg.name == "prefill_flat_zipf"):
        for name in ("decode_expert_major", "rank_major", "bandwidth_identity"):
            others[name] = other_workload(torch, m, synth, name, args.steps, with_oracle=not args.no_cpu_baseline)
        result["other_workloads"] = others
    if not args.no_cpu_baseline and not args.fp8:
        log("timing the CPU oracle on a token sample")
        cb = cpu_baseline(cfg, d, args.cpu_sample, mask_h)
        if others:
            tiny = synth.get_config("tiny_flat")
            full = {"tiny_flat": round(oracle_full_time_s(tiny, synth.make_inputs(tiny)), 4)}
            full.update({k: v["oracle_single_thread_s"] for k, v in others.items() if "oracle_single_thread_s" in v})
            cb["full_workloads_single_thread_s"] = full
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
