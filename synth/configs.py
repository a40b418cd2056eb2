"""Workload configurations of the MoE expert-parallel layer (one GPU's share).

Each entry names a workload by what it is.  Sizes follow the layer's geometry
(FlashInfer "MoE-EP implementation & usage", section 1 FleetParams and section
3 layout contracts): world W simulated source ranks of T = max_tokens_per_rank
tokens each, E global experts of which this GPU owns L = E / W starting at
rank * L, top_k picks per token, hidden H, expert intermediate I.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

LAYOUTS = {"EXPERT_MAJOR": 0, "RANK_MAJOR": 1, "FLAT": 2}


@dataclass(frozen=True)
class Config:
    name: str
    layout: str
    num_experts: int
    num_local_experts: int
    rank: int
    max_tokens_per_rank: int
    num_tokens: int
    hidden: int
    intermediate: int          # 0 = identity expert (no GEMM)
    top_k: int
    zipf_s: float = 0.0        # 0 = uniform routing

    @property
    def world(self) -> int:
        return self.num_experts // self.num_local_experts

    @property
    def layout_id(self) -> int:
        return LAYOUTS[self.layout]

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    # 64 tokens, 8 experts all local, top-2, FLAT
    "tiny_flat": Config("tiny_flat", "FLAT", 8, 8, 0, 64, 64, 128, 256, 2),
    # low-latency decode: world 8 x 128 tokens, 256 experts (32 local), top-8
    "decode_expert_major": Config("decode_expert_major", "EXPERT_MAJOR", 256, 32, 0, 128, 1024, 7168, 2048, 8),
    # rank-major: world 8 x 256 tokens, 64 experts (8 local), top-6, I=1408
    "rank_major": Config("rank_major", "RANK_MAJOR", 64, 8, 0, 256, 2048, 4096, 1408, 6),
    # high-throughput prefill: world 8 x 4096 tokens, 256 experts (32 local), top-8, Zipf(1.1)
    "prefill_flat_zipf": Config("prefill_flat_zipf", "FLAT", 256, 32, 0, 4096, 32768, 7168, 2048, 8, 1.1),
    # dispatch + combine bandwidth: 16384 tokens, 256 experts all local, top-8, identity expert
    "bandwidth_identity": Config("bandwidth_identity", "EXPERT_MAJOR", 256, 256, 0, 16384, 16384, 7168, 0, 8),
}

# Parity-only cases: the FlashInfer walkthrough's own test shape (section 4:
# E=16, top_k=8, 128 tok/rank, H=8192, I=2048, world=8) in both low-latency
# layouts, and ranks with a nonzero local-expert offset (the section 5 bug class).
EXTRA_CASES = {
    "walkthrough_expert_major": Config("walkthrough_expert_major", "EXPERT_MAJOR", 16, 2, 0, 128, 1024, 8192, 2048, 8),
    "walkthrough_rank_major": Config("walkthrough_rank_major", "RANK_MAJOR", 16, 2, 0, 128, 1024, 8192, 2048, 8),
    "walkthrough_rank_major_r5": Config("walkthrough_rank_major_r5", "RANK_MAJOR", 16, 2, 5, 128, 1024, 8192, 2048, 8),
    "decode_expert_major_r3": Config("decode_expert_major_r3", "EXPERT_MAJOR", 256, 32, 3, 128, 1024, 7168, 2048, 8),
    "rank_major_r5": Config("rank_major_r5", "RANK_MAJOR", 64, 8, 5, 256, 2048, 4096, 1408, 6),
    "prefill_flat_zipf_r3": Config("prefill_flat_zipf_r3", "FLAT", 256, 32, 3, 4096, 32768, 7168, 2048, 8, 1.1),
}


def get_config(name: str) -> Config:
    if name in CONFIGS:
        return CONFIGS[name]
    return EXTRA_CASES[name]
