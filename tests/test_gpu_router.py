"""GPU parity of the router (top_k of expert scores, softmax over the selection) against the CPU
oracle, and the router feeding the layer.

Source: Mooncake PG/EP guide quick start (topk_idx = the top_k of per-token scores, softmax
topk_weights); FlashInfer "MoE-EP implementation & usage" section 4 step 2.  Expert ids are
compared bit for bit (equal scores go to the lower id on both sides, so the answer is unique);
weights are fp32 on the GPU against the oracle's double-precision softmax rounded to fp32.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_topk_ids_amd as m
import oracle
import synth
from gpu_harness import Case, assert_close, host_f32

pytestmark = pytest.mark.gpu
W_RTOL, W_ATOL = 1e-5, 1e-9


def _scores(N, E, kind, seed):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((N, E)).astype(np.float32)
    if kind == "ties":
        s = np.round(s * 2).astype(np.float32)            # many exact ties
    elif kind == "special":
        s[rng.random(s.shape) < 0.2] = -np.inf            # unusable experts
        z = rng.random(s.shape) < 0.2
        s[z] = np.where(rng.random(z.sum()) < 0.5, np.float32(0.0), np.float32(-0.0))  # signed zeros tie
    return s


def _run(s, K):
    N, E = s.shape
    sd = torch.from_numpy(s).cuda()
    ids = torch.full((N, K), -7, dtype=torch.int64, device="cuda")
    w = torch.full((N, K), -7.0, dtype=torch.float32, device="cuda")
    m.moe_ep_router_topk(sd, K, ids, w)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("N,E,K", [(64, 8, 2), (347, 16, 5), (2048, 64, 6), (32768, 256, 8), (1000, 1000, 10),
                                   (513, 1024, 64), (100, 6, 6), (77, 65, 3)])
@pytest.mark.parametrize("kind", ["normal", "ties", "special"])
def test_router_parity(N, E, K, kind):
    s = _scores(N, E, kind, seed=N * 7 + E)
    ids, w = _run(s, K)
    rc, rids, rw = oracle.router_topk(s, K)
    assert rc == oracle.OK
    assert np.array_equal(ids, rids), f"{np.argwhere(ids != rids)[:5]}"
    np.testing.assert_allclose(w, rw, rtol=W_RTOL, atol=W_ATOL)


def test_router_zero_tokens():
    ids = torch.empty((0, 4), dtype=torch.int64, device="cuda")
    w = torch.empty((0, 4), dtype=torch.float32, device="cuda")
    m.moe_ep_router_topk(torch.empty((0, 32), dtype=torch.float32, device="cuda"), 4, ids, w)
    torch.cuda.synchronize()


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "FLAT"])
def test_router_feeds_the_layer(layout):
    # scores -> router -> fused layer forward on the GPU, against router -> forward in the oracle
    cfg = synth.Config("routed", layout, 32, 8, 1, 64, 4 * 64 - 9, 256, 128, 4)
    d = synth.make_inputs(cfg)
    s = _scores(cfg.num_tokens, cfg.num_experts, "normal", seed=5)
    ids, w = _run(s, cfg.top_k)
    rc, rids, rw = oracle.router_topk(s, cfg.top_k)
    assert rc == oracle.OK and np.array_equal(ids, rids)
    d["topk_ids"], d["topk_weights"] = rids, rw
    c = Case(cfg, d)
    c.ids = torch.from_numpy(ids).cuda()          # the router's own device outputs drive the layer
    c.w = torch.from_numpy(w).cuda()
    out = c.forward()
    assert_close(host_f32(out), c.oracle_out(np.arange(cfg.num_tokens)), f"routed {layout}")
