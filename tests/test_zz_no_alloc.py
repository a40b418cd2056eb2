"""The no-allocation fused forward (moe_ep_layer_forward_noalloc: for callers that cannot allocate
device memory) through the C ABI, against moe_ep_layer_forward on a workspace of the caller's.  Both
run the same kernels on the same inputs, so the outputs must agree bit for bit.  The static
workspace keeps each call's contents, so calls follow one another with different, smaller and
differently laid out inputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_topk_ids_amd as m
import synth
from gpu_harness import Case

pytestmark = pytest.mark.gpu


def _noalloc(c: Case) -> torch.Tensor:
    cfg = c.cfg
    out = torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    out.view(torch.int16).fill_(0x7FC0)   # a NaN pattern: every element must be written
    m.moe_ep_layer_forward_noalloc(c.p, c.x, c.ids, c.w, c.w1, c.w2, out, active_ranks=c.active)
    torch.cuda.synchronize()
    return out


def _edge(layout):
    from test_gpu_parity import _edge_inputs
    cfg = synth.Config("edge", layout, 16, 4, 2, 96, 4 * 96 - 37, 256, 192, 5)
    return cfg, _edge_inputs(cfg)


def test_noalloc_forward_matches_workspace_forward():
    cases = [(synth.get_config("rank_major"), None, None)]                 # 145 MiB of workspace
    cases += [(*_edge("FLAT"), None), (*_edge("EXPERT_MAJOR"), [1, 0, 1, 1])]  # then smaller ones
    cases += [(synth.get_config("tiny_flat"), None, None)]
    sizes = []
    for cfg, d, mask in cases:
        c = Case(cfg, d, active=mask)
        sizes.append(c.wsize)
        assert c.wsize <= m._lib.NOALLOC_WORKSPACE_BYTES
        got = _noalloc(c)
        ref = c.forward()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), cfg.name
        assert bool(torch.isfinite(ref.float()).all())
        # the same call again on the contents the previous one left
        assert torch.equal(_noalloc(c).view(torch.int16), ref.view(torch.int16)), cfg.name
        del c
    assert sizes[1] < sizes[0] and sizes[3] < sizes[2]


def test_noalloc_forward_rejects_a_layer_over_its_workspace():
    cfg = synth.get_config("decode_expert_major")     # 592 MiB of workspace
    p = m.params(cfg.num_experts, cfg.num_local_experts, cfg.rank, cfg.max_tokens_per_rank, cfg.num_tokens,
                 cfg.hidden, cfg.intermediate, cfg.top_k, cfg.layout)
    assert m.moe_ep_workspace_size(p) > m._lib.NOALLOC_WORKSPACE_BYTES
    out = torch.zeros((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MoeEpError) as e:
        m.moe_ep_layer_forward_noalloc(p, out, out, out, out, out, out)
    assert e.value.status == m._lib.EWORKSPACE
    torch.cuda.synchronize()
    assert int(out.view(torch.int16).abs().sum()) == 0
