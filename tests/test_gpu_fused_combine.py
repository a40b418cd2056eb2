"""GPU parity of the layer forward with the combine fused into the down GEMM (zero-copy combine:
Mooncake PG/EP guide, "Buffer.get_next_combine_buffer" / combine with zero_copy).  The down GEMM adds
each pick's weighted output into the token-major output with bf16 atomics in no fixed order, so the
result is compared with the oracle at the layer's float tolerance (not bit for bit with the other
forward); tokens without a local pick, and every token of an inactive source rank, must be exactly 0."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_topk_ids_amd as m
import synth
from gpu_harness import Case, assert_close, host_f32
from test_gpu_parity import SHARED_REF, _edge_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _fused(c: Case) -> torch.Tensor:
    cfg = c.cfg
    out = torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    out.view(torch.int16).fill_(0x7FC0)   # a NaN pattern: every element must be written
    m.moe_ep_layer_forward_fused_combine(c.p, c.x, c.ids, c.w, c.w1, c.w2, out, c.ws, active_ranks=c.active)
    torch.cuda.synchronize()
    return out


def _case(name, mask=None):
    if name.startswith("edge_"):
        cfg = synth.Config("edge", name[5:], 16, 4, 2, 96, 4 * 96 - 37, 256, 192, 5)
        return Case(cfg, _edge_inputs(cfg), active=mask)
    if name.startswith("many_items_"):
        cfg = synth.Config("many_items", name[11:], 8, 8, 0, 16384, 16384, 512, 2048, 2, 1.1)
        return Case(cfg, active=mask)
    return Case(synth.get_config(name), active=mask)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_flat", "rank_major", "rank_major_r5", "walkthrough_rank_major",
                                  "edge_RANK_MAJOR", "edge_FLAT", "many_items_FLAT", "many_items_RANK_MAJOR",
                                  "prefill_flat_zipf"])
def test_fused_combine_forward(name):
    c = _case(name)
    out = _fused(c)
    cfg = c.cfg
    if name in SHARED_REF:
        ref = c.oracle_out_all(key=(cfg, "synth"))
    else:
        ref = c.oracle_out_all()
    got = host_f32(out)
    rel, mx = assert_close(got, ref, f"fused combine {name}")
    assert np.all(got[np.all(ref == 0, axis=1)] == 0)
    print(f"[fused combine {name}] rel_fro={rel:.2e} max_abs={mx:.2e}", flush=True)
    # the same against the forward with the separate combine, at the same tolerance
    assert_close(got, host_f32(c.forward()), f"fused vs separate combine {name}")


@pytest.mark.parametrize("layout", ["RANK_MAJOR", "FLAT"])
def test_fused_combine_masked_rank(layout):
    c = _case(f"edge_{layout}", mask=[1, 0, 1, 1])
    got = host_f32(_fused(c))
    assert_close(got, c.oracle_out_all(), f"fused combine masked {layout}")
    T = c.cfg.max_tokens_per_rank
    assert np.all(got[T:2 * T] == 0)


def test_fused_combine_rejects_expert_major_and_identity():
    c = _case("edge_EXPERT_MAJOR")
    out = torch.zeros((c.cfg.num_tokens, c.cfg.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MoeEpError) as e:
        m.moe_ep_layer_forward_fused_combine(c.p, c.x, c.ids, c.w, c.w1, c.w2, out, c.ws)
    assert e.value.status == m._lib.EUNSUPPORTED
    cfg = synth.Config("ident", "FLAT", 8, 8, 0, 64, 64, 256, 0, 3)
    ci = Case(cfg)
    with pytest.raises(m.MoeEpError) as e:
        m.moe_ep_layer_forward_fused_combine(ci.p, ci.x, ci.ids, ci.w, None, None, out, ci.ws)
    assert e.value.status == m._lib.EUNSUPPORTED
