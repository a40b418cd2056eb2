"""GPU parity of the FP8 path against the CPU oracle.

Format (Mooncake PG/EP guide, "Buffer.dispatch": use_fp8 returns FP8 data plus scales; reading in
the oracle): OCP E4M3 codes of v * 2^-k and one scale byte k + 127 per 128 values of a row, k the
smallest integer with amax <= 448 * 2^k.  Codes and scales are integers decided by exact
arithmetic on both sides, so they must match bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import combine_topk_ids_amd as m
import oracle
import synth
from gpu_harness import dev_bf16

pytestmark = pytest.mark.gpu


def _rows(n, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (n, cols)) * np.ldexp(1.0, rng.integers(-30, 30, (n, 1)))
    x = x.astype(np.float32)
    if n > 2 and cols >= 256:
        x[1, :128] = 0.0                                  # an all-zero block
        x[2, :128] = -0.0
        table = np.array([oracle.e4m3_decode(c) for c in range(0x7F)], np.float64)
        mids = (table[1:] + table[:-1]) / 2               # exact ties of the encoder
        x[2, 128:256] = np.resize(mids, 128) * np.sign(rng.normal(size=128))
        x[2, 128] = 448.0                                 # keeps that block's scale at 2^0
    return synth.f32_to_bf16(x)


@pytest.mark.parametrize("n,cols", [(4, 128), (300, 7168), (1000, 2048), (33, 640)])
def test_quantize_fp8_matches_oracle(n, cols):
    xb = _rows(n, cols, seed=n + cols)
    rc, rq, rs = oracle.quantize_rows_fp8(xb)
    assert rc == oracle.OK
    stride = m.moe_ep_fp8_scale_stride(cols)
    q = torch.full((n, cols), 0x55, dtype=torch.uint8, device="cuda")
    s = torch.full((n, stride), 0x55, dtype=torch.uint8, device="cuda")
    m.moe_ep_quantize_fp8(dev_bf16(xb), q, s)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), rq)
    sc = s.cpu().numpy()
    assert np.array_equal(sc[:, :cols // 128], rs[:, :cols // 128])
    assert np.all(sc[:, cols // 128:] == 0)


def _fp8_case(cfg, inputs=None):
    """Device inputs, W1 quantised on the GPU (checked against the oracle), and the oracle inputs:
    hidden_states and W1 quantised then dequantised (exact in bf16)."""
    from gpu_harness import Case
    c = Case(cfg, inputs)
    L, I, H = cfg.num_local_experts, cfg.intermediate, cfg.hidden
    w1 = c.w1.view(L * 2 * I, H)
    stride = m.moe_ep_fp8_scale_stride(H)
    wq = torch.empty((L * 2 * I, H), dtype=torch.uint8, device="cuda")
    wsc = torch.empty((L * 2 * I, stride), dtype=torch.uint8, device="cuda")
    m.moe_ep_quantize_fp8(w1, wq, wsc)
    torch.cuda.synchronize()
    rc, rq, rs = oracle.quantize_rows_fp8(c.d["w_gate_up"].reshape(L * 2 * I, H))
    assert rc == oracle.OK
    assert np.array_equal(wq.cpu().numpy(), rq) and np.array_equal(wsc.cpu().numpy()[:, :H // 128], rs)
    w1_hat = synth.f32_to_bf16(oracle.dequantize_rows_fp8(rq, rs)).reshape(L, 2 * I, H)
    rc, xq, xs = oracle.quantize_rows_fp8(c.d["hidden_states"])
    assert rc == oracle.OK
    x_hat = synth.f32_to_bf16(oracle.dequantize_rows_fp8(xq, xs))
    return c, wq, wsc, x_hat, w1_hat


def _fp8_forward(c, wq, wsc):
    cfg = c.cfg
    out = torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    m.moe_ep_layer_forward_fp8(c.p, c.x, c.ids, c.w, wq, wsc, c.w2, out, c.ws)
    torch.cuda.synchronize()
    return out


def _edge(layout):
    from test_gpu_parity import _edge_inputs
    cfg = synth.Config("edge", layout, 16, 4, 2, 96, 4 * 96 - 37, 256, 192, 5)
    return cfg, _edge_inputs(cfg)


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
def test_fp8_forward_edge_shapes(layout):
    from gpu_harness import assert_close, host_f32
    cfg, d = _edge(layout)
    c, wq, wsc, x_hat, w1_hat = _fp8_case(cfg, d)
    out = _fp8_forward(c, wq, wsc)
    toks = np.arange(cfg.num_tokens)
    ref = oracle.forward_tokens(c.op, x_hat, c.d["topk_ids"], c.d["topk_weights"], w1_hat, c.d["w_down"], toks)
    assert_close(host_f32(out), ref, f"fp8 {layout}")
    # the FP8 forward is a different (coarser) computation than the bf16 one, but close to it
    ref_bf16 = c.oracle_out(toks)
    rel = np.linalg.norm(host_f32(out) - ref_bf16) / np.linalg.norm(ref_bf16)
    assert rel < 0.1, rel


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
def test_fp8_forward_single_row_h128(layout):
    # One receive row of H = 128 in every layout: its 128 code bytes are followed, 256-byte aligned,
    # by its scale, which lies past the 2 * H bytes a bf16 row would take.  I = 256 gives the FP8
    # gate_up GEMM two column blocks of that row, so a scale placed where another stage writes
    # would be read while it is overwritten.
    from gpu_harness import assert_close, host_f32
    cfg = synth.Config("one_row", layout, 1, 1, 0, 1, 1, 128, 256, 1)
    c, wq, wsc, x_hat, w1_hat = _fp8_case(cfg)
    for _ in range(3):
        out = _fp8_forward(c, wq, wsc)
        ref = oracle.forward_tokens(c.op, x_hat, c.d["topk_ids"], c.d["topk_weights"], w1_hat, c.d["w_down"],
                                    np.arange(1))
        assert_close(host_f32(out), ref, f"fp8 one row {layout}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_flat", "rank_major", "decode_expert_major", "prefill_flat_zipf"])
def test_fp8_forward_workloads(name):
    from gpu_harness import THREADS, assert_close, host_f32
    cfg = synth.get_config(name)
    c, wq, wsc, x_hat, w1_hat = _fp8_case(cfg)
    out = _fp8_forward(c, wq, wsc)
    # every token (the prefill workload takes the 16-thread oracle about a minute)
    toks = np.arange(cfg.num_tokens)
    ref = oracle.forward_tokens(c.op, x_hat, c.d["topk_ids"], c.d["topk_weights"], w1_hat, c.d["w_down"], toks,
                                threads=THREADS)
    rel, mx = assert_close(host_f32(out), ref, f"fp8 {name}")
    print(f"[fp8 {name}] rel_fro={rel:.2e} max_abs={mx:.2e}", flush=True)
    # deterministic: a second run gives the same bits
    assert torch.equal(out.view(torch.int16), _fp8_forward(c, wq, wsc).view(torch.int16))
