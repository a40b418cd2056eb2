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
