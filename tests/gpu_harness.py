"""Helpers of the GPU parity tests: device copies of the synthetic inputs, the
three stages and the fused forward through the C ABI, views of the handle's
device arrays, and the comparison rules.

Comparison rules (the layer's stated bar): integers and copied rows bit-exact;
floating-point outputs with relative Frobenius error <= 1e-2 and max abs error
<= 3e-2 * max|ref| against the fp32 oracle, computed in float64.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import combine_topk_ids_amd as m
import oracle
import synth

THREADS = max(1, min(16, os.cpu_count() or 1))
REL_FRO = 1e-2
MAX_ABS = 3e-2


def dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def view(ws: torch.Tensor, ptr: int, count: int, dtype: torch.dtype) -> torch.Tensor:
    """Device tensor over `count` elements at device address ptr inside the workspace tensor."""
    off = ptr - ws.data_ptr()
    nb = count * torch.empty((), dtype=dtype).element_size()
    assert 0 <= off and off + nb <= ws.numel()
    return ws[off:off + nb].view(dtype)


def assert_close(got: np.ndarray, ref: np.ndarray, what: str) -> tuple[float, float]:
    """The bf16 bar over the whole tensor, accumulated in float64 a block of rows at a time (the
    largest outputs are 32768 x 7168)."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    g2 = got.reshape(got.shape[0], -1) if got.ndim > 1 else got.reshape(-1, 1)
    r2 = ref.reshape(ref.shape[0], -1) if ref.ndim > 1 else ref.reshape(-1, 1)
    num = den = 0.0
    mx = rmax = 0.0
    for i in range(0, g2.shape[0], 1024):
        g = g2[i:i + 1024].astype(np.float64)
        r = r2[i:i + 1024].astype(np.float64)
        assert np.all(np.isfinite(g)), what
        d = g - r
        num += float(np.sum(d * d))
        den += float(np.sum(r * r))
        if d.size:
            mx = max(mx, float(np.abs(d).max()))
            rmax = max(rmax, float(np.abs(r).max()))
    if den == 0:
        assert mx == 0, what
        return 0.0, 0.0
    rel = float(np.sqrt(num / den))
    lim = MAX_ABS * rmax
    assert rel <= REL_FRO, f"{what}: relative Frobenius error {rel:.3e} > {REL_FRO}"
    assert mx <= lim, f"{what}: max abs error {mx:.3e} > {lim:.3e}"
    return rel, mx


# Oracle outputs of every token of a workload, kept for the rest of the process: the largest
# workloads take the 16-thread oracle about a minute, and several tests compare against them.
_FULL_REF: dict = {}


def oracle_full(key, compute):
    """compute() once per key and process; the cached array is returned read-only."""
    if key not in _FULL_REF:
        ref = compute()
        ref.setflags(write=False)
        _FULL_REF[key] = ref
    return _FULL_REF[key]


class Case:
    """One configuration on the GPU: inputs, workspace, and the ABI calls."""

    def __init__(self, cfg, inputs: dict | None = None, identity: bool | None = None, active=None):
        """active: source-rank mask (int32 [W], 0 = skipped) given to dispatch, combine and the
        fused forward, or None."""
        self.cfg = cfg
        self.d = inputs if inputs is not None else synth.make_inputs(cfg)
        identity = cfg.intermediate == 0 if identity is None else identity
        self.p = m.params(cfg.num_experts, cfg.num_local_experts, cfg.rank, cfg.max_tokens_per_rank,
                          cfg.num_tokens, cfg.hidden, cfg.intermediate, cfg.top_k, cfg.layout)
        self.active_h = None if active is None else np.ascontiguousarray(active, dtype=np.int32)
        self.active = None if active is None else torch.from_numpy(self.active_h).cuda()
        self.op = oracle.params(cfg, active_ranks=self.active_h)
        self.x = dev_bf16(self.d["hidden_states"])
        self.ids = torch.from_numpy(np.ascontiguousarray(self.d["topk_ids"])).cuda()
        self.w = torch.from_numpy(np.ascontiguousarray(self.d["topk_weights"])).cuda()
        self.w1 = None if identity else dev_bf16(self.d["w_gate_up"])
        self.w2 = None if identity else dev_bf16(self.d["w_down"])
        self.wsize = m.moe_ep_workspace_size(self.p)
        assert self.wsize > 0
        self.ws = torch.zeros(self.wsize, dtype=torch.uint8, device="cuda")
        W, T, L, N, H = cfg.world, cfg.max_tokens_per_rank, cfg.num_local_experts, cfg.num_tokens, cfg.hidden
        self.cap = W * T
        self.rows = {"EXPERT_MAJOR": L * W * T, "RANK_MAJOR": W * T, "FLAT": N}[cfg.layout]
        self.h = None

    # -- ABI calls
    def dispatch(self):
        self.h = m.moe_ep_dispatch(self.p, self.x, self.ids, self.w, self.ws, active_ranks=self.active)
        return self.h

    def stages(self):
        cfg = self.cfg
        h = self.dispatch()
        eo = torch.zeros((self.rows, cfg.hidden), dtype=torch.bfloat16, device="cuda")
        m.moe_ep_expert_compute(self.p, h, self.w1, self.w2, eo)
        out = torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
        m.moe_ep_combine(self.p, h, eo, self.w, out, active_ranks=self.active)
        torch.cuda.synchronize()
        return eo, out

    def forward(self):
        cfg = self.cfg
        out = torch.empty((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
        m.moe_ep_layer_forward(self.p, self.x, self.ids, self.w, self.w1, self.w2, out, self.ws,
                               active_ranks=self.active)
        torch.cuda.synchronize()
        return out

    def status(self) -> int:
        return m.moe_ep_query_status(self.h)

    # -- handle arrays (device)
    def arr(self, name: str, count: int, dtype=torch.int32) -> torch.Tensor:
        ptr = getattr(self.h, name)
        assert ptr, name
        return view(self.ws, ptr, count, dtype)

    def recv_x(self) -> torch.Tensor:
        return view(self.ws, self.h.recv_x, self.rows * self.cfg.hidden, torch.bfloat16).view(self.rows,
                                                                                             self.cfg.hidden)

    # -- oracle
    def oracle_route(self):
        rc, r = oracle.route(self.op, self.d["topk_ids"], self.d["topk_weights"])
        assert rc == oracle.OK
        return r

    def oracle_out(self, tokens) -> np.ndarray:
        return oracle.forward_tokens(self.op, self.d["hidden_states"], self.d["topk_ids"], self.d["topk_weights"],
                                     None if self.w1 is None else self.d["w_gate_up"],
                                     None if self.w2 is None else self.d["w_down"], tokens, threads=THREADS)

    def oracle_out_all(self, key=None) -> np.ndarray:
        """The oracle's output for every token; with a key (for the synthetic inputs of a named
        workload without a mask) it is computed once per process and shared between tests."""
        if key is None:
            return self.oracle_out(np.arange(self.cfg.num_tokens))
        return oracle_full(key, lambda: self.oracle_out(np.arange(self.cfg.num_tokens)))


def sample_tokens(n: int, k: int, seed: int = 0) -> np.ndarray:
    if n <= k:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    s = set(rng.choice(n, size=k - 2, replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(s))
