"""ctypes wrapper of the CPU oracle (liboracle.so, built from moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg.  The GPU library never imports it, and it
imports nothing of the GPU library.  The oracle functions are single
threaded; ctypes releases the GIL during each call, so the callers here may
run independent calls on disjoint token sets in parallel threads.
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

OK, EINVAL, EEXPERT_ID, ECAPACITY = 0, 1, 2, 3
LAYOUTS = {"EXPERT_MAJOR": 0, "RANK_MAJOR": 1, "FLAT": 2}


class Params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_experts", "num_local_experts", "rank", "max_tokens_per_rank", "num_tokens",
        "hidden", "intermediate", "top_k", "layout")] + [("active_ranks", ctypes.c_void_p)]


class _Route(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "recv_count", "expert_offsets", "slot_of", "src_info", "layout_range", "recv_topk_idx",
        "recv_topk_weights", "row_of_token", "recv_src_idx", "num_recv")]


class _Bridge(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "pick_count", "pick_offsets", "perm", "pick_slot", "topk_gid", "topk_wmask")]


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            from .build import build
            build()
        lib = ctypes.CDLL(path)
        P, vp, i32 = ctypes.POINTER(Params), ctypes.c_void_p, ctypes.c_int32
        lib.orc_recv_rows.argtypes = [P]
        lib.orc_recv_rows.restype = ctypes.c_int64
        lib.orc_check_params.argtypes = [P]
        lib.orc_route.argtypes = [P, vp, vp, ctypes.POINTER(_Route)]
        lib.orc_bridge.argtypes = [P, i32, vp, vp, ctypes.POINTER(_Bridge)]
        lib.orc_expert_ffn.argtypes = [i32, i32, vp, vp, vp, vp, vp]
        lib.orc_expert_ffn.restype = None
        lib.orc_forward_tokens.argtypes = [P, vp, vp, vp, vp, vp, i32, vp, vp]
        lib.orc_recv_rows_z.argtypes = [P, vp, vp, vp, vp, vp, i32, vp, vp]
        lib.orc_router_topk.argtypes = [i32, i32, i32, vp, vp, vp]
        lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_decode.restype = ctypes.c_float
        lib.orc_quantize_rows_fp8.argtypes = [ctypes.c_int64, i32, vp, vp, vp]
        lib.orc_quantize_rows_fp8.restype = ctypes.c_int
        for f in (lib.orc_check_params, lib.orc_route, lib.orc_bridge, lib.orc_forward_tokens,
                  lib.orc_recv_rows_z, lib.orc_router_topk):
            f.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def params(cfg=None, active_ranks=None, **kw) -> Params:
    """Params from a synth Config (or keywords with the same field names).  active_ranks: an
    int32 [W] mask (0 = source rank skipped) or None; the returned Params keeps it alive."""
    d = {}
    if cfg is not None:
        d = dict(num_experts=cfg.num_experts, num_local_experts=cfg.num_local_experts, rank=cfg.rank,
                 max_tokens_per_rank=cfg.max_tokens_per_rank, num_tokens=cfg.num_tokens, hidden=cfg.hidden,
                 intermediate=cfg.intermediate, top_k=cfg.top_k, layout=LAYOUTS[cfg.layout])
    d.update(kw)
    if isinstance(d.get("layout"), str):
        d["layout"] = LAYOUTS[d["layout"]]
    mask = None if active_ranks is None else np.ascontiguousarray(active_ranks, dtype=np.int32)
    p = Params(**d, active_ranks=None if mask is None else mask.ctypes.data)
    p._mask = mask
    return p


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def check_params(p: Params) -> int:
    return _lib().orc_check_params(ctypes.byref(p))


def route(p: Params, topk_ids: np.ndarray, topk_weights: np.ndarray):
    """Dispatch routing integers.  Returns (status, dict of arrays)."""
    ids = _c(topk_ids, np.int64)
    w = _c(topk_weights, np.float32)
    L, K, N, E, T = p.num_local_experts, p.top_k, p.num_tokens, p.num_experts, p.max_tokens_per_rank
    W = E // L
    cap = W * T
    out = {"recv_count": np.zeros(L, np.int32), "expert_offsets": np.zeros(L + 1, np.int32)}
    if p.layout == 0:
        out.update(slot_of=np.zeros(N * K, np.int32), src_info=np.zeros(L * cap, np.int32),
                   layout_range=np.zeros(L * W * 2, np.int32))
    else:
        rows = W * T if p.layout == 1 else N
        out.update(recv_topk_idx=np.zeros(rows * K, np.int32), recv_topk_weights=np.zeros(rows * K, np.float32),
                   row_of_token=np.zeros(N, np.int32))
        if p.layout == 2:
            out.update(recv_src_idx=np.zeros(N, np.int32), num_recv=np.zeros(1, np.int32))
    r = _Route(**{k: _p(v) for k, v in out.items()})
    rc = _lib().orc_route(ctypes.byref(p), _p(ids), _p(w), ctypes.byref(r))
    return rc, out


def bridge(p: Params, rows: int, recv_topk_idx: np.ndarray, recv_topk_weights: np.ndarray):
    """Compute-side bridge over `rows` received rows.  Returns (status, dict of arrays)."""
    idx = _c(recv_topk_idx, np.int32)
    w = _c(recv_topk_weights, np.float32)
    L, K = p.num_local_experts, p.top_k
    out = {"pick_count": np.zeros(L, np.int32), "pick_offsets": np.zeros(L + 1, np.int32),
           "perm": np.zeros(max(rows * K, 1), np.int32), "pick_slot": np.zeros(rows * K, np.int32),
           "topk_gid": np.zeros(rows * K, np.int32), "topk_wmask": np.zeros(rows * K, np.float32)}
    b = _Bridge(**{k: _p(v) for k, v in out.items()})
    rc = _lib().orc_bridge(ctypes.byref(p), rows, _p(idx), _p(w), ctypes.byref(b))
    if rc == OK:
        out["perm"] = out["perm"][: int(out["pick_offsets"][-1])]
    return rc, out


def expert_ffn(x_row: np.ndarray, w_gate_up_e, w_down_e, H: int, I: int) -> np.ndarray:
    x = _c(x_row, np.uint16)
    w1, w2 = _c(w_gate_up_e, np.uint16), _c(w_down_e, np.uint16)
    y = np.zeros(H, np.float32)
    a = np.zeros(max(I, 1), np.float32)
    _lib().orc_expert_ffn(H, I, _p(x), _p(w1), _p(w2), _p(y), _p(a))
    return y


def _split(items: np.ndarray, threads: int):
    threads = max(1, min(threads, len(items)))
    return [c for c in np.array_split(items, threads) if len(c)]


def forward_tokens(p: Params, x, topk_ids, topk_weights, w_gate_up, w_down, tokens, threads: int = 1):
    """fp32 [len(tokens), H] layer outputs.  threads > 1 runs independent single-threaded calls
    on disjoint token subsets (results are identical: tokens are independent)."""
    x, ids, w = _c(x, np.uint16), _c(topk_ids, np.int64), _c(topk_weights, np.float32)
    w1, w2 = _c(w_gate_up, np.uint16), _c(w_down, np.uint16)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    out = np.zeros((len(tokens), p.hidden), np.float32)
    chunks = _split(np.arange(len(tokens)), threads)

    def run(ix):
        sub = np.ascontiguousarray(tokens[ix])
        o = np.zeros((len(ix), p.hidden), np.float32)
        rc = _lib().orc_forward_tokens(ctypes.byref(p), _p(x), _p(ids), _p(w), _p(w1), _p(w2), len(sub),
                                       _p(sub), _p(o))
        out[ix] = o
        return rc

    if len(chunks) <= 1:
        rcs = [run(c) for c in chunks]
    else:
        with ThreadPoolExecutor(len(chunks)) as ex:
            rcs = list(ex.map(run, chunks))
    bad = [r for r in rcs if r != OK]
    if bad:
        raise RuntimeError(f"oracle forward failed with status {bad[0]}")
    return out


def recv_rows_z(p: Params, recv_x, recv_topk_idx, recv_topk_weights, w_gate_up, w_down, rows, threads: int = 1):
    """fp32 [len(rows), H] RANK_MAJOR/FLAT expert-stage values of the listed received rows."""
    rx, idx, w = _c(recv_x, np.uint16), _c(recv_topk_idx, np.int32), _c(recv_topk_weights, np.float32)
    w1, w2 = _c(w_gate_up, np.uint16), _c(w_down, np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    out = np.zeros((len(rows), p.hidden), np.float32)
    chunks = _split(np.arange(len(rows)), threads)

    def run(ix):
        sub = np.ascontiguousarray(rows[ix])
        o = np.zeros((len(ix), p.hidden), np.float32)
        rc = _lib().orc_recv_rows_z(ctypes.byref(p), _p(rx), _p(idx), _p(w), _p(w1), _p(w2), len(sub),
                                    _p(sub), _p(o))
        out[ix] = o
        return rc

    if len(chunks) <= 1:
        rcs = [run(c) for c in chunks]
    else:
        with ThreadPoolExecutor(len(chunks)) as ex:
            rcs = list(ex.map(run, chunks))
    bad = [r for r in rcs if r != OK]
    if bad:
        raise RuntimeError(f"oracle recv_rows_z failed with status {bad[0]}")
    return out


def router_topk(scores: np.ndarray, top_k: int):
    """Router: (status, topk_ids int64 [N, K], topk_weights fp32 [N, K]) from fp32 scores [N, E]."""
    sc = np.ascontiguousarray(scores, dtype=np.float32)
    N, E = sc.shape
    ids = np.zeros((N, top_k), np.int64)
    w = np.zeros((N, top_k), np.float32)
    rc = _lib().orc_router_topk(N, E, top_k, _p(sc), _p(ids), _p(w))
    return rc, ids, w


def e4m3_encode(v: float) -> int:
    return int(_lib().orc_e4m3_encode(float(v)))


def e4m3_decode(code: int) -> float:
    return float(_lib().orc_e4m3_decode(int(code)))


def quantize_rows_fp8(x: np.ndarray):
    """bf16 bits [n, cols] -> (status, e4m3 codes uint8 [n, cols], scale bytes uint8 [n, cols/128])."""
    xs = np.ascontiguousarray(x, dtype=np.uint16)
    n, cols = xs.shape
    codes = np.zeros((n, cols), np.uint8)
    scales = np.zeros((n, max(cols // 128, 1)), np.uint8)
    rc = _lib().orc_quantize_rows_fp8(n, cols, _p(xs), _p(codes), _p(scales))
    return rc, codes, scales


def dequantize_rows_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp32 values code * 2^(scale - 127), from the oracle's own decoder (one table of 256)."""
    table = np.array([e4m3_decode(c) for c in range(256)], np.float32)
    n, cols = codes.shape
    k = scales.astype(np.int32) - 127
    return (table[codes].reshape(n, cols // 128, 128) * np.ldexp(np.float32(1), k)[:, :, None]).reshape(n, cols)
