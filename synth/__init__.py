"""Seeded synthetic inputs for the MoE expert-parallel layer.

Holds random-number generation only (no dispatch, GEMM or combine
arithmetic): both the CPU oracle and the GPU library read the arrays made
here.  The generator is counter-based SplitMix64 (Steele, Lea & Flood,
OOPSLA 2014) written in C (``synth.c``); see that file for the exact
definitions.  Arrays use numpy; bf16 tensors are stored as their uint16 bit
patterns.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .configs import CONFIGS, EXTRA_CASES, Config, get_config  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

TAG_X, TAG_SCORE, TAG_LOGIT, TAG_W_GATE_UP, TAG_W_DOWN = 1, 2, 3, 4, 5
WEIGHT_SEED = 2024          # FlashInfer walkthrough, step 1: torch.Generator.manual_seed(2024)
TOKEN_SEED_BASE = 1000      # FlashInfer walkthrough, step 2: manual_seed(1000 + rank)


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            from .build import build
            build()
        lib = ctypes.CDLL(path)
        u64, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_double, ctypes.c_void_p)
        lib.synth_key.argtypes = [u64, u64]
        lib.synth_key.restype = u64
        lib.synth_normal_bf16.argtypes = [u64, u64, u64, i64, dbl, vp]
        lib.synth_normal_f32.argtypes = [u64, u64, u64, i64, dbl, vp]
        lib.synth_raw.argtypes = [u64, u64, u64, i64, vp]
        lib.synth_raw_key.argtypes = [u64, u64, i64, vp]
        lib.synth_tokens_bf16.argtypes = [u64, i32, i32, i32, vp]
        lib.synth_routing.argtypes = [u64, i32, i32, i32, i32, dbl, vp, vp]
        for f in (lib.synth_normal_bf16, lib.synth_normal_f32, lib.synth_raw, lib.synth_raw_key,
                  lib.synth_tokens_bf16, lib.synth_routing):
            f.restype = None
        _LIB = lib
    return _LIB


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def raw(seed: int, tag: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint64)
    _lib().synth_raw(seed, tag, start, count, _ptr(out))
    return out


def raw_key(key: int, start: int, count: int) -> np.ndarray:
    """Outputs start.. of a SplitMix64 generator whose state starts at `key`."""
    out = np.empty(count, dtype=np.uint64)
    _lib().synth_raw_key(key, start, count, _ptr(out))
    return out


def normal_bf16(seed: int, tag: int, start: int, count: int, std: float = 1.0) -> np.ndarray:
    out = np.empty(count, dtype=np.uint16)
    _lib().synth_normal_bf16(seed, tag, start, count, float(std), _ptr(out))
    return out


def normal_f32(seed: int, tag: int, start: int, count: int, std: float = 1.0) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    _lib().synth_normal_f32(seed, tag, start, count, float(std), _ptr(out))
    return out


def tokens(T: int, N: int, H: int, seed_base: int = TOKEN_SEED_BASE) -> np.ndarray:
    """hidden_states bf16 bits [N, H]; token t is row t % T of source rank t // T."""
    x = np.empty((N, H), dtype=np.uint16)
    _lib().synth_tokens_bf16(seed_base, T, N, H, _ptr(x))
    return x


def routing(T: int, N: int, E: int, K: int, zipf_s: float = 0.0, seed_base: int = TOKEN_SEED_BASE):
    """(topk_ids int64 [N, K], topk_weights fp32 [N, K]); K distinct experts per token."""
    if not (1 <= K <= min(E, 64)):
        raise ValueError("routing needs 1 <= top_k <= min(num_experts, 64)")
    ids = np.empty((N, K), dtype=np.int64)
    w = np.empty((N, K), dtype=np.float32)
    _lib().synth_routing(seed_base, T, N, E, K, float(zipf_s), _ptr(ids), _ptr(w))
    return ids, w


def expert_weights(E: int, L: int, rank: int, H: int, I: int, seed: int = WEIGHT_SEED):
    """Local slice of the full weight set: (w_gate_up [L, 2I, H], w_down [L, H, I]) as bf16 bits.

    The full set is w_gate_up [E, 2I, H] with std 1/sqrt(H) and w_down [E, H, I]
    with std 1/sqrt(I); only experts [rank*L, rank*L + L) are materialised.
    """
    o = rank * L
    w1 = normal_bf16(seed, TAG_W_GATE_UP, o * 2 * I * H, L * 2 * I * H, 1.0 / np.sqrt(H)).reshape(L, 2 * I, H)
    w2 = normal_bf16(seed, TAG_W_DOWN, o * H * I, L * H * I, 1.0 / np.sqrt(I)).reshape(L, H, I)
    return w1, w2


def make_inputs(cfg: "Config", with_weights: bool = True) -> dict:
    """All inputs of one configuration (host numpy arrays)."""
    x = tokens(cfg.max_tokens_per_rank, cfg.num_tokens, cfg.hidden)
    ids, w = routing(cfg.max_tokens_per_rank, cfg.num_tokens, cfg.num_experts, cfg.top_k, cfg.zipf_s)
    d = {"hidden_states": x, "topk_ids": ids, "topk_weights": w, "w_gate_up": None, "w_down": None}
    if with_weights and cfg.intermediate > 0:
        d["w_gate_up"], d["w_down"] = expert_weights(cfg.num_experts, cfg.num_local_experts, cfg.rank,
                                                     cfg.hidden, cfg.intermediate)
    return d


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (test helper for hand-made inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)
