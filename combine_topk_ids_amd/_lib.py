"""ctypes binding of libmoe_ep.so (include/moe_ep.h): argument marshalling only.

Every function here has the name of the C entry point it calls.  Tensors are
torch tensors on the GPU (or raw integer device addresses); streams default to
torch's current stream.  Every step of the layer runs in the HIP library; if
the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

# torch ships its own HIP runtime (libamdhip64.so, soname libamdhip64.so.7).  Loading torch
# first makes the dynamic linker bind libmoe_ep.so to that same runtime, so kernels, streams
# and allocations all live in one HIP runtime; loading the library first would map a second
# runtime from /opt/rocm next to torch's and hand torch's streams to it.
import torch  # noqa: F401  (must precede the CDLL load below)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_ep.so")

EXPERT_MAJOR, RANK_MAJOR, FLAT = 0, 1, 2
LAYOUTS = {"EXPERT_MAJOR": EXPERT_MAJOR, "RANK_MAJOR": RANK_MAJOR, "FLAT": FLAT}
STATUS = ["MOE_EP_OK", "MOE_EP_EINVAL", "MOE_EP_EUNSUPPORTED", "MOE_EP_EWORKSPACE", "MOE_EP_EEXPERT_ID",
          "MOE_EP_ECAPACITY", "MOE_EP_ESTALE_HANDLE", "MOE_EP_EHIP"]
OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EEXPERT_ID, ECAPACITY, ESTALE_HANDLE, EHIP = range(8)
# the static workspace of moe_ep_layer_forward_noalloc (MOE_EP_NOALLOC_WORKSPACE_BYTES in the header)
NOALLOC_WORKSPACE_BYTES = 256 << 20
EXPORTED = ["moe_ep_workspace_size", "moe_ep_dispatch", "moe_ep_expert_compute", "moe_ep_combine",
            "moe_ep_layer_forward", "moe_ep_layer_forward_timed", "moe_ep_query_status", "moe_ep_strerror"]


class MoeEpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS[status] if 0 <= status < len(STATUS) else str(status)
        super().__init__(f"{where}: {name} ({strerror(status)})")


class Params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_experts", "num_local_experts", "rank", "max_tokens_per_rank", "num_tokens", "hidden",
        "intermediate", "top_k", "layout")]


class Handle(ctypes.Structure):
    _fields_ = [("epoch", ctypes.c_uint64), ("workspace", ctypes.c_void_p), ("params", Params)] + [
        (n, ctypes.c_void_p) for n in (
            "recv_x", "recv_count", "expert_offsets", "slot_of", "src_info", "layout_range", "recv_topk_idx",
            "recv_topk_weights", "row_of_token", "recv_src_idx", "num_recv", "pick_count", "pick_offsets", "perm",
            "pick_slot", "topk_gid", "topk_wmask", "status", "internal")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                          "or `python combine_topk_ids_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _mapped_hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError("more than one HIP runtime is mapped in this process: " + ", ".join(runtimes))
    P, H, vp = ctypes.POINTER(Params), ctypes.POINTER(Handle), ctypes.c_void_p
    lib.moe_ep_workspace_size.argtypes = [P]
    lib.moe_ep_workspace_size.restype = ctypes.c_size_t
    lib.moe_ep_dispatch.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_size_t, H, vp]
    lib.moe_ep_expert_compute.argtypes = [P, H, vp, vp, vp, vp]
    lib.moe_ep_combine.argtypes = [P, H, vp, vp, vp, vp, vp]
    lib.moe_ep_layer_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.moe_ep_layer_forward_timed.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                               ctypes.POINTER(vp), vp]
    lib.moe_ep_layer_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_ep_layer_forward_fused_combine.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                                       ctypes.POINTER(vp), vp]
    lib.moe_ep_router_topk.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, vp]
    lib.moe_ep_fp8_scale_stride.argtypes = [ctypes.c_int32]
    lib.moe_ep_fp8_scale_stride.restype = ctypes.c_int32
    lib.moe_ep_quantize_fp8.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, vp, vp, vp]
    lib.moe_ep_layer_forward_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                             ctypes.POINTER(vp), vp]
    lib.moe_ep_query_status.argtypes = [H, vp]
    lib.moe_ep_strerror.argtypes = [ctypes.c_int]
    lib.moe_ep_strerror.restype = ctypes.c_char_p
    for f in ("moe_ep_dispatch", "moe_ep_expert_compute", "moe_ep_combine", "moe_ep_layer_forward",
              "moe_ep_layer_forward_timed", "moe_ep_query_status", "moe_ep_router_topk", "moe_ep_quantize_fp8",
              "moe_ep_layer_forward_fp8", "moe_ep_layer_forward_noalloc", "moe_ep_layer_forward_fused_combine"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _mapped_hip_runtimes() -> list:
    try:
        with open("/proc/self/maps") as f:
            paths = {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:
        return []
    return sorted({os.path.realpath(p) for p in paths})


LIB = _load()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str) -> None:
    if rc != OK:
        raise MoeEpError(rc, where)


def params(num_experts, num_local_experts, rank, max_tokens_per_rank, num_tokens, hidden, intermediate, top_k,
           layout) -> Params:
    if isinstance(layout, str):
        layout = LAYOUTS[layout]
    return Params(num_experts, num_local_experts, rank, max_tokens_per_rank, num_tokens, hidden, intermediate,
                  top_k, layout)


def strerror(status: int) -> str:
    return LIB.moe_ep_strerror(status).decode()


def moe_ep_workspace_size(p: Params) -> int:
    return int(LIB.moe_ep_workspace_size(ctypes.byref(p)))


def moe_ep_dispatch(p: Params, hidden_states, topk_ids, topk_weights, workspace, workspace_bytes=None,
                    handle: Handle | None = None, stream=None, active_ranks=None) -> Handle:
    """active_ranks: device int32 [W] source-rank mask or None (the C argument after topk_weights)."""
    handle = handle if handle is not None else Handle()
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    rc = LIB.moe_ep_dispatch(ctypes.byref(p), _ptr(hidden_states), _ptr(topk_ids), _ptr(topk_weights),
                             _ptr(active_ranks), _ptr(workspace), nbytes, ctypes.byref(handle), _stream(stream))
    _check(rc, "moe_ep_dispatch")
    return handle


def moe_ep_expert_compute(p: Params, handle: Handle, w_gate_up, w_down, expert_out, stream=None) -> None:
    rc = LIB.moe_ep_expert_compute(ctypes.byref(p), ctypes.byref(handle), _ptr(w_gate_up), _ptr(w_down),
                                   _ptr(expert_out), _stream(stream))
    _check(rc, "moe_ep_expert_compute")


def moe_ep_combine(p: Params, handle: Handle, expert_out, topk_weights, out, stream=None,
                   active_ranks=None) -> None:
    rc = LIB.moe_ep_combine(ctypes.byref(p), ctypes.byref(handle), _ptr(expert_out), _ptr(topk_weights),
                            _ptr(active_ranks), _ptr(out), _stream(stream))
    _check(rc, "moe_ep_combine")


def moe_ep_layer_forward(p: Params, hidden_states, topk_ids, topk_weights, w_gate_up, w_down, out, workspace,
                         workspace_bytes=None, stream=None, active_ranks=None) -> None:
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    rc = LIB.moe_ep_layer_forward(ctypes.byref(p), _ptr(hidden_states), _ptr(topk_ids), _ptr(topk_weights),
                                  _ptr(active_ranks), _ptr(w_gate_up), _ptr(w_down), _ptr(out), _ptr(workspace),
                                  nbytes, _stream(stream))
    _check(rc, "moe_ep_layer_forward")


def moe_ep_layer_forward_noalloc(p: Params, hidden_states, topk_ids, topk_weights, w_gate_up, w_down, out,
                                 stream=None, active_ranks=None) -> None:
    """The fused forward on the library's static per-GPU workspace (no workspace argument)."""
    rc = LIB.moe_ep_layer_forward_noalloc(ctypes.byref(p), _ptr(hidden_states), _ptr(topk_ids), _ptr(topk_weights),
                                          _ptr(active_ranks), _ptr(w_gate_up), _ptr(w_down), _ptr(out),
                                          _stream(stream))
    _check(rc, "moe_ep_layer_forward_noalloc")


def moe_ep_layer_forward_timed(p: Params, hidden_states, topk_ids, topk_weights, w_gate_up, w_down, out,
                               workspace, events, workspace_bytes=None, stream=None, active_ranks=None) -> None:
    """events: 6 torch.cuda.Event (or None entries) recorded at the stage boundaries.  torch makes an
    event's HIP handle on its first record(), so record each event once before passing it."""
    for e in events:
        if e is not None and not e.cuda_event:
            raise ValueError("record() each torch.cuda.Event once before passing it")
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    arr = (ctypes.c_void_p * 6)(*[None if e is None else e.cuda_event for e in events])
    rc = LIB.moe_ep_layer_forward_timed(ctypes.byref(p), _ptr(hidden_states), _ptr(topk_ids), _ptr(topk_weights),
                                        _ptr(active_ranks), _ptr(w_gate_up), _ptr(w_down), _ptr(out),
                                        _ptr(workspace), nbytes, arr, _stream(stream))
    _check(rc, "moe_ep_layer_forward_timed")


def moe_ep_layer_forward_fused_combine(p: Params, hidden_states, topk_ids, topk_weights, w_gate_up, w_down, out,
                                       workspace, events=None, workspace_bytes=None, stream=None,
                                       active_ranks=None) -> None:
    """RANK_MAJOR / FLAT forward with the combine fused into the down GEMM; events: None or 6 recorded
    torch.cuda.Event."""
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    arr = None
    if events is not None:
        for e in events:
            if e is not None and not e.cuda_event:
                raise ValueError("record() each torch.cuda.Event once before passing it")
        arr = (ctypes.c_void_p * 6)(*[None if e is None else e.cuda_event for e in events])
    rc = LIB.moe_ep_layer_forward_fused_combine(ctypes.byref(p), _ptr(hidden_states), _ptr(topk_ids),
                                                _ptr(topk_weights), _ptr(active_ranks), _ptr(w_gate_up),
                                                _ptr(w_down), _ptr(out), _ptr(workspace), nbytes, arr, _stream(stream))
    _check(rc, "moe_ep_layer_forward_fused_combine")


def moe_ep_router_topk(scores, top_k: int, topk_ids, topk_weights, stream=None) -> None:
    """scores: device fp32 [N, E]; fills topk_ids (int64 [N, top_k]) and topk_weights (fp32 [N, top_k])."""
    n, e = (int(scores.shape[0]), int(scores.shape[1])) if scores is not None else (0, 0)
    rc = LIB.moe_ep_router_topk(_ptr(scores), n, e, top_k, _ptr(topk_ids), _ptr(topk_weights), _stream(stream))
    _check(rc, "moe_ep_router_topk")


def moe_ep_fp8_scale_stride(cols: int) -> int:
    return int(LIB.moe_ep_fp8_scale_stride(cols))


def moe_ep_quantize_fp8(x, codes, scales, stream=None) -> None:
    """x: device bf16 [rows, cols]; codes: uint8 [rows, cols]; scales: uint8 [rows, fp8_scale_stride(cols)]."""
    rows, cols = (int(x.shape[0]), int(x.shape[1])) if x is not None else (0, 128)
    rc = LIB.moe_ep_quantize_fp8(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(stream))
    _check(rc, "moe_ep_quantize_fp8")


def moe_ep_layer_forward_fp8(p: Params, hidden_states, topk_ids, topk_weights, w_gate_up_fp8, w_gate_up_scales,
                             w_down, out, workspace, events=None, workspace_bytes=None, stream=None,
                             active_ranks=None) -> None:
    """FP8 dispatch + FP8 gate_up GEMM forward; events: None or 6 recorded torch.cuda.Event."""
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    arr = None
    if events is not None:
        for e in events:
            if e is not None and not e.cuda_event:
                raise ValueError("record() each torch.cuda.Event once before passing it")
        arr = (ctypes.c_void_p * 6)(*[None if e is None else e.cuda_event for e in events])
    rc = LIB.moe_ep_layer_forward_fp8(ctypes.byref(p), _ptr(hidden_states), _ptr(topk_ids), _ptr(topk_weights),
                                      _ptr(active_ranks), _ptr(w_gate_up_fp8), _ptr(w_gate_up_scales),
                                      _ptr(w_down), _ptr(out), _ptr(workspace), nbytes, arr, _stream(stream))
    _check(rc, "moe_ep_layer_forward_fp8")


def moe_ep_query_status(handle: Handle, stream=None) -> int:
    return int(LIB.moe_ep_query_status(ctypes.byref(handle), _stream(stream)))
