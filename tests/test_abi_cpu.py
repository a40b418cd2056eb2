"""The C ABI without a GPU: the library loads, exports every entry point of
include/moe_ep.h, sizes workspaces, and rejects bad arguments before touching
the device (no kernel is launched in this file)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "moe_ep.h")).read()
    return sorted(set(re.findall(r"^\S[^\n(]*?\b(moe_ep_\w+)\(", src, flags=re.M)))


def test_header_declares_the_stage_entry_points():
    names = _header_functions()
    for n in ("moe_ep_dispatch", "moe_ep_expert_compute", "moe_ep_combine", "moe_ep_layer_forward",
              "moe_ep_workspace_size", "moe_ep_query_status", "moe_ep_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from combine_topk_ids_amd import _lib
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in _header_functions():
        assert hasattr(lib, n), n


def test_handle_struct_matches_header_field_order():
    from combine_topk_ids_amd import _lib
    src = open(os.path.join(ROOT, "include", "moe_ep.h")).read()
    body = src[src.index("typedef struct {\n  uint64_t epoch;"):src.index("} moe_ep_handle_t;")]
    fields = re.findall(r"^\s+[\w\s\*]+?\b(\w+);", body, flags=re.M)
    assert [f[0] for f in _lib.Handle._fields_] == fields
    pbody = src[src.index("typedef struct {\n  int32_t num_experts;"):src.index("} moe_ep_params_t;")]
    assert [f[0] for f in _lib.Params._fields_] == re.findall(r"int32_t (\w+);", pbody)


import combine_topk_ids_amd as m  # noqa: E402


def _p(**kw):
    base = dict(num_experts=256, num_local_experts=32, rank=0, max_tokens_per_rank=128, num_tokens=1024,
                hidden=7168, intermediate=2048, top_k=8, layout="EXPERT_MAJOR")
    base.update(kw)
    return m.params(**base)


def test_workspace_size_scales_with_layout():
    em = m.moe_ep_workspace_size(_p())
    # EM receive buffer alone: L * W*T * H * 2 bytes
    assert em >= 32 * 1024 * 7168 * 2
    flat = m.moe_ep_workspace_size(_p(layout="FLAT"))
    assert 1024 * 7168 * 2 <= flat < em
    ident = m.moe_ep_workspace_size(_p(intermediate=0))
    assert ident < em


@pytest.mark.parametrize("bad,code", [
    (dict(num_local_experts=3), m._lib.EINVAL),       # E % L != 0
    (dict(rank=8), m._lib.EINVAL),                   # rank outside [0, W)
    (dict(num_tokens=1025), m._lib.EINVAL),          # N > W*T
    (dict(hidden=7000), m._lib.EINVAL),              # hidden % 128 != 0
    (dict(top_k=0), m._lib.EINVAL),
    (dict(layout=3), m._lib.EINVAL),
    (dict(intermediate=100), m._lib.EUNSUPPORTED),   # not a multiple of 64
    (dict(top_k=65), m._lib.EUNSUPPORTED),
    (dict(num_experts=2048, num_local_experts=2048, max_tokens_per_rank=1024), m._lib.EUNSUPPORTED),
])
def test_bad_params_rejected_before_launch(bad, code):
    p = _p(**bad)
    assert m.moe_ep_workspace_size(p) == 0
    h = m.Handle()
    fake = 1 << 20  # never dereferenced: validation fails first
    rc = m._lib.LIB.moe_ep_dispatch(ctypes.byref(p), fake, fake, fake, None, fake * 256, 1 << 40, ctypes.byref(h), 0)
    assert rc == code
    rc = m._lib.LIB.moe_ep_layer_forward(ctypes.byref(p), fake, fake, fake, None, fake, fake, fake, fake * 256, 1 << 40, 0)
    assert rc == code


def test_null_and_workspace_errors():
    p = _p()
    need = m.moe_ep_workspace_size(p)
    h = m.Handle()
    f = 1 << 20
    L = m._lib.LIB
    assert L.moe_ep_dispatch(ctypes.byref(p), None, f, f, None, f * 256, need, ctypes.byref(h), 0) == m._lib.EINVAL
    assert L.moe_ep_dispatch(ctypes.byref(p), f, f, f, None, None, need, ctypes.byref(h), 0) == m._lib.EINVAL
    assert L.moe_ep_dispatch(ctypes.byref(p), f, f, f, None, f * 256, need - 1, ctypes.byref(h), 0) == m._lib.EWORKSPACE
    assert L.moe_ep_dispatch(ctypes.byref(p), f, f, f, None, f * 256 + 16, need, ctypes.byref(h), 0) == m._lib.EWORKSPACE
    # RANK_MAJOR / FLAT carry the weights in dispatch: NULL weights rejected
    pr = _p(layout="FLAT")
    assert L.moe_ep_dispatch(ctypes.byref(pr), f, f, None, None, f * 256, 1 << 40, ctypes.byref(h), 0) == m._lib.EINVAL
    # exactly one of the two weight tensors given
    assert L.moe_ep_layer_forward(ctypes.byref(p), f, f, f, None, f, None, f, f * 256, 1 << 40, 0) == m._lib.EINVAL
    # weights given with the identity expert geometry
    pi = _p(intermediate=0)
    assert L.moe_ep_layer_forward(ctypes.byref(pi), f, f, f, None, f, f, f, f * 256, 1 << 40, 0) == m._lib.EINVAL


def test_handle_checks_without_dispatch():
    p = _p()
    h = m.Handle()  # never dispatched: no workspace
    L = m._lib.LIB
    assert L.moe_ep_expert_compute(ctypes.byref(p), ctypes.byref(h), None, None, 1 << 20, 0) == m._lib.EINVAL
    h.workspace = 1 << 30
    h.params = p
    h.epoch = 7  # no dispatch ever ran on this workspace
    assert L.moe_ep_combine(ctypes.byref(p), ctypes.byref(h), 1 << 20, 1 << 20, None, 1 << 20, 0) == m._lib.ESTALE_HANDLE
    q = _p(rank=1)  # params that do not match the handle
    assert L.moe_ep_combine(ctypes.byref(q), ctypes.byref(h), 1 << 20, 1 << 20, None, 1 << 20, 0) == m._lib.EINVAL


def test_router_argument_errors_before_launch():
    L = m._lib.LIB
    f = 1 << 20  # a fake device address: none of these calls may launch
    assert L.moe_ep_router_topk(f, 4, 8, 0, f, f, 0) == m._lib.EINVAL     # top_k < 1
    assert L.moe_ep_router_topk(f, 4, 8, 9, f, f, 0) == m._lib.EINVAL     # top_k > num_experts
    assert L.moe_ep_router_topk(f, -1, 8, 2, f, f, 0) == m._lib.EINVAL    # negative token count
    assert L.moe_ep_router_topk(None, 4, 8, 2, f, f, 0) == m._lib.EINVAL  # null scores
    assert L.moe_ep_router_topk(f, 4, 8, 2, f, None, 0) == m._lib.EINVAL  # null weights
    assert L.moe_ep_router_topk(f, 4, 2048, 8, f, f, 0) == m._lib.EUNSUPPORTED
    assert L.moe_ep_router_topk(f, 4, 256, 65, f, f, 0) == m._lib.EUNSUPPORTED
    assert L.moe_ep_router_topk(None, 0, 8, 2, None, None, 0) == m._lib.OK  # nothing to do


def test_strerror_covers_every_status():
    for s in range(8):
        assert m.strerror(s) and m.strerror(s) != "unknown status"


def test_noalloc_forward_size_limit_before_launch():
    # the static workspace's size in the header is the binding's; a layer over it is rejected before
    # anything touches a device (fake addresses below are never dereferenced)
    src = open(os.path.join(ROOT, "include", "moe_ep.h")).read()
    val = re.search(r"#define MOE_EP_NOALLOC_WORKSPACE_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert val and int(val.group(1)) << int(val.group(2)) == m._lib.NOALLOC_WORKSPACE_BYTES
    L = m._lib.LIB
    f = 1 << 20
    big = _p()   # 1024-token EXPERT_MAJOR decode, H = 7168: 592 MiB of workspace
    assert m.moe_ep_workspace_size(big) > m._lib.NOALLOC_WORKSPACE_BYTES
    assert L.moe_ep_layer_forward_noalloc(ctypes.byref(big), f, f, f, None, f, f, f, 0) == m._lib.EWORKSPACE
    bad = _p(num_local_experts=3)
    assert L.moe_ep_layer_forward_noalloc(ctypes.byref(bad), f, f, f, None, f, f, f, 0) == m._lib.EINVAL
