"""GPU parity: the HIP library through the C ABI against the CPU oracle.

Integer outputs (counts, offsets, slots, source info, layout ranges, received
routing, the bridge's pick order, local -> global ids) and every copied row
must match bit for bit; floating-point outputs must meet the layer's bf16
tolerance.  Workloads: the five named configurations (sampled tokens where the
oracle would take minutes), the FlashInfer walkthrough shape in both
low-latency layouts, nonzero-rank variants, and edge cases.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import combine_topk_ids_amd as m
import oracle
import synth
from gpu_harness import THREADS, Case, assert_close, dev_bf16, host_bits, host_f32, sample_tokens

pytestmark = pytest.mark.gpu

ALL = ["tiny_flat", "decode_expert_major", "rank_major", "prefill_flat_zipf", "bandwidth_identity",
       "walkthrough_expert_major", "walkthrough_rank_major", "walkthrough_rank_major_r5", "decode_expert_major_r3",
       "rank_major_r5", "prefill_flat_zipf_r3"]
# workloads whose full oracle output other test modules compare against too (kept per process)
SHARED_REF = {"prefill_flat_zipf"}


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _cpu(t):
    return t.cpu().numpy()


def check_dispatch(c: Case, r: dict):
    cfg = c.cfg
    L, K, N, cap = cfg.num_local_experts, cfg.top_k, cfg.num_tokens, c.cap
    assert np.array_equal(_cpu(c.arr("recv_count", L)), r["recv_count"])
    assert np.array_equal(_cpu(c.arr("expert_offsets", L + 1)), r["expert_offsets"])
    rx = c.recv_x().view(torch.int16)
    x = c.x.view(torch.int16)
    if cfg.layout == "EXPERT_MAJOR":
        assert np.array_equal(_cpu(c.arr("slot_of", N * K)), r["slot_of"])
        assert np.array_equal(_cpu(c.arr("layout_range", L * cfg.world * 2)), r["layout_range"])
        cnt = np.minimum(r["recv_count"], cap)
        used = np.concatenate([e * cap + np.arange(cnt[e]) for e in range(L)]).astype(np.int64)
        si = _cpu(c.arr("src_info", L * cap))
        assert np.array_equal(si[used], r["src_info"][used])
        ui = torch.from_numpy(used).cuda()
        src = torch.from_numpy(r["src_info"][used].astype(np.int64)).cuda()
        assert torch.equal(rx[ui], x[src]), "recv_x slots differ from their source rows"
        # unused slots keep the zeros the workspace was allocated with (sampled on big buffers)
        unused = np.setdiff1d(np.arange(L * cap), used)
        if len(unused) > 4096:
            unused = np.random.default_rng(1).choice(unused, 4096, replace=False)
        if len(unused):
            assert int(rx[torch.from_numpy(unused).cuda()].abs().sum()) == 0
        return
    rows = c.rows if cfg.layout == "RANK_MAJOR" else int(r["num_recv"][0])
    if cfg.layout == "FLAT":
        assert int(_cpu(c.arr("num_recv", 1))[0]) == rows
        assert np.array_equal(_cpu(c.arr("recv_src_idx", N))[:rows], r["recv_src_idx"][:rows])
    assert np.array_equal(_cpu(c.arr("row_of_token", N)), r["row_of_token"])
    assert np.array_equal(_cpu(c.arr("recv_topk_idx", c.rows * K))[:rows * K], r["recv_topk_idx"][:rows * K])
    assert np.array_equal(_cpu(c.arr("recv_topk_weights", c.rows * K, torch.float32))[:rows * K],
                          r["recv_topk_weights"][:rows * K])
    tok = np.nonzero(r["row_of_token"] >= 0)[0]
    rw = torch.from_numpy(r["row_of_token"][tok].astype(np.int64)).cuda()
    assert torch.equal(rx[rw], x[torch.from_numpy(tok).cuda()]), "received rows differ from their source rows"


def check_bridge(c: Case, r: dict):
    cfg = c.cfg
    L, K = cfg.num_local_experts, cfg.top_k
    rows = c.rows if cfg.layout == "RANK_MAJOR" else int(r["num_recv"][0])
    rc, b = oracle.bridge(c.op, rows, r["recv_topk_idx"][:rows * K], r["recv_topk_weights"][:rows * K])
    assert rc == oracle.OK
    P = len(b["perm"])
    assert np.array_equal(_cpu(c.arr("pick_count", L)), b["pick_count"])
    assert np.array_equal(_cpu(c.arr("pick_offsets", L + 1)), b["pick_offsets"])
    assert np.array_equal(_cpu(c.arr("perm", max(P, 1)))[:P], b["perm"])
    for name, dt in (("pick_slot", torch.int32), ("topk_gid", torch.int32), ("topk_wmask", torch.float32)):
        assert np.array_equal(_cpu(c.arr(name, c.rows * K, dt))[:rows * K], b[name]), name
    return b


def oracle_em_slots(c: Case, r: dict, slots: np.ndarray) -> np.ndarray:
    cfg = c.cfg
    H, I, cap = cfg.hidden, cfg.intermediate, c.cap
    x = c.d["hidden_states"]

    def one(s):
        el = int(s) // cap
        t = int(r["src_info"][s])
        return oracle.expert_ffn(x[t], c.d["w_gate_up"][el], c.d["w_down"][el], H, I)

    with ThreadPoolExecutor(THREADS) as ex:
        return np.stack(list(ex.map(one, slots))) if len(slots) else np.zeros((0, H), np.float32)


@pytest.fixture(params=["default", "multi_launch"])
def dispatch_path(request, monkeypatch):
    """Small layers take the one-launch dispatch by default; the library's test knob forces the
    multi-launch path (routing kernels + permute) that the large layers take."""
    if request.param == "multi_launch":
        monkeypatch.setenv("MOE_EP_MULTI_LAUNCH_DISPATCH", "1")
    return request.param


@pytest.mark.parametrize("name", ALL)
def test_dispatch_parity(name, dispatch_path):
    cfg = synth.get_config(name)
    c = Case(cfg, synth.make_inputs(cfg, with_weights=False), identity=True)
    c.dispatch()
    torch.cuda.synchronize()
    assert c.status() == m._lib.OK
    check_dispatch(c, c.oracle_route())


@pytest.mark.parametrize("name", ["tiny_flat", "rank_major", "rank_major_r5", "walkthrough_rank_major",
                                  "walkthrough_rank_major_r5", "edge_RANK_MAJOR", "edge_FLAT"])
def test_fused_forward_bridge_arrays(name, dispatch_path):
    # The fused forward's compute-side bridge (written by the one-launch dispatch on small layers, by
    # the bridge kernels otherwise) against the oracle's bridge over the received routing: read back
    # from the workspace through the handle of a dispatch on the same workspace.
    if name.startswith("edge_"):
        cfg = synth.Config("edge", name[5:], 16, 4, 2, 96, 4 * 96 - 37, 256, 192, 5)
        c = Case(cfg, _edge_inputs(cfg))
    else:
        cfg = synth.get_config(name)
        c = Case(cfg)
    c.dispatch()
    c.ws.fill_(0x5A)           # what the forward does not write stays visibly wrong
    out = c.forward()
    r = c.oracle_route()
    check_dispatch(c, r)
    check_bridge(c, r)
    ref = c.oracle_out_all()
    assert_close(host_f32(out), ref, f"{name} fused forward")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ALL)
def test_stages_and_fused_forward(name):
    cfg = synth.get_config(name)
    c = Case(cfg)
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    r = c.oracle_route()
    check_dispatch(c, r)
    # the layer output, every token, against the oracle (the two largest workloads take the
    # 16-thread oracle about a minute each)
    ref = c.oracle_out_all(key=(cfg, "synth") if name in SHARED_REF else None)
    rel, mx = assert_close(host_f32(out), ref, f"{name} out")
    print(f"[{name}] out rel_fro={rel:.2e} max_abs={mx:.2e} over {cfg.num_tokens} x {cfg.hidden}", flush=True)
    # the expert stage's output, every row that holds a pick
    if cfg.layout == "EXPERT_MAJOR":
        cnt = np.minimum(r["recv_count"], c.cap)
        used = np.concatenate([e * c.cap + np.arange(cnt[e]) for e in range(cfg.num_local_experts)])
        ui = torch.from_numpy(used.astype(np.int64)).cuda()
        if cfg.intermediate == 0:
            assert torch.equal(eo[ui], c.recv_x()[ui])
        else:
            rel, mx = assert_close(host_f32(eo[ui]), oracle_em_slots(c, r, used), f"{name} expert_out")
            print(f"[{name}] expert_out rel_fro={rel:.2e} max_abs={mx:.2e} over {len(used)} slots", flush=True)
    else:
        check_bridge(c, r)
        tok = np.nonzero(r["row_of_token"] >= 0)[0]
        rows = r["row_of_token"][tok].astype(np.int64)
        # A received row's expert-stage value is, in the oracle, its source token's layer output:
        # the same row bits (checked bit for bit above), the same picks, the same order.  That is
        # pinned here on sampled rows against the oracle's own per-row function, then used for all.
        smp = sample_tokens(len(tok), 32, seed=11)
        rx = np.zeros((c.rows, cfg.hidden), np.uint16)
        rx[rows[smp]] = host_bits(c.recv_x()[torch.from_numpy(rows[smp]).cuda()])
        z = oracle.recv_rows_z(c.op, rx, r["recv_topk_idx"], r["recv_topk_weights"], c.d["w_gate_up"],
                               c.d["w_down"], rows[smp], threads=THREADS)
        assert np.array_equal(z, ref[tok[smp]])
        rel, mx = assert_close(host_f32(eo[torch.from_numpy(rows).cuda()]), ref[tok], f"{name} expert_out rows")
        print(f"[{name}] expert_out rel_fro={rel:.2e} max_abs={mx:.2e} over {len(rows)} rows", flush=True)
    # the fused forward computes the same values as the three stages, bit for bit
    out2 = c.forward()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    if cfg.intermediate == 0:
        # identity expert and softmax weights summing to 1 -> the input comes back exactly
        if cfg.num_local_experts == cfg.num_experts:
            assert torch.equal(out.view(torch.int16), c.x.view(torch.int16))


def test_determinism_of_routing():
    for name in ("decode_expert_major", "prefill_flat_zipf"):
        c = Case(synth.get_config(name), identity=True)
        c.dispatch()
        torch.cuda.synchronize()
        first = c.ws.clone()
        c.dispatch()
        torch.cuda.synchronize()
        assert torch.equal(first, c.ws), name


def _edge_inputs(cfg, seed=77):
    d = synth.make_inputs(cfg)
    ids = d["topk_ids"].copy()
    rng = np.random.default_rng(seed)
    ids[rng.random(ids.shape) < 0.1] = -1          # scattered masked picks
    ids[3, :] = -1                                 # all masked
    o = cfg.rank * cfg.num_local_experts
    ids[5, :] = [o, o, o + 1, -1, o + 2][: cfg.top_k]  # repeated expert in one token
    ids[7, :] = (o + cfg.num_local_experts) % cfg.num_experts  # only non-local picks
    ids[9, :] = o + cfg.num_local_experts - 1      # every pick on the last local expert
    d["topk_ids"] = ids
    return d


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
def test_edge_cases(layout):
    # 16 experts, 4 local at rank 2, ragged 347 tokens (2 routing chunks), top-5, H=256, I=192
    cfg = synth.Config("edge", layout, 16, 4, 2, 96, 4 * 96 - 37, 256, 192, 5)
    c = Case(cfg, _edge_inputs(cfg))
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    r = c.oracle_route()
    check_dispatch(c, r)
    if layout != "EXPERT_MAJOR":
        check_bridge(c, r)
    ref = c.oracle_out(np.arange(cfg.num_tokens))
    assert_close(host_f32(out), ref, f"edge {layout} out")
    o = host_f32(out)
    assert np.all(o[3] == 0) and np.all(o[7] == 0)
    assert torch.equal(out.view(torch.int16), c.forward().view(torch.int16))


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
@pytest.mark.parametrize("H,I", [(128, 64), (256, 192), (384, 320)])
def test_large_row_tiles_short_k(layout, H, I):
    # 1500 tokens x top-4 over 8 experts: about 750 rows per local expert, so the GEMMs take 256-row
    # tiles (the path chosen from 512 expected rows per expert on), each expert ending in a ragged
    # tile.  H and I give 2 / 4 / 6 gate_up and 1 / 3 / 5 down k-slices of 64 (the pipeline's
    # prologue and tail slices without a steady state) and ragged 128-column gate_up blocks.
    cfg = synth.Config("big_tiles", layout, 8, 4, 1, 1024, 1500, H, I, 4)
    assert cfg.num_tokens * cfg.top_k // cfg.num_experts >= 512
    c = Case(cfg)
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    ref = c.oracle_out(np.arange(cfg.num_tokens))
    assert_close(host_f32(out), ref, f"large tiles {layout} H={H} I={I}")
    assert torch.equal(out.view(torch.int16), c.forward().view(torch.int16))


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
@pytest.mark.parametrize("H,I", [(128, 64), (128, 192), (256, 64)])
def test_small_row_tiles_short_k(layout, H, I):
    # 600 tokens x top-3 over 32 experts, 8 local: about 56 rows per local expert, so the GEMMs take
    # 64-row tiles, and with few items the gate_up GEMM takes the narrow 64x128 tiles with three
    # k-slice stages.  H and I give 2 / 2 / 4 gate_up and 1 / 3 / 1 down k-slices of 64 (H is a
    # multiple of 128: the three-stage prologue with two slices, and a steady state of two) and
    # ragged tiles.
    cfg = synth.Config("small_tiles", layout, 32, 8, 1, 256, 600, H, I, 3)
    assert cfg.num_tokens * cfg.top_k // cfg.num_experts < 512
    c = Case(cfg, _edge_inputs(cfg))
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    ref = c.oracle_out(np.arange(cfg.num_tokens))
    assert_close(host_f32(out), ref, f"small tiles {layout} H={H} I={I}")
    assert torch.equal(out.view(torch.int16), c.forward().view(torch.int16))


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
@pytest.mark.parametrize("H,I", [(256, 320), (128, 4096)])
def test_small_row_tiles_many_per_expert(layout, H, I):
    # 1024 tokens x top-2 over 16 experts, 8 local, Zipf(1.3) routing with the edge-case picks: 64-row
    # tiles (128 rows per expert on average), the local experts holding 10, 6, 4, 3, 2, 2, 2 and 1 row
    # tiles.  The 64-row kernels group an expert's row tiles four at a time, the last group of each
    # expert holding what is left (here three, two or one tile), and take item after item from that
    # order: experts with several groups and short last groups.  (256, 320): narrow gate_up tiles and
    # the 64-row down kernel (I not a multiple of 256); (128, 4096): the 64x256 gate_up kernel (two
    # 64x256 items per CU under even routing) and the weight-streaming down kernel.
    cfg = synth.Config("zipf_tiles", layout, 16, 8, 0, 1024, 1024, H, I, 2, 1.3)
    assert cfg.num_tokens * cfg.top_k // cfg.num_experts < 512
    c = Case(cfg, _edge_inputs(cfg))
    r = c.oracle_route()
    tiles = -(-np.minimum(r["recv_count"].astype(np.int64), c.cap) // 64)
    assert tiles.max() > 8 and np.any(tiles % 4 == 1) and np.any(tiles % 4 == 2) and np.any(tiles % 4 == 3)
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    check_dispatch(c, r)
    rel, mx = assert_close(host_f32(out), c.oracle_out(np.arange(cfg.num_tokens)), f"zipf tiles {layout} H={H} I={I}")
    print(f"[zipf tiles {layout} H={H} I={I}] tiles per expert {tiles.tolist()}, out rel_fro={rel:.2e} max_abs={mx:.2e}",
          flush=True)
    assert torch.equal(out.view(torch.int16), c.forward().view(torch.int16))


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
@pytest.mark.parametrize("H,I", [(128, 448), (256, 384), (384, 320), (512, 192), (640, 128), (2048, 448)])
def test_64_row_tiles_k_slices(layout, H, I):
    # 2048 tokens x top-8 over 64 experts, all local: about 256 rows per expert, so 64-row tiles, and
    # 64 x 4 row tiles x ceil(I / 128) >= 512 gate_up items under even routing, so the 64x256 gate_up
    # kernel (except at I = 128: the narrow one); I not a multiple of 256, so the 64x256 down kernel
    # rather than the weight-streaming one.  H and I give gate_up 2 / 4 / 6 / 8 / 10 / 32 and down
    # 7 / 6 / 5 / 3 / 2 / 7 k-slices of 64: the two-stage prologue, a short steady state and the tail.
    # At H = 2048 the rows are 4 KB apart, and the gate_up items take their slices in rotated order.
    cfg = synth.Config("k_slices_64", layout, 64, 64, 0, 2048, 2048, H, I, 8)
    assert cfg.num_tokens * cfg.top_k // cfg.num_experts < 512 and I % 256 != 0
    c = Case(cfg)
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    rel, mx = assert_close(host_f32(out), c.oracle_out_all(), f"64-row k-slices {layout} H={H} I={I}")
    print(f"[64-row k-slices {layout} H={H} I={I}] out rel_fro={rel:.2e} max_abs={mx:.2e}", flush=True)
    assert torch.equal(out.view(torch.int16), c.forward().view(torch.int16))


@pytest.mark.parametrize("E,N", [(7, 3600), (7, 3700), (7, 3800), (5, 1400)])
def test_large_row_tiles_last_rounds_by_ticket(E, N):
    # Every expert local, top-2, H = 256, I = 4096: 256-row tiles (about 560-1090 rows per expert), 32
    # gate_up column blocks, and too many items for split-K.  The 256-row gate_up kernel deals its
    # items statically but hands the last three rounds out by ticket, counting the items without the
    # padding of the last scheduling group of four row tiles: here 33, 34, 35 and 15 row tiles, so the
    # last group holds one, two or three real tiles, with two static rounds before the tickets (3600,
    # 3700, 3800 tokens) or none (1400).  Every output is checked, and the layer repeats bit for bit.
    cfg = synth.Config("ticket_rounds", "FLAT", E, E, 0, N, N, 256, 4096, 2)
    c = Case(cfg)
    r = c.oracle_route()
    nrt = int(np.sum(-(-r["recv_count"].astype(np.int64) // 256)))
    grid = torch.cuda.get_device_properties(0).multi_processor_count // 8 * 8
    rounds = -(-(-(-nrt // 4) * 4 * 32) // grid)
    assert nrt % 4 != 0, nrt
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    rel, mx = assert_close(host_f32(out), c.oracle_out_all(), f"ticket rounds E={E} N={N}")
    print(f"[ticket rounds E={E} N={N}] {nrt} row tiles, {rounds} rounds on {grid} workgroups, "
          f"out rel_fro={rel:.2e} max_abs={mx:.2e}", flush=True)
    out2 = c.forward()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(out2.view(torch.int16), c.forward().view(torch.int16))


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
@pytest.mark.parametrize("N", [2080, 600])
def test_split_tail_of_narrow_gate_up(layout, N):
    # Top-4 over 32 experts, 8 local, H = 2048 (32 k-slices), I = 1024: the narrow 64x128 gate_up
    # tiles (even routing gives fewer than two 64x256 items per CU).  N = 2080: 36 row tiles, 576
    # items, one full round of the 512-workgroup grid and 64 items left over; N = 600: 240 items, no
    # full round.  The items of the last, partial round are split along K into parts (4 and 2 here)
    # that the workgroups finishing first take by ticket; the last part of an item to arrive adds the
    # parts' fp32 partials in k order.  Every output is checked, and the layer repeats bit for bit.
    cfg = synth.Config("split_tail", layout, 32, 8, 0, N, N, 2048, 1024, 4)
    c = Case(cfg)
    r = c.oracle_route()
    tiles = int(np.sum(-(-np.minimum(r["recv_count"].astype(np.int64), c.cap) // 64)))
    grid = torch.cuda.get_device_properties(0).multi_processor_count * 2 // 8 * 8
    items = tiles * (cfg.intermediate // 64)
    assert items % grid > 0, (items, grid)
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    rel, mx = assert_close(host_f32(out), c.oracle_out_all(), f"split tail {layout} N={N}")
    print(f"[split tail {layout} N={N}] {items} items on {grid} workgroups, out rel_fro={rel:.2e} max_abs={mx:.2e}",
          flush=True)
    out2 = c.forward()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(out2.view(torch.int16), c.forward().view(torch.int16))


@pytest.mark.parametrize("layout,H,I", [("FLAT", 512, 2048), ("RANK_MAJOR", 512, 2048), ("EXPERT_MAJOR", 2048, 512)])
def test_large_row_tiles_many_items_per_workgroup(layout, H, I):
    # 16384 tokens x top-2 over 8 local experts with Zipf(1.1) routing: about 2k to 10k rows per
    # expert in 256-row tiles, and enough items that every persistent workgroup of the 256x256
    # kernels runs several in a row (I = 2048: about 8 gate_up items each; H = 2048: about 4 down
    # items each).  That is the path where the next item's setup loads and first k-slices are
    # issued during the current item, with experts' ragged last tiles in the middle of a
    # workgroup's sequence.  Every output element is checked.
    cfg = synth.Config("many_items", layout, 8, 8, 0, 16384, 16384, H, I, 2, 1.1)
    c = Case(cfg)
    r = c.oracle_route()
    cnt = np.minimum(r["recv_count"].astype(np.int64), c.cap)
    groups = -(-int(np.sum(-(-cnt // 256))) // 4) * 4                  # row tiles in groups of 4
    items = groups * max(-(-I // 128), -(-H // 256))                 # gate_up / down column blocks
    assert items >= 4 * torch.cuda.get_device_properties(0).multi_processor_count
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    check_dispatch(c, r)
    rel, mx = assert_close(host_f32(out), c.oracle_out_all(), f"many items {layout} H={H} I={I}")
    print(f"[many items {layout} H={H} I={I}] {items} items, out rel_fro={rel:.2e} max_abs={mx:.2e}", flush=True)
    assert torch.equal(out.view(torch.int16), c.forward().view(torch.int16))


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
@pytest.mark.parametrize("H,I,zipf", [(2048, 512, 0.0), (512, 2048, 1.5)])
def test_split_k_partials(layout, H, I, zipf):
    # About 550 rows per local expert (256-row tiles, three per expert; with Zipf 1.5 uneven and
    # ragged) and so few items that the 256-row GEMM with the long contraction splits K 8 ways:
    # gate_up at H = 2048 (48 items of 32 slices), down at I = 2048 (24 items of 32 slices).  Every
    # split writes an fp32 partial and the last to arrive sums them in split order: the output
    # matches the oracle and repeats bit for bit.
    cfg = synth.Config("split_k", layout, 4, 4, 0, 1100, 1100, H, I, 2, zipf)
    c = Case(cfg)
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    rel, mx = assert_close(host_f32(out), c.oracle_out_all(), f"split-K {layout} H={H} I={I} zipf={zipf}")
    print(f"[split-K {layout} H={H} I={I} zipf={zipf}] rel_fro={rel:.2e} max_abs={mx:.2e}", flush=True)
    out2 = c.forward()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(out2.view(torch.int16), c.forward().view(torch.int16))


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
@pytest.mark.parametrize("H,I,zipf", [(256, 256, 0.0), (512, 768, 1.2), (768, 512, 0.0)])
def test_weight_streaming_small_tiles(layout, H, I, zipf):
    # 64-row tiles (about 20 rows per local expert) with I a multiple of 256: the weight-streaming
    # down GEMM at 1 / 2 / 3 k-stages of 256, its 32-row path on short tiles and (Zipf) its 64-row
    # path on experts with several tiles next to experts with none; ragged and single-row tiles
    cfg = synth.Config("stream", layout, 32, 8, 2, 192, 160, H, I, 4, zipf)
    assert cfg.num_tokens * cfg.top_k // cfg.num_experts < 512
    c = Case(cfg)
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    ref = c.oracle_out(np.arange(cfg.num_tokens))
    assert_close(host_f32(out), ref, f"streaming {layout} H={H} I={I} zipf={zipf}")
    assert torch.equal(out.view(torch.int16), c.forward().view(torch.int16))


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
@pytest.mark.parametrize("H,I,zipf", [(2048, 256, 1.2), (2048, 512, 0.0), (1024, 768, 1.2)])
def test_weight_streaming_many_items_per_workgroup(layout, H, I, zipf):
    # 32 local experts, 1024 tokens x top-4: 64-row tiles (the mean is 128 rows per expert), a few
    # thousand 64-column items, so each workgroup of the weight-streaming down GEMM runs many items
    # in a row, tiles of at most 32 rows (three 48 KB stage slots) next to fuller ones (two of
    # 64 KB) in the same LDS; 1 / 2 / 3 k-stages
    cfg = synth.Config("stream_items", layout, 32, 32, 0, 1024, 1024, H, I, 4, zipf)
    assert cfg.num_tokens * cfg.top_k // cfg.num_experts < 512
    c = Case(cfg)
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    rel, mx = assert_close(host_f32(out), c.oracle_out_all(), f"stream items {layout} H={H} I={I} zipf={zipf}")
    print(f"[stream items {layout} H={H} I={I} zipf={zipf}] rel_fro={rel:.2e} max_abs={mx:.2e}", flush=True)
    assert torch.equal(out.view(torch.int16), c.forward().view(torch.int16))


@pytest.mark.parametrize("masked", [False, True])
@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
@pytest.mark.parametrize("H", [4096, 7168, 8192])
def test_weighted_sums_over_few_rows(layout, H, masked):
    # 300 tokens of wide rows: the combine / finalize kernels with 4, 7 and 8 pieces per thread
    # (buffer-range loads of up to 8 picks per batch) on few rows; 4 of 16 experts local, so
    # some tokens have no local pick (zero rows), and with the mask one source rank's tokens are
    # skipped
    cfg = synth.Config("row_shares", layout, 16, 4, 1, 128, 300, H, 64, 3)
    c = Case(cfg, active=[1, 0, 1, 1] if masked else None)
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    rel, mx = assert_close(host_f32(out), c.oracle_out_all(), f"few rows {layout} H={H} masked={masked}")
    print(f"[few rows {layout} H={H} masked={masked}] rel_fro={rel:.2e} max_abs={mx:.2e}", flush=True)
    assert torch.equal(out.view(torch.int16), c.forward().view(torch.int16))


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
@pytest.mark.parametrize("L", [512, 1024])
def test_more_local_experts_than_threads(layout, L):
    # one rank holding L experts (up to the build's maximum of 1024): the routing kernels' per-expert
    # loops and scans, and the GEMM tile table the fused routing writes, stride over more experts than
    # a workgroup has threads
    cfg = synth.Config("many_experts", layout, L, L, 0, 2048, 2048, 128, 64, 2)
    c = Case(cfg)
    eo, out = c.stages()
    assert c.status() == m._lib.OK
    r = c.oracle_route()
    check_dispatch(c, r)
    ref = c.oracle_out(np.arange(cfg.num_tokens))
    assert_close(host_f32(out), ref, f"{L} local experts {layout}")
    assert torch.equal(out.view(torch.int16), c.forward().view(torch.int16))


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
def test_cross_rank_additivity(layout):
    # FlashInfer walkthrough: a token's expert-parallel output is the sum over the ranks of each
    # rank's local-pick share.  The W per-rank shares, run one after another on this GPU with each
    # rank's slice of one weight set, add up (in fp32) to the layer with every expert local.
    W, E, T, H, I, K = 4, 16, 64, 256, 128, 4
    N = W * T
    d = synth.make_inputs(synth.Config("add", layout, E, E // W, 0, T, N, H, I, K), with_weights=False)
    w1_all, w2_all = synth.expert_weights(E, E, 0, H, I)
    L = E // W
    total = np.zeros((N, H), np.float64)
    for r in range(W):
        cfg = synth.Config("add", layout, E, L, r, T, N, H, I, K)
        share = dict(d, w_gate_up=w1_all[r * L:(r + 1) * L], w_down=w2_all[r * L:(r + 1) * L])
        total += host_f32(Case(cfg, share).forward())
    every = synth.Config("add_all_local", layout, E, E, 0, N, N, H, I, K)
    c = Case(every, dict(d, w_gate_up=w1_all, w_down=w2_all))
    _, whole = c.stages()
    assert c.status() == m._lib.OK
    assert torch.equal(whole.view(torch.int16), c.forward().view(torch.int16))
    assert_close(total.astype(np.float32), host_f32(whole), f"sum of {W} rank shares vs all local, {layout}")
    # and both agree with the oracle of the all-local layer
    assert_close(host_f32(whole), c.oracle_out(np.arange(N)), f"all local {layout}")


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
def test_zero_tokens(layout):
    cfg = synth.Config("empty", layout, 8, 4, 1, 16, 0, 128, 64, 2)
    d = {"hidden_states": np.zeros((0, 128), np.uint16), "topk_ids": np.zeros((0, 2), np.int64),
         "topk_weights": np.zeros((0, 2), np.float32), **dict(zip(("w_gate_up", "w_down"),
                                                                  synth.expert_weights(8, 4, 1, 128, 64)))}
    c = Case(cfg, d)
    c.stages()
    c.forward()
    assert c.status() == m._lib.OK
    assert np.all(_cpu(c.arr("recv_count", 4)) == 0)


def test_identity_expert_rank_major_and_flat():
    for layout in ("RANK_MAJOR", "FLAT"):
        cfg = synth.Config("ident", layout, 8, 8, 0, 64, 64, 256, 0, 3)
        c = Case(cfg)
        eo, out = c.stages()
        assert torch.equal(out.view(torch.int16), c.x.view(torch.int16)), layout


def test_bad_expert_id_is_latched_and_skipped():
    cfg = synth.Config("badid", "FLAT", 16, 4, 1, 32, 64, 128, 64, 3)
    d = synth.make_inputs(cfg)
    d["topk_ids"] = d["topk_ids"].copy()
    d["topk_ids"][10, 1] = 16   # outside [-1, E)
    d["topk_ids"][11, 0] = -5
    c = Case(cfg, d)
    c.stages()
    assert c.status() == m._lib.EEXPERT_ID
    for layout in ("EXPERT_MAJOR", "RANK_MAJOR"):
        c2 = Case(cfg.with_(layout=layout), d)
        c2.stages()
        assert c2.status() == m._lib.EEXPERT_ID


def test_capacity_overflow_is_latched():
    # cap = W*T = 1: a token that picks expert 1 twice overflows it
    cfg = synth.Config("cap", "EXPERT_MAJOR", 2, 2, 0, 1, 1, 128, 64, 2)
    d = synth.make_inputs(cfg)
    d["topk_ids"] = np.array([[1, 1]], np.int64)
    c = Case(cfg, d)
    c.stages()
    assert c.status() == m._lib.ECAPACITY
    assert int(_cpu(c.arr("recv_count", 2))[1]) == 2
    c.forward()


def test_stale_handle_rejected():
    cfg = synth.get_config("tiny_flat")
    c = Case(cfg)
    h1 = c.dispatch()
    old = m.Handle.from_buffer_copy(h1)
    c.dispatch()
    eo = torch.zeros((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MoeEpError) as e:
        m.moe_ep_expert_compute(c.p, old, c.w1, c.w2, eo)
    assert e.value.status == m._lib.ESTALE_HANDLE
    torch.cuda.synchronize()


def test_handle_record_kept_for_the_most_recent_workspaces():
    # The library keeps the last dispatch of the 1024 most recently dispatched workspaces of the
    # process: dispatching on 1024 other workspaces (slices of one buffer) drops the first one's
    # record, so its handle is rejected as stale while the newer ones' still work.
    cfg = synth.get_config("tiny_flat")
    c = Case(cfg)
    stride = (c.wsize + 4095) // 4096 * 4096
    big = torch.zeros(1025 * stride, dtype=torch.uint8, device="cuda")
    wss = [big[i * stride: i * stride + c.wsize] for i in range(1025)]
    handles = [m.Handle.from_buffer_copy(m.moe_ep_dispatch(c.p, c.x, c.ids, c.w, ws)) for ws in wss]
    eo = torch.zeros((cfg.num_tokens, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MoeEpError) as e:
        m.moe_ep_expert_compute(c.p, handles[0], c.w1, c.w2, eo)
    assert e.value.status == m._lib.ESTALE_HANDLE
    m.moe_ep_expert_compute(c.p, handles[-1], c.w1, c.w2, eo)
    m.moe_ep_expert_compute(c.p, handles[1], c.w1, c.w2, eo)
    torch.cuda.synchronize()
