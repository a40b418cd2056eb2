"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test ties the oracle to something it cannot agree with by construction:
a routing example derived by hand from the pages' layout contracts, closed
forms, exhaustive enumeration against an independently written sort-based
definition, the dense-MoE formulation of FlashInfer's correctness test in
float64, structural invariants, and exact scaling/permutation identities.

Sources: FlashInfer "MoE-EP implementation & usage" section 3 (layout
contracts, local ids, masking) and section 4 (dense reference, seeds, weight
shapes); Mooncake PG/EP guide "Buffer.dispatch" / "Buffer.combine".
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- hand-derived routing

@pytest.mark.parametrize("golden", ["routing_hand.json", "routing_hand_masked.json"])
@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
def test_routing_hand_example(layout, golden):
    g = _load(golden)
    p = oracle.params(layout=layout, active_ranks=g.get("active_ranks"), **g["geometry"])
    ids = np.array(g["topk_ids"], np.int64)
    w = np.array(g["topk_weights"], np.float32)
    rc, r = oracle.route(p, ids, w)
    assert rc == oracle.OK
    ex = g["expected"]
    assert r["recv_count"].tolist() == ex["recv_count"]
    assert r["expert_offsets"].tolist() == ex["expert_offsets"]
    if layout == "EXPERT_MAJOR":
        for k in ("slot_of", "src_info", "layout_range"):
            assert r[k].tolist() == ex[k], k
        return
    sub = ex["rank_major" if layout == "RANK_MAJOR" else "flat"]
    rows = len(sub["recv_topk_idx"]) // p.top_k
    assert r["recv_topk_idx"][: rows * p.top_k].tolist() == sub["recv_topk_idx"]
    assert r["recv_topk_weights"][: rows * p.top_k].tolist() == sub["recv_topk_weights"]
    assert r["row_of_token"].tolist() == sub["row_of_token"]
    if layout == "FLAT":
        assert int(r["num_recv"][0]) == sub["num_recv"]
        assert r["recv_src_idx"][: sub["num_recv"]].tolist() == sub["recv_src_idx"]
    rc, b = oracle.bridge(p, rows, r["recv_topk_idx"], r["recv_topk_weights"])
    assert rc == oracle.OK
    for k, v in sub["bridge"].items():
        assert b[k].tolist() == v, k


# ---------------------------------------------------------------- closed forms of the expert

def _bf(vals):
    return synth.f32_to_bf16(np.array(vals, np.float32))


def test_expert_ffn_closed_form():
    # H=2, I=1: gate row (1, 0), up row (0, 1), down column (1, 0.5); x = (1, 2).
    # gate = 1, up = 2, a = SiLU(1) * 2 = 2 / (1 + e^-1); y = (a, a/2).
    x = _bf([1.0, 2.0])
    w1 = _bf([[1.0, 0.0], [0.0, 1.0]]).reshape(2, 2)
    w2 = _bf([[1.0], [0.5]]).reshape(2, 1)
    y = oracle.expert_ffn(x, w1, w2, 2, 1)
    a = 2.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(y, [a, a / 2], rtol=2e-7)
    # gate/up swapped would give SiLU(2)*1 = 1.7616 instead of 1.4621: the closed form tells them apart
    assert abs(y[0] - 2.0 / (1.0 + math.exp(-2.0))) > 0.1


def test_expert_ffn_silu_of_negative_gate_and_down_layout():
    # H=2, I=2, distinct entries so that a transposed w_down or swapped halves fail.
    x = _bf([0.5, -1.0])
    w1 = _bf([[1.0, 1.0],     # gate 0 -> -0.5
              [2.0, 0.0],     # gate 1 -> 1.0
              [0.0, -2.0],    # up 0   -> 2.0
              [4.0, 1.0]]).reshape(4, 2)  # up 1 -> 1.0
    w2 = _bf([[1.0, 2.0],
              [-3.0, 0.25]]).reshape(2, 2)
    y = oracle.expert_ffn(x, w1, w2, 2, 2)
    s = lambda g: g / (1.0 + math.exp(-g))
    a0, a1 = s(-0.5) * 2.0, s(1.0) * 1.0
    np.testing.assert_allclose(y, [1.0 * a0 + 2.0 * a1, -3.0 * a0 + 0.25 * a1], rtol=1e-6)


def test_identity_expert_returns_row():
    x = synth.normal_bf16(7, 99, 0, 256)
    y = oracle.expert_ffn(x, None, None, 256, 0)
    assert np.array_equal(y, synth.bf16_to_f32(x))


# ---------------------------------------------------------------- exhaustive routing vs a sort-based definition

def _sorted_definition(ids, E, L, rank, T, K):
    """Independent statement of the slot rule: stable sort of the local picks by (local expert, token, k)."""
    o = rank * L
    N = ids.shape[0]
    t_idx, k_idx = np.meshgrid(np.arange(N), np.arange(K), indexing="ij")
    loc = (ids >= o) & (ids < o + L)
    el = ids[loc] - o
    tt, kk = t_idx[loc], k_idx[loc]
    order = np.lexsort((kk, tt, el))
    counts = np.bincount(el, minlength=L)
    offs = np.concatenate([[0], np.cumsum(counts)])
    cap = (E // L) * T
    slot_of = -np.ones(N * K, np.int64)
    for pos, q in enumerate(order):
        e = el[q]
        slot_of[tt[q] * K + kk[q]] = e * cap + (pos - offs[e])
    return counts, offs, slot_of


def test_routing_exhaustive_tiny():
    # every topk_ids in {-1..E-1}^(N*K) for N=2, K=2, E=4, for each rank of W=2 (L=2) and W=1
    E, K, N = 4, 2, 2
    for L, T in ((2, 1), (4, 2)):
        W = E // L
        for rank in range(W):
            for combo in itertools.product(range(-1, E), repeat=N * K):
                ids = np.array(combo, np.int64).reshape(N, K)
                w = np.full((N, K), 0.5, np.float32)
                p = oracle.params(num_experts=E, num_local_experts=L, rank=rank, max_tokens_per_rank=T,
                                  num_tokens=N, hidden=128, intermediate=0, top_k=K, layout="EXPERT_MAJOR")
                rc, r = oracle.route(p, ids, w)
                counts, offs, slot_of = _sorted_definition(ids, E, L, rank, T, K)
                if counts.max(initial=0) > W * T:
                    assert rc == oracle.ECAPACITY
                    continue
                assert rc == oracle.OK
                assert r["recv_count"].tolist() == counts.tolist()
                assert r["expert_offsets"].tolist() == offs.tolist()
                assert r["slot_of"].tolist() == slot_of.tolist()
                # the bridge over FLAT-received routing orders the same picks the same way
                pf = oracle.params(num_experts=E, num_local_experts=L, rank=rank, max_tokens_per_rank=T,
                                   num_tokens=N, hidden=128, intermediate=0, top_k=K, layout="FLAT")
                rc, rf = oracle.route(pf, ids, w)
                assert rc == oracle.OK
                nr = int(rf["num_recv"][0])
                rc, b = oracle.bridge(pf, nr, rf["recv_topk_idx"], rf["recv_topk_weights"])
                assert rc == oracle.OK
                assert b["pick_count"].tolist() == counts.tolist()
                src = rf["recv_src_idx"][:nr]
                perm_tok = [(int(src[q // K]), q % K) for q in b["perm"]]
                exp_tok = []
                for e in range(L):
                    for t in range(N):
                        for k in range(K):
                            if ids[t, k] == e + rank * L:
                                exp_tok.append((t, k))
                assert perm_tok == exp_tok


# ---------------------------------------------------------------- invariants on the workloads

ROUTE_CASES = ["tiny_flat", "decode_expert_major", "rank_major", "bandwidth_identity",
               "decode_expert_major_r3", "rank_major_r5", "walkthrough_rank_major_r5"]


def _check_invariants(cfg, ids, r):
    p = oracle.params(cfg)
    L, K, N, T, W = cfg.num_local_experts, cfg.top_k, cfg.num_tokens, cfg.max_tokens_per_rank, cfg.world
    o = cfg.rank * L
    cap = W * T
    loc = (ids >= o) & (ids < o + L)
    P = int(loc.sum())
    assert int(r["recv_count"].sum()) == P
    assert np.array_equal(r["expert_offsets"], np.concatenate([[0], np.cumsum(r["recv_count"])]))
    assert np.array_equal(r["recv_count"], np.bincount((ids[loc] - o), minlength=L))
    if cfg.layout == "EXPERT_MAJOR":
        so = r["slot_of"].reshape(N, K)
        assert np.array_equal(so >= 0, loc)
        el, slot = so[loc] // cap, so[loc] % cap
        assert np.array_equal(el, ids[loc] - o)
        # bijection onto [0, count_el) per expert
        for e in range(L):
            s = np.sort(slot[el == e])
            assert np.array_equal(s, np.arange(r["recv_count"][e]))
        # src_info o slot_of = token, and slots increase with (token, k)
        t_of = np.nonzero(loc)[0]
        assert np.array_equal(r["src_info"][so[loc]], t_of)
        si = r["src_info"].reshape(L, cap)
        for e in range(L):
            c = r["recv_count"][e]
            assert np.all(np.diff(si[e, :c]) >= 0) and np.all(si[e, c:] == -1)
        lr = r["layout_range"].reshape(L, W, 2)
        assert np.array_equal(lr[:, :, 1].sum(1), r["recv_count"])
        assert np.array_equal(lr[:, :, 0], np.cumsum(lr[:, :, 1], 1) - lr[:, :, 1])
        return
    has = loc.any(1)
    rows = W * T if cfg.layout == "RANK_MAJOR" else int(has.sum())
    if cfg.layout == "FLAT":
        assert int(r["num_recv"][0]) == rows
        assert np.array_equal(r["recv_src_idx"][:rows], np.nonzero(has)[0])
    rot = r["row_of_token"]
    assert np.array_equal(rot >= 0, has)
    idx = r["recv_topk_idx"].reshape(-1, K)[:rows]
    # received ids are local (-1 = non-local) and match the sender's picks
    assert np.array_equal(idx[rot[has]], np.where(loc[has], ids[has] - o, -1))
    rc, b = oracle.bridge(p, rows, r["recv_topk_idx"], r["recv_topk_weights"])
    assert rc == oracle.OK
    gid = b["topk_gid"].reshape(-1, K)
    assert np.array_equal(gid[idx >= 0] - o, idx[idx >= 0]) and np.all(gid[idx < 0] == -1)
    assert np.all(b["topk_wmask"].reshape(-1, K)[idx < 0] == 0)
    assert np.array_equal(b["pick_count"], r["recv_count"])
    perm = b["perm"]
    assert len(perm) == P and len(np.unique(perm)) == P
    e_of = idx.reshape(-1)[perm]
    assert np.all(np.diff(e_of) >= 0)
    for e in range(L):
        seg = perm[b["pick_offsets"][e]:b["pick_offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
    assert np.array_equal(b["pick_slot"][perm], np.arange(P))


@pytest.mark.parametrize("name", ROUTE_CASES)
def test_routing_invariants(name):
    cfg = synth.get_config(name)
    ids, w = synth.routing(cfg.max_tokens_per_rank, cfg.num_tokens, cfg.num_experts, cfg.top_k, cfg.zipf_s)
    rc, r = oracle.route(oracle.params(cfg), ids, w)
    assert rc == oracle.OK
    _check_invariants(cfg, ids, r)


@pytest.mark.slow
def test_routing_invariants_prefill_zipf():
    cfg = synth.get_config("prefill_flat_zipf")
    ids, w = synth.routing(cfg.max_tokens_per_rank, cfg.num_tokens, cfg.num_experts, cfg.top_k, cfg.zipf_s)
    rc, r = oracle.route(oracle.params(cfg), ids, w)
    assert rc == oracle.OK
    _check_invariants(cfg, ids, r)


def test_routing_edge_cases():
    # duplicates, -1 ids, all-masked tokens, fewer tokens than the ranks can hold
    E, L, K, T = 8, 4, 3, 4
    ids = np.array([[4, 4, -1], [-1, -1, -1], [0, 1, 2], [7, 5, 4], [6, -1, 6]], np.int64)
    w = np.full(ids.shape, 1.0 / 3, np.float32)
    for layout in ("EXPERT_MAJOR", "RANK_MAJOR", "FLAT"):
        p = oracle.params(num_experts=E, num_local_experts=L, rank=1, max_tokens_per_rank=T, num_tokens=5,
                          hidden=128, intermediate=0, top_k=K, layout=layout)
        rc, r = oracle.route(p, ids, w)
        assert rc == oracle.OK
        assert r["recv_count"].tolist() == [3, 1, 2, 1]  # experts 4,5,6,7 local
        if layout == "EXPERT_MAJOR":
            cap = 2 * T
            assert r["slot_of"].tolist() == [0, 1, -1, -1, -1, -1, -1, -1, -1, 3 * cap, cap, 2, 2 * cap,
                                             -1, 2 * cap + 1]
    # capacity overflow needs repeated ids: cap = W*T = 1 slot
    p = oracle.params(num_experts=2, num_local_experts=2, rank=0, max_tokens_per_rank=1, num_tokens=1, hidden=128,
                      intermediate=0, top_k=2, layout="EXPERT_MAJOR")
    assert oracle.route(p, np.array([[1, 1]]), np.ones((1, 2), np.float32))[0] == oracle.ECAPACITY
    # ids outside [-1, E)
    p = oracle.params(num_experts=4, num_local_experts=2, rank=0, max_tokens_per_rank=2, num_tokens=2, hidden=128,
                      intermediate=0, top_k=1, layout="FLAT")
    assert oracle.route(p, np.array([[0], [4]]), np.ones((2, 1), np.float32))[0] == oracle.EEXPERT_ID
    assert oracle.route(p, np.array([[-2], [0]]), np.ones((2, 1), np.float32))[0] == oracle.EEXPERT_ID


def test_param_rules():
    base = dict(num_experts=8, num_local_experts=4, rank=1, max_tokens_per_rank=4, num_tokens=8, hidden=256,
                intermediate=64, top_k=2, layout="FLAT")
    assert oracle.check_params(oracle.params(**base)) == oracle.OK
    for bad in (dict(num_local_experts=3), dict(rank=2), dict(num_tokens=9), dict(hidden=192), dict(top_k=0),
                dict(layout=3), dict(rank=-1)):
        assert oracle.check_params(oracle.params(**{**base, **bad})) == oracle.EINVAL, bad


# ---------------------------------------------------------------- float64 dense MoE on tiny shapes

def _tiny_inputs(E, L, rank, T, N, H, I, K, seed=5):
    ids, w = synth.routing(T, N, E, K, seed_base=seed)
    x = synth.tokens(T, N, H, seed_base=seed)
    w1, w2 = synth.expert_weights(E, E, 0, H, I, seed=seed)   # full weight set [E, ...]
    return x, ids, w, w1, w2


def _dense_moe_f64(x, ids, w, w1, w2, E, o, L, I):
    """Single-process dense MoE: every local expert on every token, weighted by a dense gate matrix."""
    X = synth.bf16_to_f32(x).astype(np.float64)
    N = X.shape[0]
    G = np.zeros((N, E))
    for k in range(ids.shape[1]):
        m = ids[:, k] >= 0
        np.add.at(G, (np.nonzero(m)[0], ids[m, k]), w[m, k].astype(np.float64))
    out = np.zeros_like(X)
    for e in range(o, o + L):
        W1 = synth.bf16_to_f32(w1[e]).astype(np.float64)
        W2 = synth.bf16_to_f32(w2[e]).astype(np.float64)
        gu = X @ W1.T
        a = gu[:, :I] / (1.0 + np.exp(-gu[:, :I])) * gu[:, I:]
        out += G[:, e:e + 1] * (a @ W2.T)
    return out


@pytest.mark.parametrize("E,L,rank,K", [(8, 8, 0, 2), (8, 4, 1, 3), (6, 2, 2, 2)])
def test_forward_vs_dense_moe_f64(E, L, rank, K):
    T, H, I = 8, 128, 96
    W = E // L
    N = W * T - 3  # ragged: the last source rank is not full
    x, ids, w, w1, w2 = _tiny_inputs(E, L, rank, T, N, H, I, K)
    o = rank * L
    p = oracle.params(num_experts=E, num_local_experts=L, rank=rank, max_tokens_per_rank=T, num_tokens=N,
                      hidden=H, intermediate=I, top_k=K, layout="FLAT")
    got = oracle.forward_tokens(p, x, ids, w, w1[o:o + L], w2[o:o + L], np.arange(N))
    ref = _dense_moe_f64(x, ids, w, w1, w2, E, o, L, I)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err < 1e-5, err


def test_topk1_weight1_single_expert_is_dense_ffn():
    H, I, N = 256, 128, 16
    x = synth.tokens(N, N, H, seed_base=11)
    w1, w2 = synth.expert_weights(1, 1, 0, H, I, seed=12)
    p = oracle.params(num_experts=1, num_local_experts=1, rank=0, max_tokens_per_rank=N, num_tokens=N, hidden=H,
                      intermediate=I, top_k=1, layout="EXPERT_MAJOR")
    got = oracle.forward_tokens(p, x, np.zeros((N, 1), np.int64), np.ones((N, 1), np.float32), w1, w2, np.arange(N))
    X = synth.bf16_to_f32(x).astype(np.float64)
    W1 = synth.bf16_to_f32(w1[0]).astype(np.float64)
    W2 = synth.bf16_to_f32(w2[0]).astype(np.float64)
    g, u = X @ W1[:I].T, X @ W1[I:].T
    ref = (g / (1 + np.exp(-g)) * u) @ W2.T
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-5 * np.abs(ref).max())


def test_identity_expert_weights_sum_to_one_returns_input():
    cfg = synth.get_config("tiny_flat").with_(intermediate=0)
    d = synth.make_inputs(cfg)
    p = oracle.params(cfg)
    out = oracle.forward_tokens(p, d["hidden_states"], d["topk_ids"], d["topk_weights"], None, None,
                                np.arange(cfg.num_tokens))
    # all 8 experts are local and softmax weights sum to 1 -> bf16(out) == hidden_states exactly
    assert np.array_equal(synth.f32_to_bf16(out), d["hidden_states"])


def test_all_masked_tokens_are_zero():
    cfg = synth.get_config("tiny_flat")
    d = synth.make_inputs(cfg)
    ids = d["topk_ids"].copy()
    ids[5] = -1
    ids[9, :] = -1
    p = oracle.params(cfg.with_(num_experts=16, num_local_experts=8, rank=1))  # ids 0..7 now non-local
    out = oracle.forward_tokens(p, d["hidden_states"], ids, d["topk_weights"], d["w_gate_up"], d["w_down"],
                                np.arange(16))
    assert np.all(out == 0.0)


def test_exact_scaling_and_token_permutation():
    cfg = synth.get_config("tiny_flat")
    d = synth.make_inputs(cfg)
    p = oracle.params(cfg)
    toks = np.arange(cfg.num_tokens)
    base = oracle.forward_tokens(p, d["hidden_states"], d["topk_ids"], d["topk_weights"], d["w_gate_up"],
                                 d["w_down"], toks)
    # power-of-two weight scaling is exact in binary floating point
    twice = oracle.forward_tokens(p, d["hidden_states"], d["topk_ids"], 2 * d["topk_weights"], d["w_gate_up"],
                                  d["w_down"], toks)
    assert np.array_equal(twice, 2 * base)
    # tokens are independent: permuting the inputs permutes the outputs bit for bit
    perm = np.random.default_rng(3).permutation(cfg.num_tokens)
    pert = oracle.forward_tokens(p, d["hidden_states"][perm], d["topk_ids"][perm], d["topk_weights"][perm],
                                 d["w_gate_up"], d["w_down"], toks)
    assert np.array_equal(pert, base[perm])


def test_cross_rank_additivity():
    # FlashInfer walkthrough: a token's EP output is the sum over ranks of each rank's local-pick share
    E, K, T, H, I = 8, 3, 6, 128, 64
    W = 4
    N = W * T
    x, ids, w, w1, w2 = _tiny_inputs(E, E // W, 0, T, N, H, I, K, seed=21)
    L = E // W
    total = np.zeros((N, H), np.float64)
    for r in range(W):
        p = oracle.params(num_experts=E, num_local_experts=L, rank=r, max_tokens_per_rank=T, num_tokens=N,
                          hidden=H, intermediate=I, top_k=K, layout="RANK_MAJOR")
        total += oracle.forward_tokens(p, x, ids, w, w1[r * L:(r + 1) * L], w2[r * L:(r + 1) * L], np.arange(N))
    p1 = oracle.params(num_experts=E, num_local_experts=E, rank=0, max_tokens_per_rank=N, num_tokens=N, hidden=H,
                       intermediate=I, top_k=K, layout="FLAT")
    whole = oracle.forward_tokens(p1, x, ids, w, w1, w2, np.arange(N))
    np.testing.assert_allclose(total, whole, rtol=0, atol=2e-6 * np.abs(whole).max())


def test_recv_rows_z_matches_forward_on_rank_major():
    # RANK_MAJOR row t holds token t; z (masked weights, real top_k) equals the token's output
    cfg = synth.get_config("tiny_flat").with_(layout="RANK_MAJOR", num_experts=16, rank=1)
    d = synth.make_inputs(cfg)
    p = oracle.params(cfg)
    rc, r = oracle.route(p, d["topk_ids"], d["topk_weights"])
    assert rc == oracle.OK
    toks = np.nonzero(r["row_of_token"] >= 0)[0]
    z = oracle.recv_rows_z(p, d["hidden_states"], r["recv_topk_idx"], r["recv_topk_weights"], d["w_gate_up"],
                           d["w_down"], toks)
    f = oracle.forward_tokens(p, d["hidden_states"], d["topk_ids"], d["topk_weights"], d["w_gate_up"],
                              d["w_down"], toks)
    assert np.array_equal(z, f)


# ---------------------------------------------------------------- active_ranks source-rank mask
# Mooncake PG/EP guide, "Buffer.dispatch" / "Buffer.combine": active_ranks [num_ranks] int32 is the
# EP-level rank-health tensor; tokens of an inactive source rank are skipped by both.

def _mask_case(layout, seed):
    E, L, rank, T, K, H, I = 16, 4, 1, 5, 3, 128, 64
    W = E // L
    N = W * T - 2                     # last source rank sends fewer than T tokens
    x, ids, w, w1, w2 = _tiny_inputs(E, L, rank, T, N, H, I, K, seed=seed)
    p = dict(num_experts=E, num_local_experts=L, rank=rank, max_tokens_per_rank=T, num_tokens=N, hidden=H,
             intermediate=I, top_k=K, layout=layout)
    return p, x, ids, w, w1[rank * L:(rank + 1) * L], w2[rank * L:(rank + 1) * L]


@pytest.mark.parametrize("layout", ["EXPERT_MAJOR", "RANK_MAJOR", "FLAT"])
def test_mask_skipping_a_rank_equals_masking_its_ids(layout):
    # skipping source rank r is the same as marking every pick of its tokens -1 (a masked pick)
    kw, x, ids, w, w1, w2 = _mask_case(layout, seed=31)
    T, W = kw["max_tokens_per_rank"], kw["num_experts"] // kw["num_local_experts"]
    for mask in ([1, 0, 1, 1], [0, 1, 1, 0], [1, 1, 1, 0]):
        dropped = ids.copy()
        for r in range(W):
            if not mask[r]:
                dropped[r * T:(r + 1) * T] = -1
        rc_a, a = oracle.route(oracle.params(active_ranks=mask, **kw), ids, w)
        rc_b, b = oracle.route(oracle.params(**kw), dropped, w)
        assert rc_a == rc_b == oracle.OK
        for k in a:
            assert np.array_equal(a[k], b[k]), (mask, k)
        toks = np.arange(kw["num_tokens"])
        fa = oracle.forward_tokens(oracle.params(active_ranks=mask, **kw), x, ids, w, w1, w2, toks)
        fb = oracle.forward_tokens(oracle.params(**kw), x, dropped, w, w1, w2, toks)
        assert np.array_equal(fa, fb)
        inactive = np.repeat(np.array(mask) == 0, T)[: kw["num_tokens"]]
        assert np.all(fa[inactive] == 0.0) and np.any(fa[~inactive] != 0.0)


def test_mask_all_active_equals_no_mask_and_all_inactive_is_empty():
    kw, x, ids, w, w1, w2 = _mask_case("FLAT", seed=32)
    toks = np.arange(kw["num_tokens"])
    base = oracle.forward_tokens(oracle.params(**kw), x, ids, w, w1, w2, toks)
    ones = oracle.forward_tokens(oracle.params(active_ranks=[1, 1, 1, 1], **kw), x, ids, w, w1, w2, toks)
    assert np.array_equal(base, ones)
    nz = oracle.forward_tokens(oracle.params(active_ranks=[7, -1, 2, 1], **kw), x, ids, w, w1, w2, toks)
    assert np.array_equal(base, nz)   # any nonzero entry means active
    rc, r = oracle.route(oracle.params(active_ranks=[0, 0, 0, 0], **kw), ids, w)
    assert rc == oracle.OK and r["recv_count"].sum() == 0 and int(r["num_recv"][0]) == 0
    zero = oracle.forward_tokens(oracle.params(active_ranks=[0, 0, 0, 0], **kw), x, ids, w, w1, w2, toks)
    assert np.all(zero == 0.0)


def test_mask_ids_of_inactive_ranks_are_not_checked():
    kw, x, ids, w, w1, w2 = _mask_case("EXPERT_MAJOR", seed=33)
    bad = ids.copy()
    bad[1, 0] = 10_000                # token 1 belongs to source rank 0
    assert oracle.route(oracle.params(**kw), bad, w)[0] == oracle.EEXPERT_ID
    assert oracle.route(oracle.params(active_ranks=[0, 1, 1, 1], **kw), bad, w)[0] == oracle.OK
    assert oracle.route(oracle.params(active_ranks=[1, 0, 1, 1], **kw), bad, w)[0] == oracle.EEXPERT_ID


# ---------------------------------------------------------------- router (top-k of scores + softmax)
# Mooncake PG/EP guide quick start / FlashInfer section 4 step 2: topk_idx = top_k of the scores,
# softmax weights (reading: over the selected scores; equal scores ordered by the lower id).

def _router_scores(raw):
    conv = {"ln2": math.log(2), "ln3": math.log(3), "ln5": math.log(5), "-inf": -math.inf}
    return np.array([[conv[v] if isinstance(v, str) else v for v in row] for row in raw], np.float32)


def test_router_hand_example():
    g = _load("router_hand.json")
    rc, ids, w = oracle.router_topk(_router_scores(g["scores"]), g["top_k"])
    assert rc == oracle.OK
    assert ids.tolist() == g["expected_ids"]
    np.testing.assert_allclose(w, np.array(g["expected_weights"]), rtol=1e-6, atol=1e-7)


def test_router_against_sort_definition_with_ties():
    from scipy.special import softmax
    rng = np.random.default_rng(41)
    for N, E, K in [(200, 8, 2), (100, 16, 5), (50, 64, 6), (20, 100, 10), (30, 6, 6)]:
        s = np.round(rng.standard_normal((N, E)) * 2).astype(np.float32)   # many exact ties
        rc, ids, w = oracle.router_topk(s, K)
        assert rc == oracle.OK
        order = np.lexsort((np.broadcast_to(np.arange(E), s.shape), -s.astype(np.float64)), axis=1)[:, :K]
        assert np.array_equal(ids, order)
        ref = softmax(np.take_along_axis(s, order, 1).astype(np.float64), axis=1)
        np.testing.assert_allclose(w, ref, rtol=2e-7, atol=0)
        assert np.all(np.diff(w, axis=1) <= 0)


def test_router_matches_torch_topk_on_distinct_scores():
    import torch
    rng = np.random.default_rng(42)
    s = rng.standard_normal((300, 256)).astype(np.float32)
    assert all(len(np.unique(r)) == 256 for r in s)
    rc, ids, w = oracle.router_topk(s, 8)
    assert rc == oracle.OK
    t = torch.topk(torch.from_numpy(s).double(), 8, dim=-1)
    assert np.array_equal(ids, t.indices.numpy())
    np.testing.assert_allclose(w, torch.softmax(t.values, dim=-1).numpy(), rtol=2e-7, atol=0)


def test_router_argument_rules():
    s = np.zeros((2, 4), np.float32)
    assert oracle.router_topk(s, 0)[0] == oracle.EINVAL
    assert oracle.router_topk(s, 5)[0] == oracle.EINVAL
    s[1, 2] = np.nan
    assert oracle.router_topk(s, 2)[0] == oracle.EINVAL
    assert oracle.router_topk(np.zeros((0, 4), np.float32), 2)[0] == oracle.OK


# ---------------------------------------------------------------- FP8 dispatch format
# Mooncake PG/EP guide, "Buffer.dispatch": use_fp8 returns FP8 data plus scales.  Reading: OCP E4M3
# codes, one power-of-two scale per 128 values of a row (the smallest 2^k with amax <= 448 * 2^k).

def test_e4m3_hand_codes():
    for c in _load("e4m3_hand.json")["cases"]:
        assert oracle.e4m3_encode(c["value"]) == c["code"], c["why"]
        if c["code"] not in (0, 128):
            assert oracle.e4m3_decode(c["code"]) == c["value"] or c["value"] in (17.0, 19.0, 0.3, 0.0029296875)


def test_e4m3_matches_torch_float8_e4m3fn():
    import torch
    rng = np.random.default_rng(51)
    v = np.concatenate([rng.uniform(-448, 448, 20000), rng.normal(0, 1, 20000), rng.normal(0, 0.01, 20000),
                        [np.float32(oracle.e4m3_decode(c)) for c in range(256) if (c & 0x7F) != 0x7F]]).astype(np.float32)
    ours = np.array([oracle.e4m3_encode(x) for x in v], np.uint8)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(np.array([oracle.e4m3_decode(int(c)) for c in codes], np.float32), dec)


def test_fp8_row_quantisation_round_trips_and_scale_is_minimal():
    rng = np.random.default_rng(52)
    table = np.array([oracle.e4m3_decode(c) for c in range(256)], np.float64)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    n, cols = 6, 512
    codes = rng.choice(finite, size=(n, cols)).astype(np.uint8)
    k = rng.integers(-20, 20, size=(n, cols // 128))
    # every block holds a value in (224, 448] so that its own scale is exactly 2^k
    for r in range(n):
        for b in range(cols // 128):
            codes[r, b * 128 + rng.integers(128)] = oracle.e4m3_encode(float(rng.choice([240.0, 288.0, 448.0])))
    x = (table[codes].reshape(n, cols // 128, 128) * np.ldexp(1.0, k)[:, :, None]).reshape(n, cols)
    xb = synth.f32_to_bf16(x.astype(np.float32))
    assert np.array_equal(synth.bf16_to_f32(xb).astype(np.float64), x)   # exact in bf16
    rc, q, s = oracle.quantize_rows_fp8(xb)
    assert rc == oracle.OK
    assert np.array_equal(s.astype(np.int64) - 127, k)
    assert np.array_equal(oracle.dequantize_rows_fp8(q, s).astype(np.float64), x)
    # on random data: the scale is the smallest power of two that keeps every value within 448
    xr = synth.f32_to_bf16(rng.normal(0, 3, (8, 384)).astype(np.float32))
    xr[2, :128] = 0
    rc, q, s = oracle.quantize_rows_fp8(xr)
    a = np.abs(synth.bf16_to_f32(xr).astype(np.float64)).reshape(8, 3, 128).max(axis=2)
    kk = s.astype(np.int64) - 127
    assert kk[2, 0] == 0 and np.all(q[2, :128] == 0)
    nz = a > 0
    assert np.all(a[nz] <= 448 * np.ldexp(1.0, kk[nz])) and np.all(a[nz] > 224 * np.ldexp(1.0, kk[nz]))
    assert np.all((q & 0x7F) != 0x7F)
    err = np.abs(oracle.dequantize_rows_fp8(q, s).astype(np.float64) - synth.bf16_to_f32(xr))
    # round to nearest: at most half a step, a step being 2^(e-3) * 2^k for a value in [2^e, 2^(e+1))
    mag = np.abs(synth.bf16_to_f32(xr).astype(np.float64)) * np.ldexp(1.0, -np.repeat(kk, 128, axis=1))
    e = np.maximum(np.floor(np.log2(np.maximum(mag, 1e-30))), -6).astype(np.int64)
    step = np.ldexp(1.0, e - 3) * np.ldexp(1.0, np.repeat(kk, 128, axis=1))
    assert np.all(err <= step / 2 + 1e-30)
