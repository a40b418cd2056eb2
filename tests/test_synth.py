"""The seeded input generator (no GPU): published SplitMix64 outputs, distribution
shape, slice consistency, and the routing recipe (distinct picks, softmax weights)."""
import numpy as np

import synth


def test_splitmix64_published_sequence():
    # SplitMix64 (Steele, Lea & Flood 2014) from state 1234567: the first three
    # outputs listed with the public reference implementation.
    assert synth.raw_key(1234567, 0, 3).tolist() == [6457827717110365317, 3203168211198807973,
                                                      9817491932198370423]


def test_counter_based_slices_agree():
    full = synth.normal_bf16(2024, synth.TAG_W_GATE_UP, 0, 10000, 0.1)
    part = synth.normal_bf16(2024, synth.TAG_W_GATE_UP, 4000, 3000, 0.1)
    assert np.array_equal(full[4000:7000], part)
    w1a, w2a = synth.expert_weights(8, 8, 0, 128, 64)
    w1b, w2b = synth.expert_weights(8, 2, 3, 128, 64)
    assert np.array_equal(w1a[6:8], w1b) and np.array_equal(w2a[6:8], w2b)


def test_normal_moments():
    z = synth.normal_f32(1, 9, 0, 400000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert abs(((z > 1.959964) | (z < -1.959964)).mean() - 0.05) < 0.003


def test_tokens_follow_source_rank_seed():
    x = synth.tokens(4, 12, 128)
    r1 = synth.normal_bf16(1001, synth.TAG_X, 0, 4 * 128).reshape(4, 128)
    assert np.array_equal(x[4:8], r1)


def test_routing_recipe():
    ids, w = synth.routing(64, 512, 32, 6)
    assert ids.min() >= 0 and ids.max() < 32
    assert all(len(set(r)) == 6 for r in ids.tolist())
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-6)
    assert np.all(w > 0)
    # uniform: every expert about equally popular
    c = np.bincount(ids.ravel(), minlength=32)
    assert c.min() > 0.6 * c.mean() and c.max() < 1.4 * c.mean()


def test_zipf_routing_is_skewed():
    ids, _ = synth.routing(4096, 4096, 256, 8, zipf_s=1.1)
    c = np.bincount(ids.ravel(), minlength=256)
    assert all(len(set(r)) == 8 for r in ids[:200].tolist())
    assert c[0] > c[1] > c[4] > c[31] > c[255]
    # expert 0 is in nearly every token's top-8 (p_0 ~ 0.17 of the mass, drawn without replacement)
    assert c[0] > 0.85 * 4096


def test_bench_counts_from_routing():
    # bench.py's host counts of local picks, tokens with a local pick and local experts with rows,
    # on a hand-made routing: rank 1 of 4 (experts 4..7), one masked-out source rank
    import sys, os
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    cfg = synth.Config("t", "FLAT", 16, 4, 1, 2, 6, 128, 64, 2)
    ids = np.array([[4, 0], [5, 4], [1, 2], [7, 7], [6, 9], [4, 5]], dtype=np.int64)
    assert bench.algorithmic_units(cfg, ids) == (8, 5)
    assert bench.experts_with_rows(cfg, ids) == 4
    mask = np.array([1, 0, 1], dtype=np.int32)  # source rank 1 holds tokens 2 and 3
    assert bench.algorithmic_units(cfg, ids, mask) == (6, 4)
    assert bench.experts_with_rows(cfg, ids, mask) == 3  # expert 7's picks are all in token 3
    mask = np.array([0, 1, 0], dtype=np.int32)
    assert bench.algorithmic_units(cfg, ids, mask) == (2, 1)
    assert bench.experts_with_rows(cfg, ids, mask) == 1


def test_bench_gate_up_roofline_bound():
    # bench.py's roofline of the gate_up GEMM: MFMA-bound with thousands of rows per expert, HBM-bound
    # (weight streaming) with a few dozen; the byte count written out by hand for the decode case
    import sys, os
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    pre = synth.CONFIGS["prefill_flat_zipf"]
    r = bench.gate_up_roofline(pre, 173420, 32, 7.1026, False, None)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and "256-row" in r["kernel"]
    assert abs(r["achieved"] - 4 * 173420 * 2048 * 7168 / 7.1026e-3 / 1e12) < 0.1
    dec = synth.CONFIGS["decode_expert_major"]
    r = bench.gate_up_roofline(dec, 1008, 32, 0.33052, False, None)
    # W1 of 32 experts (2 x 2048 rows of 7168 bf16) + 1008 A rows (7168 bf16) + 1008 h rows (2048 bf16)
    nbytes = 32 * 2 * 2048 * 7168 * 2 + 1008 * 7168 * 2 + 1008 * 2048 * 2
    assert nbytes == 1_897_627_648
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and "64-row" in r["kernel"]
    assert r["algorithmic_bytes"] == nbytes
    assert abs(r["achieved"] - nbytes / 0.33052e-3 / 1e9) < 0.1 and r["peak"] == 8000


def test_bench_down_roofline_bound():
    # bench.py's roofline of the down GEMM: MFMA-bound on the prefill share, HBM-bound (W2 streaming)
    # on the rank-major share; the byte count written out by hand for the latter
    import sys, os
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    pre = synth.CONFIGS["prefill_flat_zipf"]
    r = bench.down_roofline(pre, 173420, 32, 3.8)
    assert r["bound"] == "mfma" and abs(r["achieved"] - 2 * 173420 * 2048 * 7168 / 3.8e-3 / 1e12) < 0.1
    rm = synth.CONFIGS["rank_major"]
    r = bench.down_roofline(rm, 1536, 8, 0.0428)
    # W2 of 8 experts (4096 rows of 1408 bf16) + 1536 h rows (1408 bf16) read + 1536 y rows (4096 bf16)
    nbytes = 8 * 4096 * 1408 * 2 + 1536 * 1408 * 2 + 1536 * 4096 * 2
    assert r["bound"] == "hbm" and r["algorithmic_bytes"] == nbytes
    assert abs(r["achieved"] - nbytes / 0.0428e-3 / 1e9) < 0.1
