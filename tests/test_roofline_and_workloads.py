"""CPU tests: the pages' roofline table and the seeded workload generator."""
import json
import os

import numpy as np

import workloads
from paged_kv_cache_64_amd import roofline

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_roofline_model_reproduces_the_pages_table():
    with open(os.path.join(GOLDEN, "roofline_rtx4090.json")) as f:
        g = json.load(f)
    x = g["inputs"]
    fmt = {"bytes_per_step_GB": "%.2f", "step_ms": "%.2f", "tok_s_total": "%.0f",
           "tok_s_per_seq": "%.1f", "flop_util_pct": "%.2f"}
    for row in g["rows"]:
        r = roofline.decode_step_model(x["params"], x["bits_per_weight"], x["peak_flops"],
                                       x["bandwidth"], x["context"], x["kv_bytes_per_token"],
                                       row[0])
        for col, want in zip(g["columns"][1:], row[1:]):
            assert fmt[col] % r[col] == want, (row[0], col)
        if row[0] == 32:
            assert "%.2f" % r["kv_GB"] == g["kv_gb_at_batch_32"]
    assert roofline.sequences_that_fit(x["params"], x["bits_per_weight"], x["vram_bytes"],
                                       x["context"], x["kv_bytes_per_token"]) == g["sequences_that_fit"]


def test_kv_bytes_per_token_layer_is_4_kib_for_8b():
    assert roofline.kv_bytes_per_token_layer(8, 128) * 32 == 128 * 1024


def test_configs_are_deterministic_and_shaped():
    for k in (1, 2, 4, 5):
        a, b = workloads.config(k), workloads.config(k)
        assert np.array_equal(a.ctx_lens, b.ctx_lens)
        assert np.array_equal(a.tables(0), b.tables(0))
        assert np.array_equal(a.q(0), b.q(0))
        assert a.q(0).shape == (a.batch, 32, 128) and a.q(0).dtype == np.float16
    assert workloads.config(1).batch == 1 and workloads.config(1).max_context_len == 256
    assert workloads.config(2).batch == 8 and workloads.config(3).layers == 32
    assert workloads.config(3).batch == 32
    c4 = workloads.config(4)
    assert c4.batch == 64 and c4.ctx_lens.min() >= 1 and c4.ctx_lens.max() <= 8192
    assert np.any(c4.ctx_lens % 16 != 0)
    c5 = workloads.config(5)
    assert c5.batch == 256 and c5.ctx_lens.min() >= 2048 and c5.ctx_lens.max() <= 2048 + 6144
    c8 = workloads.config(8)
    assert c8.layers == 32 and c8.batch == 1 and c8.max_context_len == 256 and c8.pool_blocks == 64
    assert not np.array_equal(c8.tables(0), c8.tables(1))       # a fresh table per layer
    assert all(len(np.unique(c8.tables(L)[0])) == 16 for L in (0, 31))
    c9 = workloads.config(9)
    assert c9.layers == 1 and c9.batch == 1024 and np.all(c9.ctx_lens == 128) and c9.max_blocks == 8


def test_tables_are_distinct_non_contiguous_and_inside_the_pool():
    for k in (1, 2, 4, 9):
        w = workloads.config(k)
        t = w.tables(0)
        held = w.blocks_held()
        used = np.concatenate([t[s, :held[s]] for s in range(w.batch)])
        assert used.min() >= 0 and used.max() < w.pool_blocks
        assert len(np.unique(used)) == len(used)
        row = t[0, :held[0]]
        assert np.any(np.diff(row) != 1)
    c1 = workloads.config(1)
    assert c1.pool_blocks == 64 and c1.tables(0).shape == (1, 16)


def test_fresh_tables_per_layer():
    w = workloads.custom([64, 64], layers=3, seed=7)
    w.fresh_tables_per_layer = True
    assert not np.array_equal(w.tables(0), w.tables(1))


def test_prefix_groups_share_blocks_with_refcount_16():
    w = workloads.config(5)
    t = w.tables(0)
    held = w.blocks_held()
    ids, counts = np.unique(np.concatenate([t[s, :held[s]] for s in range(w.batch)]),
                            return_counts=True)
    assert set(np.unique(counts)) == {1, 16}
    assert int((counts == 16).sum()) == 16 * 128
    for grp in range(16):
        rows = t[grp * 16:(grp + 1) * 16, :128]
        assert np.all(rows == rows[0])


def test_block_values_are_consistent_for_subsets_and_f16_normal():
    w = workloads.custom([300, 17, 1000], seed=3)
    ids, k, v = w.kv_blocks(0)
    sub = ids[[0, 5, len(ids) - 1]]
    ids2, k2, v2 = w.kv_blocks(0, sub)
    assert np.array_equal(k2, k[[0, 5, len(ids) - 1]])
    assert np.array_equal(v2, v[[0, 5, len(ids) - 1]])
    x = k.astype(np.float64).ravel()
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_key_boost_hits_about_one_percent_of_key_vectors():
    w = workloads.custom([4096] * 4, seed=5, key_boost_prob=0.01)
    ids, k, v = w.kv_blocks(0)
    norms = np.linalg.norm(k.astype(np.float32), axis=-1)
    frac = float((norms > 4 * np.sqrt(128)).mean())
    assert 0.007 < frac < 0.013
    vn = np.linalg.norm(v.astype(np.float32), axis=-1)
    assert float((vn > 4 * np.sqrt(128)).mean()) == 0.0


def test_pages_context_rows_are_the_printed_table():
    with open(os.path.join(GOLDEN, "roofline_rtx4090.json")) as f:
        g = json.load(f)
    ctx = roofline.pages_context()
    for row, want in zip(ctx["rows"], g["rows"]):
        assert row["batch"] == want[0]
        assert "%.2f" % row["bytes_per_step_GB"] == want[1] and "%.2f" % row["rtx4090_step_ms"] == want[2]
    assert "%.2f" % ctx["rows"][-1]["kv_GB"] == g["kv_gb_at_batch_32"]
    # at MI355X's 8 TB/s the batch-32 step is bandwidth-bound too: 21.70 GB / 8 TB/s
    assert abs(ctx["rows"][-1]["mi355x_peak_step_ms"] - 21.70e9 / 8e12 * 1e3) < 0.01


def test_split_kernel_bytes_counts_every_stream_once():
    b = roofline.split_kernel_bytes([4096] * 32, 32, 8, 128, 16)
    assert b["kv"] == 32 * 4096 * 4096
    assert b["q"] == b["out"] == 32 * 32 * 128 * 2
    assert b["table"] == 32 * 256 * 4
    assert b["total"] == 537165824 + 32 * 8192      # 537,427,968 B per launch
