"""Pins for the fp64 oracle, each against something other than the oracle.

CPU only.  The pins are chosen so that a plausible slip in the oracle (a
dropped scale, a wrong KV-head group, a transposed operand, a missed max
shift, an off-by-one in the table gather, a wrong slot formula) breaks at
least one of them; tests/test_oracle_mutants.py checks that claim by planting
such slips in copies of the oracle.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


def _paged(logical_k, logical_v, block_size, num_blocks, rng, fill=np.nan):
    """Scatter per-sequence contiguous caches into a pool through random tables.

    logical_k[s] is [ctx_s, Hkv, d].  Logical block j of sequence s is stored
    whole in physical block tables[s][j]; every physical block is used once.
    """
    batch = len(logical_k)
    hkv, d = logical_k[0].shape[1:]
    nblk = [-(-k.shape[0] // block_size) for k in logical_k]
    perm = rng.permutation(num_blocks).astype(np.int32)
    assert sum(nblk) <= num_blocks
    tables = np.zeros((batch, max(1, max(nblk))), np.int32)
    pool_k = np.full((num_blocks, block_size, hkv, d), fill, np.float16)
    pool_v = np.full((num_blocks, block_size, hkv, d), fill, np.float16)
    nxt = 0
    for s in range(batch):
        ctx = logical_k[s].shape[0]
        for j in range(nblk[s]):
            pb = perm[nxt]
            nxt += 1
            tables[s, j] = pb
            lo, hi = j * block_size, min(ctx, (j + 1) * block_size)
            pool_k[pb, :hi - lo] = logical_k[s][lo:hi]
            pool_v[pb, :hi - lo] = logical_v[s][lo:hi]
    shape = (num_blocks * block_size, hkv, d)
    return pool_k.reshape(shape), pool_v.reshape(shape), tables


def _brute(q, k, v, scale):
    """Two-pass softmax attention for one sequence over a contiguous cache.

    q [Hq, d], k/v [ctx, Hkv, d]; written with plain Python loops.
    """
    hq, d = q.shape
    ctx, hkv, _ = k.shape
    grp = hq // hkv
    out = np.zeros((hq, d))
    for h in range(hq):
        g = h // grp
        logits = []
        for t in range(ctx):
            acc = 0.0
            for i in range(d):
                acc += float(q[h, i]) * float(k[t, g, i])
            logits.append(acc * scale)
        if ctx == 0:
            continue
        top = max(logits)
        weights = [math.exp(x - top) for x in logits]
        total = sum(weights)
        for i in range(d):
            out[h, i] = sum(weights[t] * float(v[t, g, i]) for t in range(ctx)) / total
    return out


# --------------------------------------------------------------------------
# binary16 decoding
# --------------------------------------------------------------------------
def test_f16_decoder_matches_numpy_on_every_bit_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    ours = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


# --------------------------------------------------------------------------
# the pages' worked numbers
# --------------------------------------------------------------------------
def test_slot_example_from_the_pages():
    g = _golden("slot_example.json")
    bs = g["block_size"]
    for req, pos, want in g["cases"]:
        assert oracle.slot(g["tables"][req], bs, pos) == want
    unused = sum(len(t) * bs - g["tokens"][r] for r, t in g["tables"].items())
    assert unused == g["reserved_but_unused_slots"]


def test_sizing_figures_from_the_pages():
    g = _golden("kv_sizing.json")
    p = g["page_bytes"]
    page = oracle.page_bytes(p["block_size"], p["kv_heads"], p["key_dim"], p["value_dim"],
                             p["bytes_per_value"])
    assert page == p["expected"]
    assert page * p["layers"] // 1024 == p["expected_all_layers_kib"]
    page8 = oracle.page_bytes(p["block_size"], p["kv_heads"], p["key_dim"], p["value_dim"],
                              p["fp8_bytes_per_value"])
    assert page8 * p["layers"] // 1024 == p["expected_fp8_all_layers_kib"]
    t = g["kv_per_token"]
    assert oracle.kv_bytes_per_token(t["layers"], t["kv_heads"], t["head_dim"],
                                     t["bytes_per_value"]) == t["expected"] == 128 * 1024
    ll = g["tiny_llama_log"]
    total = ll["cells"] * oracle.kv_bytes_per_token(ll["layers"], ll["kv_heads"], ll["head_dim"],
                                                    ll["bytes_per_value"])
    assert total == ll["expected_total_bytes"]
    assert total // 2 == ll["expected_k_bytes"]


# --------------------------------------------------------------------------
# brute force and a library routine
# --------------------------------------------------------------------------
@pytest.mark.parametrize("ctx_lens", [[1, 3, 4], [5, 9, 2], [4, 8, 13]])
def test_matches_brute_force_over_contiguous_cache(ctx_lens):
    rng = np.random.default_rng(sum(ctx_lens))
    hq, hkv, d, bs = 4, 2, 8, 4
    q = _f16(rng, (len(ctx_lens), hq, d))
    lk = [_f16(rng, (c, hkv, d)) for c in ctx_lens]
    lv = [_f16(rng, (c, hkv, d)) for c in ctx_lens]
    kp, vp, tables = _paged(lk, lv, bs, 16, rng)
    got = oracle.decode(q, kp, vp, tables, np.array(ctx_lens, np.int32), 1 / math.sqrt(d), bs)
    for s in range(len(ctx_lens)):
        want = _brute(q[s], lk[s], lv[s], 1 / math.sqrt(d))
        np.testing.assert_allclose(got[s], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8), (16, 2)])
def test_matches_torch_sdpa_in_fp64(hq, hkv):
    rng = np.random.default_rng(hq * 100 + hkv)
    d, bs = 128, 16
    ctx_lens = [1, 17, 64, 250]
    q = _f16(rng, (len(ctx_lens), hq, d))
    lk = [_f16(rng, (c, hkv, d), 2.0) for c in ctx_lens]
    lv = [_f16(rng, (c, hkv, d)) for c in ctx_lens]
    kp, vp, tables = _paged(lk, lv, bs, 64, rng)
    scale = 1 / math.sqrt(d)
    got = oracle.decode(q, kp, vp, tables, np.array(ctx_lens, np.int32), scale, bs)
    for s, c in enumerate(ctx_lens):
        qt = torch.from_numpy(q[s].astype(np.float64))[None, :, None, :]
        kt = torch.from_numpy(lk[s].astype(np.float64)).permute(1, 0, 2)
        vt = torch.from_numpy(lv[s].astype(np.float64)).permute(1, 0, 2)
        kt = kt.repeat_interleave(hq // hkv, dim=0)[None]
        vt = vt.repeat_interleave(hq // hkv, dim=0)[None]
        want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        np.testing.assert_allclose(got[s], want[0, :, 0, :].numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# invariants and closed forms
# --------------------------------------------------------------------------
def _random_case(seed, ctx_lens, hq=8, hkv=2, d=16, bs=4, pool=64):
    rng = np.random.default_rng(seed)
    q = _f16(rng, (len(ctx_lens), hq, d))
    lk = [_f16(rng, (c, hkv, d)) for c in ctx_lens]
    lv = [_f16(rng, (c, hkv, d)) for c in ctx_lens]
    kp, vp, tables = _paged(lk, lv, bs, pool, rng)
    return rng, q, lk, lv, kp, vp, tables, np.array(ctx_lens, np.int32), bs


def test_block_relabelling_is_bitwise_invariant():
    rng, q, _, _, kp, vp, tables, lens, bs = _random_case(1, [7, 16, 33, 2])
    scale = 0.25
    base = oracle.decode(q, kp, vp, tables, lens, scale, bs)
    nb = kp.shape[0] // bs
    pi = rng.permutation(nb)
    kb = kp.reshape(nb, bs, *kp.shape[1:])
    vb = vp.reshape(nb, bs, *vp.shape[1:])
    k2 = np.empty_like(kb)
    v2 = np.empty_like(vb)
    k2[pi] = kb
    v2[pi] = vb
    t2 = pi[tables].astype(np.int32)
    moved = oracle.decode(q, k2.reshape(kp.shape), v2.reshape(vp.shape), t2, lens, scale, bs)
    assert np.array_equal(base, moved)


def test_context_of_one_returns_v0_exactly():
    _, q, lk, lv, kp, vp, tables, lens, bs = _random_case(2, [1, 1, 1])
    got = oracle.decode(q, kp, vp, tables, lens, 0.3, bs)
    grp = q.shape[1] // lv[0].shape[1]
    for s in range(3):
        for h in range(q.shape[1]):
            assert np.array_equal(got[s, h], lv[s][0, h // grp].astype(np.float64))


def test_identical_keys_average_values():
    rng, q, lk, lv, _, _, _, _, bs = _random_case(3, [5, 12, 31])
    lk = [np.broadcast_to(k[:1], k.shape).copy() for k in lk]
    kp, vp, tables = _paged(lk, lv, bs, 64, rng)
    lens = np.array([5, 12, 31], np.int32)
    got = oracle.decode(q, kp, vp, tables, lens, 0.7, bs)
    grp = q.shape[1] // lv[0].shape[1]
    for s in range(3):
        mean = lv[s].astype(np.float64).mean(axis=0)
        for h in range(q.shape[1]):
            np.testing.assert_allclose(got[s, h], mean[h // grp], rtol=0, atol=1e-13)


def test_two_tokens_closed_form():
    _, q, lk, lv, kp, vp, tables, lens, bs = _random_case(4, [2, 2])
    scale = 0.5
    got = oracle.decode(q, kp, vp, tables, lens, scale, bs)
    grp = q.shape[1] // lv[0].shape[1]
    for s in range(2):
        for h in range(q.shape[1]):
            g = h // grp
            z = [scale * float(np.dot(q[s, h].astype(np.float64), lk[s][t, g].astype(np.float64)))
                 for t in range(2)]
            sig = 1.0 / (1.0 + math.exp(-(z[1] - z[0])))
            want = sig * lv[s][1, g].astype(np.float64) + (1 - sig) * lv[s][0, g].astype(np.float64)
            np.testing.assert_allclose(got[s, h], want, rtol=0, atol=1e-14)


def test_scaling_values_scales_output():
    _, q, _, _, kp, vp, tables, lens, bs = _random_case(5, [9, 21])
    a = oracle.decode(q, kp, vp, tables, lens, 0.4, bs)
    b = oracle.decode(q, kp, (vp.astype(np.float32) * 2).astype(np.float16), tables, lens, 0.4, bs)
    assert np.array_equal(2 * a, b)


def test_equal_heads_in_a_group_agree_and_groups_are_contiguous():
    _, q, _, lv, kp, vp, tables, lens, bs = _random_case(6, [11, 40], hq=8, hkv=2)
    q[:, 1] = q[:, 0]          # heads 0,1 share KV head 0 (contiguous groups of 4)
    q[:, 4] = q[:, 0]          # head 4 uses KV head 1
    got = oracle.decode(q, kp, vp, tables, lens, 0.3, bs)
    assert np.array_equal(got[:, 0], got[:, 1])
    assert not np.allclose(got[:, 0], got[:, 4])


def test_logical_token_order_does_not_matter():
    rng, q, lk, lv, _, _, _, _, bs = _random_case(7, [13, 29])
    lens = np.array([13, 29], np.int32)
    kp, vp, tables = _paged(lk, lv, bs, 64, rng)
    a = oracle.decode(q, kp, vp, tables, lens, 0.3, bs)
    perms = [rng.permutation(c) for c in lens]
    kp2, vp2, t2 = _paged([k[p] for k, p in zip(lk, perms)], [v[p] for v, p in zip(lv, perms)],
                          bs, 64, rng)
    b = oracle.decode(q, kp2, vp2, t2, lens, 0.3, bs)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_softmax_is_max_shifted():
    """Huge logits overflow a naive exp; the max-shifted form stays finite."""
    _, q, lk, lv, _, _, _, _, bs = _random_case(8, [6])
    rng = np.random.default_rng(0)
    lk = [np.full_like(lk[0], 60.0)]
    lk[0][3] = 64.0
    kp, vp, tables = _paged(lk, lv, bs, 16, rng)
    q = np.full_like(q, 16.0)
    got = oracle.decode(q, kp, vp, tables, np.array([6], np.int32), 1.0, bs)
    grp = q.shape[1] // lv[0].shape[1]
    assert np.all(np.isfinite(got))
    for h in range(q.shape[1]):
        np.testing.assert_array_equal(got[0, h], lv[0][3, h // grp].astype(np.float64))


def test_empty_context_gives_zeros_and_skips_the_table():
    _, q, _, _, kp, vp, tables, _, bs = _random_case(9, [4, 4])
    tables[1, :] = 10 ** 6      # never read when ctx is 0
    got = oracle.decode(q, kp, vp, tables, np.array([4, 0], np.int32), 0.3, bs)
    assert np.all(got[1] == 0.0)
    assert np.all(np.isfinite(got[0]))


def test_rejects_tables_outside_the_pool():
    _, q, _, _, kp, vp, tables, lens, bs = _random_case(10, [4, 8])
    tables[1, 1] = kp.shape[0] // bs
    with pytest.raises(ValueError):
        oracle.decode(q, kp, vp, tables, lens, 0.3, bs)


def test_shared_blocks_and_nan_outside_context_are_harmless():
    """Two sequences point at the same blocks; slots past ctx hold NaN."""
    rng = np.random.default_rng(11)
    hq, hkv, d, bs = 8, 2, 16, 4
    q = _f16(rng, (2, hq, d))
    lk = [_f16(rng, (10, hkv, d))]
    lv = [_f16(rng, (10, hkv, d))]
    kp, vp, tables = _paged(lk, lv, bs, 8, rng, fill=np.nan)
    tables = np.repeat(tables, 2, axis=0)
    lens = np.array([10, 10], np.int32)
    got = oracle.decode(q, kp, vp, tables, lens, 0.3, bs)
    assert np.all(np.isfinite(got))
    for s in range(2):
        np.testing.assert_allclose(got[s], _brute(q[s], lk[0], lv[0], 0.3), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# the compact relabelled cache the GPU tests hand to the oracle
# --------------------------------------------------------------------------
@pytest.mark.parametrize("shuffle", [False, True])
def test_relabelled_cache_matches_the_uncompacted_slot_cache(shuffle):
    """oracle.relabelled_cache compacts the referenced blocks into blocks
    0..n-1 and rewrites the tables.  Against the full slot-indexed cache of the
    pool (host_cache: every referenced block at its own id, NaN elsewhere) and
    the original tables it must give the same gathered rows and the same
    decode, bit for bit -- also with block ids listed out of order and with
    blocks shared by several tables."""
    import workloads

    for w in (workloads.custom([1, 15, 16, 17, 0, 40, 33], seed=41),
              workloads.custom([40, 48, 35, 64], seed=42, prefix_groups=(2, 2, 2))):
        B = w.block_size
        ids, k, v = w.kv_blocks(0)
        if shuffle:
            p = np.random.default_rng(5).permutation(len(ids))
            ids, k, v = ids[p], k[p], v[p]
        tables, lens, q = w.tables(0), w.ctx_lens, w.q(0)
        full_k = oracle.host_cache(w.pool_blocks, B, ids, k)
        full_v = oracle.host_cache(w.pool_blocks, B, ids, v)
        kc, vc, t2 = oracle.relabelled_cache(ids, k, v, tables, lens, B)
        held = w.blocks_held()
        for s in range(w.batch):
            for j in range(int(held[s])):
                a, b = int(tables[s, j]) * B, int(t2[s, j]) * B
                assert np.array_equal(kc[b:b + B].view(np.uint16), full_k[a:a + B].view(np.uint16))
                assert np.array_equal(vc[b:b + B].view(np.uint16), full_v[a:a + B].view(np.uint16))
            assert np.all(t2[s, int(held[s]):] == 0)
        ref = oracle.decode(q, full_k, full_v, tables, lens, w.scale, B)
        got = oracle.decode(q, kc, vc, t2, lens, w.scale, B)
        assert np.array_equal(ref.view(np.uint64), got.view(np.uint64))
        assert np.all(np.isfinite(ref))


def test_relabelled_cache_rejects_tables_naming_missing_blocks():
    import workloads

    w = workloads.custom([20, 40], seed=43)
    ids, k, v = w.kv_blocks(0)
    with pytest.raises(ValueError):
        oracle.relabelled_cache(ids[1:], k[1:], v[1:], w.tables(0), w.ctx_lens, w.block_size)
