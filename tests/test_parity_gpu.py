"""GPU parity: libpa (through the C ABI) against the fp64 oracle.

Tolerance for the F16 output: max |err| <= 2e-3 and relative L2 <= 1e-3 over
each case.  Integer and byte work (pa_write_kv) is checked bit-exactly.
"""
import os

import numpy as np
import pytest
import torch

import workloads
import paged_kv_cache_64_amd as pa
from tests.gpu_harness import Staged, compare, report, slots_of, write_blocks

pytestmark = pytest.mark.gpu

RAGGED = [1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 100, 255, 256, 257, 1000, 4097]


@pytest.fixture(autouse=True)
def _no_split_override(monkeypatch):
    monkeypatch.delenv("PA_SPLIT_TOKENS", raising=False)


def _poison_tails(st, layer=0):
    """Writes NaN into the slots of each sequence's last block that lie past its context."""
    w = st.w
    _, tables = st.host[layer][0], st.host[layer][1]
    slots = []
    for s, ctx in enumerate(w.ctx_lens):
        ctx = int(ctx)
        if ctx % w.block_size == 0 or ctx == 0:
            continue
        end = (ctx + w.block_size - 1) // w.block_size * w.block_size
        slots += slots_of(tables[s], range(ctx, end), w.block_size)
    if not slots:
        return 0
    n = len(slots)
    nan = torch.full((n, w.num_kv_heads, w.head_dim), float("nan"), dtype=torch.float16,
                     device="cuda")
    st.pool.write(layer, nan, nan.clone(), torch.tensor(slots, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    return n


def test_write_kv_lands_in_the_documented_layout():
    report("write_kv layout")
    pool = pa.Pool(2, 8, fill=0.0)
    rng = np.random.default_rng(0)
    n = 40
    slots = rng.choice(8 * 16, size=n, replace=False).astype(np.int32)
    slots[3] = -1           # skipped
    slots[7] = 8 * 16       # past the pool: skipped
    k = rng.standard_normal((n, 8, 128)).astype(np.float16)
    v = rng.standard_normal((n, 8, 128)).astype(np.float16)
    pool.write(1, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
               torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    kp = pool.k.cpu().numpy()          # [layer, block, head, offset, dim]
    vp = pool.v.cpu().numpy()
    want_k = np.zeros_like(kp)
    want_v = np.zeros_like(vp)
    for i, sl in enumerate(slots):
        if 0 <= sl < 8 * 16:
            want_k[1, sl // 16, :, sl % 16, :] = k[i]
            want_v[1, sl // 16, :, sl % 16, :] = v[i]
    assert np.array_equal(kp.view(np.uint16), want_k.view(np.uint16))
    assert np.array_equal(vp.view(np.uint16), want_v.view(np.uint16))
    pool.close()


def test_small_ragged_batch_with_poisoned_tails():
    w = workloads.custom(RAGGED, seed=11)
    st = Staged(w)
    npois = _poison_tails(st)
    report("ragged", poisoned_slots=npois, split=st.pool.split_tokens(w.batch, 32, w.max_context_len))
    compare("ragged", st.decode(0), st.reference(0))
    st.close()


@pytest.mark.parametrize("split", [64, 128, 192, 1024, 4096])
def test_split_lengths_agree_with_oracle_and_phases(monkeypatch, split):
    w = workloads.custom(RAGGED, seed=12)
    st = Staged(w)
    _poison_tails(st)
    monkeypatch.setenv("PA_SPLIT_TOKENS", str(split))
    assert st.pool.split_tokens(w.batch, 32, w.max_context_len) == split
    a = st.decode(0)
    b = st.decode(0, phases=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    compare(f"split{split}", a, st.reference(0))
    st.close()


def test_empty_contexts_give_zeros():
    w = workloads.custom([0, 5, 0, 33], seed=13)
    st = Staged(w)
    out = st.decode(0)
    compare("empty", out, st.reference(0))
    assert torch.all(out[0] == 0) and torch.all(out[2] == 0)
    w0 = workloads.custom([0, 0, 0], seed=14)
    w0.pool_blocks = 4
    st0 = Staged(w0)
    out0 = torch.full((3, 32, 128), 7.0, dtype=torch.float16, device="cuda")
    q = torch.zeros_like(out0)
    tables = torch.zeros((3, 1), dtype=torch.int32, device="cuda")
    st0.pool.decode(0, q, out0, tables, st0.lens, 0, 0.1)
    torch.cuda.synchronize()
    assert torch.all(out0 == 0)
    st.close()
    st0.close()


def test_context_of_one_returns_v0_exactly():
    w = workloads.custom([1] * 6, seed=15)
    st = Staged(w)
    _poison_tails(st)
    out = st.decode(0).cpu().numpy()
    _, tables, ids, _, v = st.host[0]
    for s in range(w.batch):
        blk = tables[s, 0]
        v0 = v[np.searchsorted(ids, blk), 0]            # [Hkv, d]
        want = np.repeat(v0, 4, axis=0)                  # contiguous groups of 4 q heads
        assert np.array_equal(out[s].view(np.uint16), want.view(np.uint16))
    st.close()


def test_block_relabelling_is_bitwise_invariant():
    w = workloads.custom(RAGGED[:10], seed=16)
    st = Staged(w)
    a = st.decode(0)
    q, tables, ids, k, v = st.host[0]
    pi = np.random.default_rng(3).permutation(w.pool_blocks).astype(np.int32)
    st2 = Staged(w)
    st2.pool.k.fill_(float("nan"))
    st2.pool.v.fill_(float("nan"))
    write_blocks(st2.pool, 0, pi[ids], k, v)
    held = w.blocks_held()
    t2 = tables.copy()
    for s in range(w.batch):
        t2[s, :held[s]] = pi[tables[s, :held[s]]]
    st2.dev[0] = (st2.dev[0][0], torch.from_numpy(t2).cuda())
    b = st2.decode(0)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    st.close()
    st2.close()


def test_doubling_values_doubles_output_exactly():
    w = workloads.custom(RAGGED[:12], seed=17)
    st = Staged(w)
    a = st.decode(0)
    q, tables, ids, k, v = st.host[0]
    write_blocks(st.pool, 0, ids, k, v * np.float16(2))
    b = st.decode(0)
    # exact wherever F16 keeps full precision (2x commutes with rounding there)
    normal = a.float().abs() >= 2.0 ** -13
    assert torch.equal((a.float() * 2).half()[normal].view(torch.int16), b[normal].view(torch.int16))
    assert torch.all(((a.float() * 2) - b.float()).abs()[~normal] <= 2.0 ** -24)
    st.close()


def test_shared_prefix_blocks_and_duplicate_entries():
    lens = [48 + x for x in (0, 5, 16, 40, 77, 1)]
    w = workloads.custom(lens, seed=18, prefix_groups=(2, 3, 3))
    st = Staged(w)
    _poison_tails(st)
    compare("shared", st.decode(0), st.reference(0))
    # one table naming the same physical block twice
    q, tables, ids, k, v = st.host[0]
    tables = tables.copy()
    tables[0, 1] = tables[0, 0]
    st.host[0] = (q, tables, ids, k, v)
    st.dev[0] = (st.dev[0][0], torch.from_numpy(tables).cuda())
    compare("duplicate", st.decode(0), st.reference(0))
    st.close()


def test_lengths_past_the_hint_are_truncated():
    w = workloads.custom([300, 90, 17], seed=19)
    st = Staged(w)
    out = st.decode(0, max_context_len=100)
    w_trunc = np.minimum(w.ctx_lens, 100)
    saved = w.ctx_lens
    w.ctx_lens = w_trunc
    ref = st.reference(0)
    w.ctx_lens = saved
    compare("truncated", out, ref)
    st.close()


@pytest.mark.parametrize("k", [1, 2, 4, 5])
def test_config_full_parity(k):
    w = workloads.config(k)
    st = Staged(w)
    split = st.pool.split_tokens(w.batch, 32, w.max_context_len)
    report(f"config{k}", batch=w.batch, max_ctx=w.max_context_len, split=split)
    compare(f"config{k}", st.decode(0, phases=True), st.reference(0))
    st.close()


def test_config3_three_whole_layers():
    """The 32-layer pool at full size; three layers are written and every
    sequence of each is checked (the other layers hold NaN and are never
    read)."""
    w = workloads.config(3)
    layers = (0, 17, 31)
    st = Staged(w, layers=layers, pool_layers=32)
    for layer in layers:
        out = st.decode(layer, phases=True)
        compare(f"config3 layer{layer} all {w.batch} sequences", out, st.reference(layer))
    st.close()


@pytest.mark.parametrize("fp8", [False, True])
def test_config3_timed_launch_whole_layers(fp8):
    """The timed step's launch configuration at full size: the 32-layer pool of
    batch 32 x ctx 4096, one plan for the step, and pa_decode_run appending
    each sequence's newest token, on layers 0 and 31 (the other layers hold
    NaN and are never read).  Every sequence of both layers is checked against
    the oracle with the appended rows in place."""
    w = workloads.config(3)
    layers = (0, 31)
    kw = dict(dtype=pa.PA_FP8_E4M3, kv_scales=(0.1, 0.0173)) if fp8 else {}
    st = Staged(w, layers=layers, pool_layers=32, **kw)
    plan = st.pool.plan(w.ctx_lens)
    assert plan.info.num_items == 32 and plan.info.num_merges == 0
    rng = np.random.default_rng(12)
    for layer in layers:
        q, tables, ids, k, v = st.host[layer]
        k_new = rng.standard_normal((w.batch, 8, 128)).astype(np.float16)
        v_new = rng.standard_normal((w.batch, 8, 128)).astype(np.float16)
        qd, td = st.dev[layer]
        out = torch.empty_like(qd)
        st.pool.run(layer, plan, qd, out, td, w.scale, k_new=torch.from_numpy(k_new).cuda(),
                    v_new=torch.from_numpy(v_new).cuda())
        torch.cuda.synchronize()
        k2, v2 = k.copy(), v.copy()
        for s, c in enumerate(w.ctx_lens):
            r = np.searchsorted(ids, tables[s, (c - 1) // 16])
            k2[r, (c - 1) % 16] = k_new[s]
            v2[r, (c - 1) % 16] = v_new[s]
        st.host[layer] = (q, tables, ids, k2, v2)
        compare(f"config3 timed launch fp8={fp8} layer{layer} all {w.batch} sequences", out,
                st.reference(layer))
        del k2, v2
    st.close()


@pytest.mark.parametrize("split", [None, 64, 256])
def test_append_decode_writes_the_newest_token_and_attends_to_it(monkeypatch, split):
    """pa_append_decode == pa_write_kv(newest slots) + pa_decode, with fresh K/V
    for each sequence's newest position (the pool holds other values there)."""
    if split:
        monkeypatch.setenv("PA_SPLIT_TOKENS", str(split))
    lens = [1, 16, 17, 100, 257, 1000, 0, 4097]
    w = workloads.custom(lens, seed=21)
    st = Staged(w)
    _poison_tails(st)
    q, tables, ids, k, v = st.host[0]
    rng = np.random.default_rng(5)
    k_new = rng.standard_normal((w.batch, 8, 128)).astype(np.float16)
    v_new = rng.standard_normal((w.batch, 8, 128)).astype(np.float16)
    qd, td = st.dev[0]
    out = torch.empty_like(qd)
    st.pool.decode(0, qd, out, td, st.lens, w.max_context_len, w.scale,
                   k_new=torch.from_numpy(k_new).cuda(), v_new=torch.from_numpy(v_new).cuda())
    torch.cuda.synchronize()
    # the oracle sees the new values in the newest slots
    k2, v2 = k.copy(), v.copy()
    newest = []
    for s, c in enumerate(lens):
        if c == 0:
            continue
        blk = tables[s, (c - 1) // 16]
        r = np.searchsorted(ids, blk)
        k2[r, (c - 1) % 16] = k_new[s]
        v2[r, (c - 1) % 16] = v_new[s]
        newest.append((s, blk, (c - 1) % 16))
    st.host[0] = (q, tables, ids, k2, v2)
    compare(f"append split={split}", out, st.reference(0))
    # the pool now holds them (bit-exact), in the documented layout
    kp = st.pool.k[0].cpu().numpy()
    vp = st.pool.v[0].cpu().numpy()
    for s, blk, off in newest:
        assert np.array_equal(kp[blk, :, off, :].view(np.uint16), k_new[s].view(np.uint16))
        assert np.array_equal(vp[blk, :, off, :].view(np.uint16), v_new[s].view(np.uint16))
    # and a read-only decode afterwards gives the same bits
    again = st.decode(0)
    assert torch.equal(again.view(torch.int16), out.view(torch.int16))
    # phases: partial (with new K/V) + merge give the same bits too
    out3 = torch.empty_like(qd)
    st.pool.decode(0, qd, out3, td, st.lens, w.max_context_len, w.scale, phases=True,
                   k_new=torch.from_numpy(k_new).cuda(), v_new=torch.from_numpy(v_new).cuda())
    torch.cuda.synchronize()
    assert torch.equal(out3.view(torch.int16), out.view(torch.int16))
    st.close()


def _planned(st, layer=0, k_new=None, v_new=None, wave_heads=None):
    plan = st.pool.plan(st.w.ctx_lens)
    if wave_heads is not None:  # override the planner's choice of per-wave KV heads
        plan.info.decode_wave_heads = wave_heads
    q, tables = st.dev[layer]
    out = torch.empty_like(q)
    st.pool.run(layer, plan, q, out, tables, st.w.scale, k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    return out, plan


def test_planned_run_ragged_with_poisoned_tails():
    w = workloads.custom(RAGGED + [0, 3, 8192], seed=31, max_blocks=520)
    st = Staged(w)
    _poison_tails(st)
    out, plan = _planned(st)
    report("planned ragged", items=plan.info.num_items, merges=plan.info.num_merges,
           longest=plan.info.max_piece_tokens)
    compare("planned ragged", out, st.reference(0))
    st.close()


@pytest.mark.parametrize("k", [1, 2, 4, 5, 9])
def test_planned_run_configs(k):
    w = workloads.config(k)
    st = Staged(w)
    out, plan = _planned(st)
    assert plan.info.decode_wave_heads == (1 if k == 9 else 0)  # workload 9: per-wave KV heads
    report(f"planned config{k}", items=plan.info.num_items, merges=plan.info.num_merges,
           longest=plan.info.max_piece_tokens)
    compare(f"planned config{k}", out, st.reference(0))
    st.close()


def test_planned_uniform_batch_equals_single_split_decode_bitwise():
    w = workloads.custom([4096] * 32, seed=32)
    st = Staged(w)
    out, plan = _planned(st)
    assert plan.info.num_items == 32 and plan.info.num_merges == 0
    ref = st.decode(0)       # one split per sequence too
    assert st.pool.split_tokens(32, 32, 4096) == 4096
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    st.close()


def test_planned_run_appends_the_newest_token():
    lens = [1, 17, 300, 5000, 0, 64]
    w = workloads.custom(lens, seed=33)
    st = Staged(w)
    _poison_tails(st)
    q, tables, ids, k, v = st.host[0]
    rng = np.random.default_rng(9)
    k_new = rng.standard_normal((w.batch, 8, 128)).astype(np.float16)
    v_new = rng.standard_normal((w.batch, 8, 128)).astype(np.float16)
    out, plan = _planned(st, k_new=torch.from_numpy(k_new).cuda(), v_new=torch.from_numpy(v_new).cuda())
    assert plan.info.num_merges > 0
    k2, v2 = k.copy(), v.copy()
    for s, c in enumerate(lens):
        if c:
            r = np.searchsorted(ids, tables[s, (c - 1) // 16])
            k2[r, (c - 1) % 16] = k_new[s]
            v2[r, (c - 1) % 16] = v_new[s]
    st.host[0] = (q, tables, ids, k2, v2)
    compare("planned append", out, st.reference(0))
    again, _ = _planned(st)
    assert torch.equal(again.view(torch.int16), out.view(torch.int16))
    st.close()


WAVE_HEADS_LENS = [0, 1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 100, 255, 256, 257, 1000, 1024, 1025, 2000, 3001]


@pytest.mark.parametrize("wave_heads", [0, 1])
def test_planned_wave_heads_ragged_with_poisoned_tails(wave_heads):
    """Each wave walking a whole piece for its own KV head gives the oracle's
    result, for whole sequences, cut ones (merged records) and empty ones."""
    w = workloads.custom(WAVE_HEADS_LENS, seed=34)
    st = Staged(w)
    _poison_tails(st)
    out, plan = _planned(st, wave_heads=wave_heads)
    report(f"planned wave_heads={wave_heads}", items=plan.info.num_items, merges=plan.info.num_merges,
           longest=plan.info.max_piece_tokens)
    assert plan.info.num_merges > 0 and plan.info.max_piece_tokens <= 1024  # the mode applies
    compare(f"planned wave_heads={wave_heads}", out, st.reference(0))
    st.close()


def test_planner_picks_wave_heads_for_many_short_contexts():
    rng = np.random.default_rng(35)
    lens = rng.integers(1, 300, 1100)
    lens[::97] = 0
    w = workloads.custom([int(x) for x in lens], seed=35)
    st = Staged(w)
    _poison_tails(st)
    out, plan = _planned(st)
    report("planned many short", items=plan.info.num_items, wave_heads=plan.info.decode_wave_heads)
    assert plan.info.decode_wave_heads == 1
    compare("planned many short", out, st.reference(0))
    st.close()


def test_planned_wave_heads_appends_the_newest_token():
    """Every wave stores the newest K/V row of its own KV head."""
    lens = [1, 17, 300, 1000, 0, 64, 2000]
    w = workloads.custom(lens, seed=36)
    st = Staged(w)
    _poison_tails(st)
    q, tables, ids, k, v = st.host[0]
    rng = np.random.default_rng(10)
    k_new = rng.standard_normal((w.batch, 8, 128)).astype(np.float16)
    v_new = rng.standard_normal((w.batch, 8, 128)).astype(np.float16)
    out, plan = _planned(st, k_new=torch.from_numpy(k_new).cuda(), v_new=torch.from_numpy(v_new).cuda(),
                         wave_heads=1)
    assert plan.info.num_merges > 0 and plan.info.max_piece_tokens <= 1024
    k2, v2 = k.copy(), v.copy()
    kp, vp = st.pool.k[0].cpu().numpy(), st.pool.v[0].cpu().numpy()
    for s, c in enumerate(lens):
        if c:
            blk = tables[s, (c - 1) // 16]
            r = np.searchsorted(ids, blk)
            k2[r, (c - 1) % 16] = k_new[s]
            v2[r, (c - 1) % 16] = v_new[s]
            assert np.array_equal(kp[blk, :, (c - 1) % 16, :].view(np.int16), k_new[s].view(np.int16))
            assert np.array_equal(vp[blk, :, (c - 1) % 16, :].view(np.int16), v_new[s].view(np.int16))
    st.host[0] = (q, tables, ids, k2, v2)
    compare("planned wave_heads append", out, st.reference(0))
    again, _ = _planned(st, wave_heads=1)
    assert torch.equal(again.view(torch.int16), out.view(torch.int16))
    st.close()


@pytest.mark.parametrize("hkv", [1, 2, 4, 16])
def test_other_kv_head_counts(hkv):
    """Pools of 1, 2, 4 and 16 KV heads (4 query heads each): fixed split,
    planned, and planned with per-wave KV heads where the count allows it."""
    lens = [1, 17, 300, 1000, 0, 64, 2000, 129]
    w = workloads.custom(lens, seed=37 + hkv, num_q_heads=4 * hkv, num_kv_heads=hkv)
    st = Staged(w)
    _poison_tails(st)
    ref = st.reference(0)
    report(f"hkv {hkv}", q_heads=4 * hkv)
    compare(f"hkv {hkv} fixed split", st.decode(0), ref)
    out, plan = _planned(st)
    compare(f"hkv {hkv} planned", out, ref)
    if hkv % 4 == 0:
        out, plan = _planned(st, wave_heads=1)
        assert plan.info.max_piece_tokens <= 1024
        compare(f"hkv {hkv} planned, wave heads", out, ref)
    st.close()


def _cascade(st, group, plen, k_new=None, v_new=None):
    plan = st.pool.plan(st.w.ctx_lens, prefix_group=group, prefix_len=plen)
    q, tables = st.dev[0]
    out = torch.empty_like(q)
    st.pool.run(0, plan, q, out, tables, st.w.scale, k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    return out, plan


@pytest.mark.parametrize("groups,gsize,pblocks,extra", [(2, 3, 3, [0, 5, 16, 40, 77, 1]),
                                                        (1, 20, 5, list(range(0, 200, 10))),
                                                        (3, 16, 40, [int(x) for x in np.arange(48) * 37 % 900]),
                                                        (2, 4, 6, [0] * 8)])
def test_cascade_matches_oracle(groups, gsize, pblocks, extra):
    lens = [pblocks * 16 + e for e in extra]
    assert len(lens) == groups * gsize
    w = workloads.custom(lens, seed=40 + groups, prefix_groups=(groups, gsize, pblocks))
    st = Staged(w)
    _poison_tails(st)
    group = np.repeat(np.arange(groups), gsize).astype(np.int32)
    plen = np.full(groups, pblocks * 16, np.int32)
    out, plan = _cascade(st, group, plen)
    report("cascade", groups=groups, members=gsize, items=plan.info.num_items,
           prefix_items=plan.info.num_prefix_items, merges=plan.info.num_merges)
    # contexts equal to the prefix leave no ordinary pieces: the prefix pieces
    # then run in a launch of their own, otherwise beside the ordinary ones
    assert (plan.info.num_items == 0) == all(e == 0 for e in extra)
    compare(f"cascade g{groups}x{gsize}", out, st.reference(0))
    # the same attention as the plain planned schedule
    plain, _ = _planned(st)
    compare(f"cascade vs planned g{groups}x{gsize}", out,
            plain.cpu().numpy().astype(np.float64), max_abs=2e-3, rel_l2=1e-3)
    st.close()


def test_cascade_with_ungrouped_sequences_and_append():
    lens = [64 + 3, 64 + 100, 64 + 17, 500, 0, 64 + 1]
    w = workloads.custom(lens[:3] + lens[5:] + lens[3:5], seed=44, prefix_groups=(1, 4, 4))
    st = Staged(w)
    _poison_tails(st)
    group = np.array([0, 0, 0, 0, -1, -1], np.int32)
    plen = np.array([64], np.int32)
    q, tables, ids, k, v = st.host[0]
    rng = np.random.default_rng(11)
    k_new = rng.standard_normal((w.batch, 8, 128)).astype(np.float16)
    v_new = rng.standard_normal((w.batch, 8, 128)).astype(np.float16)
    out, plan = _cascade(st, group, plen, torch.from_numpy(k_new).cuda(),
                         torch.from_numpy(v_new).cuda())
    assert plan.info.shared_newest == 0 and plan.info.num_prefix_items > 0
    k2, v2 = k.copy(), v.copy()
    for s, c in enumerate(w.ctx_lens):
        if c:
            r = np.searchsorted(ids, tables[s, (c - 1) // 16])
            k2[r, (c - 1) % 16] = k_new[s]
            v2[r, (c - 1) % 16] = v_new[s]
    st.host[0] = (q, tables, ids, k2, v2)
    compare("cascade append", out, st.reference(0))
    st.close()


def test_cascade_prefix_workload_full():
    w = workloads.config(5)
    st = Staged(w)
    group = np.repeat(np.arange(16), 16).astype(np.int32)
    plen = np.full(16, 2048, np.int32)
    out, plan = _cascade(st, group, plen)
    report("cascade config5", prefix_items=plan.info.num_prefix_items, items=plan.info.num_items,
           merges=plan.info.num_merges)
    compare("cascade config5", out, st.reference(0))
    st.close()


@pytest.mark.parametrize("case", range(24))
def test_random_planned_decodes_against_the_oracle(case):
    """Seeded random planned decodes over the planner's paths: ragged and
    short contexts, cut and whole sequences, per-wave KV heads forced on and
    off where they apply, several KV-head counts, F16 and FP8 pools, and the
    newest token appended on odd cases."""
    rng = np.random.default_rng(3000 + case)
    hkv = int(rng.choice([1, 2, 4, 8, 16]))
    top = int(rng.choice([64, 300, 2000, 6000]))
    # about 400k (token, KV head) rows at most, so the host side stays small
    batch = int(rng.integers(1, max(2, min(300, 800_000 // (top * hkv)))))
    lens = [int(x) for x in rng.integers(0, top, size=batch)]
    fp8 = case % 3 == 1
    kw = dict(dtype=pa.PA_FP8_E4M3, kv_scales=(0.1, 0.0173)) if fp8 else {}
    w = workloads.custom(lens, seed=4000 + case, num_q_heads=4 * hkv, num_kv_heads=hkv)
    st = Staged(w, **kw)
    _poison_tails(st)
    q, tables, ids, k, v = st.host[0]
    k_new = v_new = None
    if case % 2 == 1:
        k_new = rng.standard_normal((batch, hkv, 128)).astype(np.float16)
        v_new = rng.standard_normal((batch, hkv, 128)).astype(np.float16)
    for wave_heads in (0, 1):  # the second run appends the same rows again: same result
        out, plan = _planned(st, k_new=None if k_new is None else torch.from_numpy(k_new).cuda(),
                             v_new=None if v_new is None else torch.from_numpy(v_new).cuda(),
                             wave_heads=wave_heads)
        report(f"random decode {case}", hkv=hkv, fp8=fp8, batch=batch, top=top, wave_heads=wave_heads,
               items=plan.info.num_items, merges=plan.info.num_merges, longest=plan.info.max_piece_tokens)
        if k_new is not None:
            k2, v2 = k.copy(), v.copy()
            for s, c in enumerate(lens):
                if c:
                    r = np.searchsorted(ids, tables[s, (c - 1) // 16])
                    k2[r, (c - 1) % 16] = k_new[s]
                    v2[r, (c - 1) % 16] = v_new[s]
            st.host[0] = (q, tables, ids, k2, v2)
        compare(f"random decode {case} wave_heads={wave_heads}", out, st.reference(0))
        st.host[0] = (q, tables, ids, k, v)
    st.close()
