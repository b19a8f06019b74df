"""CPU tests of the host schedule built by pa_decode_plan (integer work: exact)."""
import numpy as np
import pytest

import paged_kv_cache_64_amd as pa
import workloads

FAKE = 1 << 20


@pytest.fixture
def pool():
    handle = pa.pa_pool_create(pa.PoolDesc(1, 64, 16, 8, 128, pa.PA_F16), FAKE, FAKE)
    yield handle
    pa.pa_pool_destroy(handle)


def _decode_plan(info, plan):
    assert plan[0] == 0x50414E31
    assert plan[1] == info.batch and plan[2] == info.num_q_heads
    assert plan[3] == info.num_items and plan[4] == info.num_merges and plan[5] == info.num_slots
    items = plan[8:8 + 8 * info.num_items].reshape(-1, 8)
    merges = plan[8 + 8 * info.num_items:8 + 8 * info.num_items + 4 * info.num_merges].reshape(-1, 4)
    return items, merges


def _check_cover(lens, info, plan):
    items, merges = _decode_plan(info, plan)
    pieces = {}
    for s, t0, t1, ctx, slot, row, hsel, _ in items:
        assert ctx == lens[s] and 0 <= t0 <= t1 <= ctx and row == s and hsel == 0
        assert t0 % 16 == 0 and (t1 % 16 == 0 or t1 == ctx)
        pieces.setdefault(s, []).append((t0, t1, slot))
    assert sorted(pieces) == list(range(len(lens)))
    for s, ps in pieces.items():
        ps.sort()
        assert ps[0][0] == 0 and ps[-1][1] == lens[s]
        for (a0, a1, _), (b0, b1, _) in zip(ps, ps[1:]):
            assert a1 == b0
        if len(ps) == 1:
            assert ps[0][2] == -1           # written directly, no merge
    # longest first
    lengths = items[:, 2] - items[:, 1]
    assert np.all(np.diff(lengths) <= 0)
    # merges: exactly the cut sequences, with contiguous slots
    cut = {s for s, ps in pieces.items() if len(ps) > 1}
    assert {int(m[0]) for m in merges} == cut
    for s, first, n, _ in merges:
        assert sorted(p[2] for p in pieces[s]) == list(range(first, first + n))
    assert info.num_slots == sum(len(pieces[s]) for s in cut)
    assert info.max_piece_tokens == int(lengths.max()) if len(lengths) else True
    assert info.max_piece_tokens <= 4096
    return items, merges


def test_uniform_batch_is_one_piece_per_sequence(pool):
    lens = [4096] * 32
    info, plan = pa.pa_decode_plan(pool, lens, 32)
    items, merges = _check_cover(lens, info, plan)
    assert info.num_items == 32 and info.num_merges == 0 and info.workspace_bytes == 0


def test_ragged_batch_is_cut_into_near_equal_pieces(pool):
    lens = list(workloads.config(4).ctx_lens)
    info, plan = pa.pa_decode_plan(pool, lens, 32)
    items, merges = _check_cover(lens, info, plan)
    # pieces of a cut sequence differ by at most one block
    per = {}
    for s, t0, t1, *_ in items:
        per.setdefault(s, []).append(t1 - t0)
    for s, ls in per.items():
        if len(ls) > 1:
            full = [x for x in ls if x % 16 == 0]
            assert max(full) - min(full) <= 16 if full else True
    assert info.workspace_bytes >= info.num_slots * 32 * 130 * 4


def test_small_batches_get_pieces_of_at_least_16_blocks(pool):
    lens = [256]
    info, plan = pa.pa_decode_plan(pool, lens, 32)
    _check_cover(lens, info, plan)
    assert info.num_items == 1 and info.num_merges == 0      # one piece, no merge
    lens = [2048]
    info, plan = pa.pa_decode_plan(pool, lens, 32)
    items, _ = _check_cover(lens, info, plan)
    assert info.num_items == 8 and info.num_merges == 1      # 8 pieces of 16 blocks
    assert np.all(items[:, 2] - items[:, 1] == 256)
    lens = [1, 0, 17, 4097, 0]
    info, plan = pa.pa_decode_plan(pool, lens, 32)
    items, _ = _check_cover(lens, info, plan)
    assert info.max_piece_tokens == 256


def test_prefix_workload_plan(pool):
    lens = list(workloads.config(5).ctx_lens)
    info, plan = pa.pa_decode_plan(pool, lens, 32)
    _check_cover(lens, info, plan)


def test_plan_validation(pool):
    lib = pa.load_library()
    info = pa.PlanInfo()
    lens = np.array([5, -1], np.int32)
    assert lib.pa_decode_plan(pool, lens.ctypes.data, 2, 32, None, 0, info) == pa.PA_ERR_INVALID_ARG
    lens = np.array([5, 7], np.int32)
    assert lib.pa_decode_plan(pool, lens.ctypes.data, 2, 16, None, 0, info) == pa.PA_ERR_UNSUPPORTED
    assert lib.pa_decode_plan(pool, None, 2, 32, None, 0, info) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_decode_plan(pool, lens.ctypes.data, 2, 32, None, 0, info) == pa.PA_OK
    small = np.zeros(2, np.int32)
    assert lib.pa_decode_plan(pool, lens.ctypes.data, 2, 32, small.ctypes.data, 8, info) == pa.PA_ERR_WORKSPACE
    info0, plan0 = pa.pa_decode_plan(pool, [], 32)
    assert info0.num_items == 0
    # run with an empty plan is a no-op; a bad layer is rejected before any launch
    assert lib.pa_decode_run(pool, 0, info0, FAKE, info0.plan_bytes, FAKE, None, None, FAKE, FAKE, 1,
                             0.1, None, 0, None) == pa.PA_OK
    info1, _ = pa.pa_decode_plan(pool, [100], 32)
    pb = info1.plan_bytes
    assert lib.pa_decode_run(pool, 3, info1, FAKE, pb, FAKE, None, None, FAKE, FAKE, 7, 0.1, FAKE,
                             1 << 20, None) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_decode_run(pool, 0, info1, FAKE, pb, FAKE, None, None, FAKE, FAKE, 6, 0.1, FAKE,
                             1 << 20, None) == pa.PA_ERR_INVALID_ARG      # table too narrow
    assert lib.pa_decode_run(pool, 0, info1, FAKE, pb, FAKE, FAKE, None, FAKE, FAKE, 7, 0.1, FAKE,
                             1 << 20, None) == pa.PA_ERR_INVALID_ARG      # k_new without v_new
    assert lib.pa_decode_run(pool, 0, info1, FAKE, pb, FAKE, None, None, FAKE, FAKE, (1 << 26) + 1,
                             0.1, FAKE, 1 << 20, None) == pa.PA_ERR_UNSUPPORTED  # table wider than 2^26
    if info1.workspace_bytes:
        assert lib.pa_decode_run(pool, 0, info1, FAKE, pb, FAKE, None, None, FAKE, FAKE, 7, 0.1, FAKE,
                                 info1.workspace_bytes - 1, None) == pa.PA_ERR_WORKSPACE


def test_run_checks_the_plan_against_its_info_and_buffer(pool):
    """The kernels index the plan's sections by the counts in the info, so a run
    whose info does not describe the plan, or whose device buffer is smaller than
    the plan, is refused before anything is enqueued."""
    lib = pa.load_library()
    lens = list(workloads.config(4).ctx_lens)
    info, _ = pa.pa_decode_plan(pool, lens, 32)
    assert info.num_merges > 0
    ws = info.workspace_bytes
    run = lambda inf, nbytes: lib.pa_decode_run(pool, 0, inf, FAKE, nbytes, FAKE, None, None, FAKE,
                                                FAKE, 512, 0.1, FAKE, ws, None)
    assert run(info, info.plan_bytes - 4) == pa.PA_ERR_WORKSPACE     # buffer one word short
    # an info kept from a larger step: more items than its plan_bytes hold
    big = pa.PlanInfo.from_buffer_copy(info)
    big.num_items += 1
    assert run(big, 1 << 30) == pa.PA_ERR_INVALID_ARG
    big = pa.PlanInfo.from_buffer_copy(info)
    big.num_merges += 3
    assert run(big, 1 << 30) == pa.PA_ERR_INVALID_ARG
    big = pa.PlanInfo.from_buffer_copy(info)
    big.plan_bytes += 4
    assert run(big, 1 << 30) == pa.PA_ERR_INVALID_ARG
    # the same checks guard the prefill entry point
    pinfo, _ = pa.pa_prefill_plan(pool, np.array([0, 40, 41], np.int32), np.array([100, 60], np.int32), 32)
    prun = lambda inf, nbytes: lib.pa_prefill_run(pool, 0, inf, FAKE, nbytes, FAKE, FAKE, FAKE, 16, 0.1,
                                                  FAKE, 1 << 30, None)
    assert prun(pinfo, pinfo.plan_bytes - 1) == pa.PA_ERR_WORKSPACE
    bad = pa.PlanInfo.from_buffer_copy(pinfo)
    bad.num_prefill_items += 1
    assert prun(bad, 1 << 30) == pa.PA_ERR_INVALID_ARG


def _decode_cascade(info, plan):
    off = 8 + 8 * info.num_items + 4 * info.num_merges
    pitems = plan[off:off + 8 * info.num_prefix_items].reshape(-1, 8)
    off += 8 * info.num_prefix_items
    mlist = plan[off:off + 2 * info.num_members].reshape(-1, 2)
    return pitems, mlist


def test_cascade_plan_covers_prefix_and_suffix_once(pool):
    w = workloads.config(5)
    lens = w.ctx_lens
    group = np.repeat(np.arange(16), 16).astype(np.int32)
    plen = np.full(16, 2048, np.int32)
    info, plan = pa.pa_cascade_plan(pool, lens, group, plen, 32)
    items, merges = _decode_plan(info, plan)
    pitems, mlist = _decode_cascade(info, plan)
    assert info.num_merges == 256                    # every member merges prefix + suffix
    assert info.shared_newest == int((lens == 2048).sum())
    # suffix pieces cover [2048, ctx) of every sequence exactly
    cover = {}
    for s, t0, t1, ctx, slot, *_ in items:
        assert ctx == lens[s] and 2048 <= t0 < t1 <= ctx and slot >= 0
        cover.setdefault(s, []).append((t0, t1, slot))
    for s in range(256):
        ps = sorted(cover.get(s, []))
        if lens[s] == 2048:
            assert not ps
            continue
        assert ps[0][0] == 2048 and ps[-1][1] == lens[s]
        assert all(a[1] == b[0] for a, b in zip(ps, ps[1:]))
    # prefix pieces: per group, pieces tile [0, 2048) in whole blocks, 16 members each
    by_group = {}
    for first_seq, t0, t1, nm, moff, *_ in pitems:
        assert nm == 16 and t0 % 16 == 0 and t1 % 16 == 0 and t1 - t0 <= 32 * 16
        mem = mlist[moff:moff + nm]
        assert set(mem[:, 0]) == set(range(16 * group[first_seq], 16 * group[first_seq] + 16))
        by_group.setdefault(group[first_seq], []).append((t0, t1, mem))
    assert len(by_group) == 16
    for g, ps in by_group.items():
        ps.sort(key=lambda x: x[0])
        assert ps[0][0] == 0 and ps[-1][1] == 2048
    # each sequence's records: a contiguous run holding its prefix and suffix pieces exactly once
    recs = {}
    for s, slot in mlist:
        recs.setdefault(s, []).append(slot)
    for s, t0, t1, ctx, slot, *_ in items:
        recs.setdefault(s, []).append(slot)
    for s, first, n, _ in merges:
        assert sorted(recs[s]) == list(range(first, first + n))


def test_cascade_plan_validation_and_subgroups(pool):
    lens = np.array([100, 40, 64, 300] + [64] * 20, np.int32)
    group = np.array([0, 0, -1, 0] + [1] * 20, np.int32)
    plen = np.array([32, 64], np.int32)
    info, plan = pa.pa_cascade_plan(pool, lens, group, plen, 32)
    pitems, mlist = _decode_cascade(info, plan)
    assert sorted(pitems[:, 3].tolist()) == [3, 4, 16]            # group 1 split 16 + 4
    lib = pa.load_library()
    i2 = pa.PlanInfo()
    bad = np.array([30, 64], np.int32)                            # not whole blocks
    assert lib.pa_cascade_plan(pool, lens.ctypes.data, len(lens), group.ctypes.data,
                               bad.ctypes.data, 2, 32, None, 0, i2) == pa.PA_ERR_INVALID_ARG
    too_long = np.array([128, 64], np.int32)                      # longer than member 1's context
    assert lib.pa_cascade_plan(pool, lens.ctypes.data, len(lens), group.ctypes.data,
                               too_long.ctypes.data, 2, 32, None, 0, i2) == pa.PA_ERR_INVALID_ARG
    g_bad = group.copy()
    g_bad[0] = 5
    assert lib.pa_cascade_plan(pool, lens.ctypes.data, len(lens), g_bad.ctypes.data,
                               plen.ctypes.data, 2, 32, None, 0, i2) == pa.PA_ERR_INVALID_ARG


def test_cascade_run_rejects_appending_into_a_shared_block(pool):
    lens = np.array([64, 80], np.int32)                 # sequence 0's newest token is in the prefix
    info, _ = pa.pa_cascade_plan(pool, lens, np.array([0, 0], np.int32), np.array([64], np.int32), 32)
    assert info.shared_newest == 1
    lib = pa.load_library()
    assert lib.pa_decode_run(pool, 0, info, FAKE, info.plan_bytes, FAKE, FAKE, FAKE, FAKE, FAKE, 5, 0.1,
                             FAKE, 1 << 30, None) == pa.PA_ERR_INVALID_ARG


# ---- chunked-prefill / mixed-step schedule (pa_prefill_plan) ----------------
def _mixed_plan(info, plan):
    items, merges = _decode_plan(info, plan)
    off = 8 + 8 * info.num_items + 4 * info.num_merges
    pf = plan[off:off + 12 * info.num_prefill_items].reshape(-1, 12)
    assert plan.size * 4 >= info.plan_bytes and off + 12 * info.num_prefill_items == info.plan_bytes // 4
    return items, merges, pf


def _check_mixed(q_lens, lens, info, plan):
    """Every query row is produced exactly once: a direct decode item, a direct
    prefill piece, or the merge of a complete set of records."""
    starts = np.concatenate([[0], np.cumsum(q_lens)]).astype(int)
    items, merges, pf = _mixed_plan(info, plan)
    assert info.num_q_rows == starts[-1] and info.num_prefix_items == 0
    produced = {}
    records = {}
    for s, t0, t1, ctx, slot, row, *_ in items:
        assert q_lens[s] == 1 and ctx == lens[s] and row == starts[s]
        if slot < 0:
            assert t0 == 0 and t1 == ctx
            produced[row] = produced.get(row, 0) + 1
        else:
            records[slot] = records.get(slot, 0) + 1
    tiles = {}
    for s, row0, n_q, pos0, t0, t1, base, np_, p, *rest in pf:
        assert q_lens[s] >= 2 and 1 <= n_q <= 64 and rest == [0, 0, 0]
        assert starts[s] <= row0 and row0 + n_q <= starts[s + 1]
        assert pos0 == lens[s] - q_lens[s] + (row0 - starts[s])
        assert t0 % 16 == 0 and 0 <= t0 < t1 <= pos0 + n_q and 0 <= p < np_
        tiles.setdefault((s, row0), []).append((t0, t1, base, np_, p, n_q, pos0))
    for (s, row0), ps in tiles.items():
        ps.sort()
        n_q, pos0 = ps[0][5], ps[0][6]
        assert ps[0][0] == 0 and ps[-1][1] == pos0 + n_q               # pieces cover the keys
        for a, b in zip(ps, ps[1:]):
            assert a[1] == b[0]
        assert sorted(x[4] for x in ps) == list(range(len(ps))) and all(x[3] == len(ps) for x in ps)
        if len(ps) == 1:
            assert ps[0][2] == -1
            for k in range(n_q):
                produced[row0 + k] = produced.get(row0 + k, 0) + 1
        else:
            base = ps[0][2]
            assert all(x[2] == base for x in ps) and base >= 0
            for k in range(n_q):
                for p in range(len(ps)):
                    slot = base + k * len(ps) + p
                    records[slot] = records.get(slot, 0) + 1
    for s, first, n, row in merges:
        assert all(records.get(first + i) == 1 for i in range(n))
        produced[row] = produced.get(row, 0) + 1
    assert sorted(records) == list(range(info.num_slots))
    assert all(v == 1 for v in records.values())
    assert produced == {r: 1 for r in range(starts[-1])}
    # each kind is dispatched longest first, except a prefill-only launch of
    # one round of two work-groups per CU (256 CUs, 8 KV heads): its longest
    # 32 tiles come first and the rest follow shortest first
    if len(items):
        assert np.all(np.diff(items[:, 2] - items[:, 1]) <= 0)
    span = pf[:, 5] - pf[:, 4]
    if len(items) == 0 and 256 < 8 * len(pf) <= 512:
        assert np.all(np.diff(span[:32]) <= 0) and np.all(np.diff(span[32:]) >= 0)
        assert span[32:].max() <= span[:32].min()
    elif len(pf):
        assert np.all(np.diff(span) <= 0)
    return items, merges, pf


@pytest.mark.parametrize("q_lens,hist", [
    ([1] * 8, [100, 4095, 0, 16, 17, 2000, 300, 5]),
    ([2, 1, 17, 64, 65, 1, 255, 0], [0, 33, 500, 0, 4000, 0, 17, 9]),
    ([2016] + [1] * 32, [2016] + [4095] * 32),
    ([255, 1], [2040, 300]),
    ([4096], [0]),
    ([2016], [2016]),
    ([1056], [0]),
])
def test_mixed_plan_produces_every_row_once(pool, q_lens, hist):
    lens = [h + n for h, n in zip(hist, q_lens)]
    starts = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    info, plan = pa.pa_prefill_plan(pool, starts, lens, 32)
    _check_mixed(q_lens, lens, info, plan)
    assert info.max_context_len == max(lens)


def test_mixed_plan_long_chunk_is_cut_and_merged(pool):
    # tiles of 1,877-2,004 key blocks: longer than a piece may be (1,536 blocks)
    q_lens, lens = [2048], [32048]
    info, plan = pa.pa_prefill_plan(pool, [0, 2048], lens, 32)
    items, merges, pf = _check_mixed(q_lens, lens, info, plan)
    assert info.num_items == 0 and info.num_prefill_items == 2 * 64
    assert info.num_merges == 2048 and info.workspace_bytes > 0
    assert (pf[:, 5] - pf[:, 4]).max() <= 1536 * 16


def test_mixed_plan_keeps_tiles_whole_when_they_fit_a_piece(pool):
    # 2048 queries after 6144 tokens of history: tiles of 386-512 blocks fill
    # 64 x 8 work-groups, so none is cut and nothing is merged
    q_lens, lens = [2048], [8192]
    info, plan = pa.pa_prefill_plan(pool, [0, 2048], lens, 32)
    items, merges, pf = _check_mixed(q_lens, lens, info, plan)
    assert info.num_prefill_items == 64 and info.num_merges == 0 and info.num_slots == 0


def test_mixed_plan_rejects_bad_offsets(pool):
    lib = pa.load_library()
    info = pa.PlanInfo()
    import ctypes
    def call(qs, lens):
        qs = np.ascontiguousarray(qs, np.int32)
        lens = np.ascontiguousarray(lens, np.int32)
        return lib.pa_prefill_plan(pool, qs.ctypes.data, lens.ctypes.data, len(lens), 32, None, 0,
                                   ctypes.byref(info))
    assert call([0, 1, 3], [5, 9]) == 0
    assert call([1, 2, 3], [5, 9]) == pa.PA_ERR_INVALID_ARG        # first offset not 0
    assert call([0, 3, 2], [5, 9]) == pa.PA_ERR_INVALID_ARG        # decreasing
    assert call([0, 6, 7], [5, 9]) == pa.PA_ERR_INVALID_ARG        # chunk longer than its sequence
    assert lib.pa_prefill_plan(pool, None, None, 0, 32, None, 0, ctypes.byref(info)) == pa.PA_ERR_INVALID_ARG
    assert lib.pa_prefill_plan(pool, np.zeros(3, np.int32).ctypes.data, np.ones(2, np.int32).ctypes.data,
                               2, 16, None, 0, ctypes.byref(info)) == pa.PA_ERR_UNSUPPORTED


def test_decode_plans_carry_their_rows(pool):
    lens = [5000, 17, 300]
    info, plan = pa.pa_decode_plan(pool, lens, 32)
    items, merges = _decode_plan(info, plan)
    assert np.array_equal(items[:, 5], items[:, 0])
    assert np.array_equal(merges[:, 3], merges[:, 0]) and info.num_q_rows == 3
    assert info.num_prefill_items == 0


def test_longest_context_plans_and_longer_ones_are_unsupported(pool):
    """Contexts of up to 2^30 tokens are cut into 4096-token pieces that cover
    them exactly, for decode and mixed plans; longer ones (up to the int32
    limit) are rejected as unsupported."""
    for too_long in ((1 << 30) + 1, (1 << 31) - 1):
        with pytest.raises(pa.PaError) as e:
            pa.pa_decode_plan(pool, [too_long, 5], 32)
        assert e.value.status == pa.PA_ERR_UNSUPPORTED
        with pytest.raises(pa.PaError) as e:
            pa.pa_prefill_plan(pool, np.array([0, 1, 2], np.int32), np.array([too_long, 5], np.int32), 32)
        assert e.value.status == pa.PA_ERR_UNSUPPORTED
    big = (1 << 30) - 3
    lens = [big, 5]
    info, plan = pa.pa_decode_plan(pool, lens, 32)
    items, merges = _check_cover(lens, info, plan)
    assert info.num_merges == 1 and info.max_context_len == big
    assert info.num_items == -(-big // 4096) + 1
    starts = np.array([0, 1, 2], np.int32)
    info2, plan2 = pa.pa_prefill_plan(pool, starts, np.array(lens, np.int32), 32)
    assert info2.num_items == info.num_items and info2.num_merges == 1 and info2.max_context_len == big


def test_piece_size_balances_the_compute_units(pool):
    """Without shared prefixes the piece size comes from a model of the
    dispatch (each compute unit pulls K/V at a bounded rate, so the most loaded
    unit sets the launch time): uniform batches whose one-piece plans would
    leave some units with twice the work of others are cut so that every unit
    gets the same, and batches that fill the chip evenly are not cut."""
    cases = {  # lengths: (pieces, merged sequences, longest piece in tokens)
        (4096,) * 32: (32, 0, 4096),     # 256 work-groups of 256 blocks: even
        (4096,) * 24: (96, 24, 1024),    # 768 work-groups of 64 blocks: 3 per unit
        (4096,) * 48: (96, 48, 2048),    # 768 work-groups of 128 blocks
        (1024,) * 24: (24, 0, 1024),     # 192 work-groups, no merge
        (4096,) * 8: (32, 8, 1024),
    }
    for lens, (n_items, n_merges, longest) in cases.items():
        info, plan = pa.pa_decode_plan(pool, list(lens), 32)
        _check_cover(list(lens), info, plan)
        assert (info.num_items, info.num_merges, info.max_piece_tokens) == (n_items, n_merges, longest), lens


def test_mixed_launch_walks_decode_pieces_with_two_waves_when_the_tiles_dominate(pool):
    """pa_plan_info.mixed_decode_waves: a mixed step whose prompt tiles take longer
    than its decode pieces (32 decodes at 4096 tokens beside a 2016-token chunk)
    walks the decode pieces with 2 of 4 waves so both kinds progress side by
    side; a step dominated by its decode rows keeps 4, and so does every plan
    without both kinds."""
    cfg6_q = [2016] + [1] * 32
    cfg6_lens = [4032] + [4096] * 32
    starts = np.concatenate([[0], np.cumsum(cfg6_q)]).astype(np.int32)
    info, plan = pa.pa_prefill_plan(pool, starts, cfg6_lens, 32)
    _check_mixed(cfg6_q, cfg6_lens, info, plan)
    assert info.num_items > 0 and info.num_prefill_items > 0 and info.mixed_decode_waves == 2
    small_q = [17] + [1] * 32
    small_lens = [117] + [4096] * 32
    starts = np.concatenate([[0], np.cumsum(small_q)]).astype(np.int32)
    info, plan = pa.pa_prefill_plan(pool, starts, small_lens, 32)
    _check_mixed(small_q, small_lens, info, plan)
    assert info.num_items > 0 and info.num_prefill_items > 0 and info.mixed_decode_waves == 4
    assert pa.pa_decode_plan(pool, [4096] * 32, 32)[0].mixed_decode_waves == 4
    assert pa.pa_prefill_plan(pool, np.array([0, 1, 2], np.int32), [50, 60], 32)[0].mixed_decode_waves == 4


def test_wave_heads_for_many_short_pieces(pool):
    """Per-wave KV heads only where every piece fits one wave's table register
    (1024 tokens) and the dispatch model rates the launch of four times fewer,
    four times longer work-groups faster (each case below as measured)."""
    def wh(lens, handle=pool):
        info, _ = pa.pa_decode_plan(handle, lens, 32 if handle is pool else 8)
        return info.decode_wave_heads, info.max_piece_tokens
    assert wh([128] * 1024) == (1, 128)
    assert wh([1024] * 128) == (1, 1024)      # 128 items x 2 work-groups
    assert wh([1024] * 64) == (0, 1024)       # 128 work-groups: the four-wave split
    assert wh([1024] * 160)[0] == 0           # 320 work-groups: 64 units would take two
    assert wh([512] * 150)[0] == 0
    assert wh([64] * 2048)[0] == 1 and wh([32] * 4096)[0] == 1
    assert wh([4096] * 40) == (0, 1024)       # cut in four: 320 work-groups again
    assert wh([4096] * 32)[0] == 0            # pieces past one table register
    assert wh([4096] * 8)[0] == 0
    assert wh([0] * 600) == (1, 0)
    two = pa.pa_pool_create(pa.PoolDesc(1, 64, 16, 2, 128, pa.PA_F16), FAKE, FAKE)
    try:
        assert wh([128] * 4096, two)[0] == 0  # two KV heads: not a multiple of the four waves
    finally:
        pa.pa_pool_destroy(two)
    info, _ = pa.pa_prefill_plan(pool, [0, 1, 2], [100, 100], 32)
    assert info.decode_wave_heads == 0
