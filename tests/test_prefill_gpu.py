"""GPU parity of the chunked-prefill / mixed step (pa_prefill_plan +
pa_prefill_run) against the fp64 oracle (oracle.prefill).

Sequence s brings q_len new tokens whose K/V are already in the pool; query j
of its chunk sees positions 0 .. seq_len - q_len + j.  The pool holds every
position below seq_len (the workload's blocks); slots past seq_len in the
last block are NaN.  Tolerance as for decode: max |err| <= 2e-3, relative
L2 <= 1e-3 over each case.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import paged_kv_cache_64_amd as pa
from tests.gpu_harness import Staged, compare, report

pytestmark = pytest.mark.gpu


def _starts(q_lens):
    return np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)


class Mixed:
    """A mixed step: sequences of lengths hist + q_len staged in a pool, with
    packed query rows."""

    def __init__(self, q_lens, hist, seed, dtype=pa.PA_F16, kv_scales=(1.0, 1.0), hkv=8):
        self.q_lens = list(q_lens)
        self.lens = [h + n for h, n in zip(hist, q_lens)]
        self.w = workloads.custom(self.lens, seed=seed, num_q_heads=4 * hkv, num_kv_heads=hkv)
        self.st = Staged(self.w, dtype=dtype, kv_scales=kv_scales)
        self.starts = _starts(self.q_lens)
        self.q = self.w.q_rows(int(self.starts[-1]))
        self.qd = torch.from_numpy(self.q).cuda()
        self.scale = self.w.scale
        self.poisoned = self._poison_tails()

    def _poison_tails(self):
        w, st = self.w, self.st
        tables = st.host[0][1]
        n = 0
        for s, ctx in enumerate(self.lens):
            if ctx % 16 == 0:
                continue
            blk = int(tables[s, (ctx - 1) // 16])
            if st.fp8:
                st.pool.k[0, blk, :, ctx % 16:, :] = 0x7F
                st.pool.v[0, blk, :, ctx % 16:, :] = 0x7F
            else:
                st.pool.k[0, blk, :, ctx % 16:, :] = float("nan")
                st.pool.v[0, blk, :, ctx % 16:, :] = float("nan")
            n += 16 - ctx % 16
        torch.cuda.synchronize()
        return n

    def run(self):
        plan = self.st.pool.prefill_plan(self.starts, self.lens)
        out = torch.empty_like(self.qd)
        self.st.pool.prefill_run(0, plan, self.qd, out, self.st.dev[0][1], self.scale)
        torch.cuda.synchronize()
        return out, plan

    def _oracle(self, q, kc, vc, tables, starts, lens):
        if self.st.fp8:
            ks, vs = self.st.kv_scales
            return oracle.prefill_e4m3(q, oracle.quantize_e4m3(kc, ks), oracle.quantize_e4m3(vc, vs), tables,
                                       starts, lens, self.scale, 16, ks, vs)
        return oracle.prefill(q, kc, vc, tables, starts, lens, self.scale, 16)

    def reference(self, rows=None):
        q, tables, ids, k, v = self.st.host[0]
        kc, vc, t2 = oracle.relabelled_cache(ids, k, v, tables, self.w.ctx_lens, 16)
        if rows is None:
            return self._oracle(self.q, kc, vc, t2, self.starts, self.lens)
        # sampled rows: each as a one-token step over its own visible prefix
        owner = np.searchsorted(self.starts, rows, side="right") - 1
        q_lens = np.array(self.q_lens)
        seq_of = owner
        vis = np.array(self.lens)[seq_of] - q_lens[seq_of] + (rows - self.starts[seq_of]) + 1
        return self._oracle(self.q[rows], kc, vc, t2[seq_of], np.arange(len(rows) + 1, dtype=np.int32),
                            vis.astype(np.int32))

    def close(self):
        self.st.close()


@pytest.mark.parametrize("q_lens,hist", [
    ([1, 2, 15, 16, 17, 63, 64, 65, 100, 1, 0, 255], [100, 0, 17, 5, 0, 64, 1, 33, 4000, 4095, 9, 2000]),
    ([3, 1, 1, 130], [0, 7, 1, 1]),
])
def test_mixed_step_ragged(q_lens, hist):
    m = Mixed(q_lens, hist, seed=70 + len(q_lens))
    out, plan = m.run()
    report("mixed ragged", rows=len(m.q), decode_items=plan.info.num_items,
           prefill_items=plan.info.num_prefill_items, merges=plan.info.num_merges,
           poisoned=m.poisoned)
    compare("mixed ragged", out, m.reference())
    m.close()


@pytest.mark.parametrize("n", [2, 16, 17, 64, 65, 300])
def test_whole_prompt_prefill(n):
    m = Mixed([n], [0], seed=80 + n)
    out, _ = m.run()
    ref = m.reference()
    compare(f"whole prompt {n}", out, ref)
    # the first token sees only itself: its value row
    v0 = m.st.pool.v[0, int(m.st.host[0][1][0, 0]), :, 0, :].cpu().numpy().astype(np.float64)
    got0 = out[0].cpu().numpy().astype(np.float64)
    assert np.array_equal(got0, np.repeat(v0, 4, axis=0).astype(np.float16).astype(np.float64))
    m.close()


def test_long_chunk_split_into_merged_pieces():
    m = Mixed([300, 1, 1], [3000, 5000, 10], seed=90)
    out, plan = m.run()
    report("split pieces", prefill_items=plan.info.num_prefill_items, merges=plan.info.num_merges,
           slots=plan.info.num_slots)
    assert plan.info.num_merges > 0 and plan.info.num_prefill_items > 5
    compare("split pieces", out, m.reference())
    m.close()


def test_chunked_prompt_matches_one_chunk():
    """The same prompt as one chunk and as two consecutive chunks (the second
    with the first as history) gives rows within tolerance of each other and
    of the oracle."""
    P, cut = 200, 77
    whole = Mixed([P], [0], seed=95)
    a, _ = whole.run()
    ref = whole.reference()
    compare("one chunk", a, ref)
    # second chunk over the same pool and table: sequence length P, 123 new tokens
    m2_starts = _starts([P - cut])
    plan = whole.st.pool.prefill_plan(m2_starts, [P])
    out2 = torch.empty((P - cut, 32, 128), dtype=torch.float16, device="cuda")
    whole.st.pool.prefill_run(0, plan, whole.qd[cut:].contiguous(), out2, whole.st.dev[0][1], whole.w.scale)
    torch.cuda.synchronize()
    compare("second chunk", out2, ref[cut:])
    compare("chunked vs whole", out2, a[cut:].cpu().numpy().astype(np.float64))
    whole.close()


def test_one_token_rows_equal_the_planned_decode_bitwise():
    lens = [1, 17, 300, 4097, 64]
    m = Mixed([1] * len(lens), [x - 1 for x in lens], seed=99)
    out, _ = m.run()
    plan = m.st.pool.plan(np.array(lens, np.int32))
    out2 = torch.empty_like(m.qd)
    m.st.pool.run(0, plan, m.qd, out2, m.st.dev[0][1], m.w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    compare("decode rows", out, m.reference())
    m.close()


def test_mixed_step_under_a_2048_token_budget_sampled():
    """32 decoding sequences at 4096 tokens plus a 2016-token prompt chunk
    (second chunk of a 4032-token prompt): 2048 tokens, the default budget of
    smaller GPUs in the vLLM page, Example 5.  Rows are sampled."""
    q_lens = [2016] + [1] * 32
    hist = [2016] + [4095] * 32
    m = Mixed(q_lens, hist, seed=101)
    out, plan = m.run()
    report("budget 2048", decode_items=plan.info.num_items, prefill_items=plan.info.num_prefill_items,
           merges=plan.info.num_merges)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, 63, 64, 2015], rng.choice(2016, 24, replace=False),
                                     2016 + np.arange(32)[::4]])).astype(np.int64)
    compare("budget 2048 sampled", out[torch.from_numpy(rows).cuda()], m.reference(rows))
    m.close()


def test_prompt_chunk_alone_sampled():
    """The 2016-token chunk of the step above on its own: 63 tiles, one round
    of two work-groups per CU, dispatched longest half first and then
    shortest first.  Rows are sampled."""
    m = Mixed([2016], [2016], seed=102)
    out, plan = m.run()
    assert plan.info.num_items == 0 and plan.info.num_prefill_items == 63 and plan.info.num_merges == 0
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 1000, 1983, 1984, 2015],
                                     rng.choice(2016, 24, replace=False)])).astype(np.int64)
    compare("chunk alone sampled", out[torch.from_numpy(rows).cuda()], m.reference(rows))
    m.close()


def test_mixed_step_under_a_16384_token_budget_sampled():
    """32 decoding sequences at 4096 tokens plus the second 16,352-token chunk
    of a 32,704-token prompt: 16,384 tokens, the default budget of the largest
    GPUs in the vLLM page, Example 5.  Tiles are cut into merged pieces and
    the launch runs three work-groups per CU.  Rows are sampled."""
    q_lens = [16352] + [1] * 32
    hist = [16352] + [4095] * 32
    m = Mixed(q_lens, hist, seed=104)
    out, plan = m.run()
    report("budget 16384", decode_items=plan.info.num_items, prefill_items=plan.info.num_prefill_items,
           merges=plan.info.num_merges)
    assert plan.info.num_prefill_items * 8 > 512 and plan.info.num_merges > 32
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 8191, 16351], rng.choice(16352, 24, replace=False),
                                     16352 + np.arange(32)[::4]])).astype(np.int64)
    compare("budget 16384 sampled", out[torch.from_numpy(rows).cuda()], m.reference(rows))
    m.close()


def test_long_history_chunk_merges_with_eight_heads_per_work_group_sampled():
    """A 1,024-token chunk after 26,000 tokens of history: its 32 tiles of
    1,627-1,689 key blocks exceed a piece (1,536 blocks) and are cut in two,
    so 1,024 query tokens are merged, with the merge launch's eight-head
    work-groups (512-2,047 merges).  Rows are sampled."""
    m = Mixed([1024], [26000], seed=105)
    out, plan = m.run()
    report("1024 after 26000", prefill_items=plan.info.num_prefill_items, merges=plan.info.num_merges)
    assert plan.info.num_prefill_items == 64 and plan.info.num_merges == 1024
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 511, 1023], rng.choice(1024, 10, replace=False)])).astype(np.int64)
    compare("1024 after 26000 sampled", out[torch.from_numpy(rows).cuda()], m.reference(rows))
    m.close()


@pytest.mark.parametrize("q_lens,hist", [([2100], [0]), ([2100, 1, 1, 1], [0, 4000, 100, 2047])])
def test_more_tiles_than_one_round_sampled(q_lens, hist):
    """66 prompt tiles (528 work-groups, more than one round of two per CU):
    the launch takes the three-per-CU kernels, alone and with decode rows.
    Rows are sampled."""
    m = Mixed(q_lens, hist, seed=103 + len(q_lens))
    out, plan = m.run()
    assert plan.info.num_prefill_items * 8 > 512
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 2067, 2068, 2099], rng.choice(2100, 24, replace=False),
                                     np.arange(2100, len(m.q))])).astype(np.int64)
    compare("66 tiles sampled", out[torch.from_numpy(rows).cuda()], m.reference(rows))
    m.close()


@pytest.mark.parametrize("scale", [0.75, 1.0, 3.0])
def test_prompt_rows_with_softmax_scales_past_one(scale):
    """Softmax scales past 1 (peaked weights, scores of tens in log2 units):
    the scores stay in fp32 up to the exponential, so the error stays at the
    F16 rounding of the output."""
    m = Mixed([40, 100, 1, 33], [10, 300, 50, 2000], seed=140)
    m.scale = scale
    out, plan = m.run()
    assert plan.info.num_prefill_items > 0
    compare(f"prompt rows at scale {scale}", out, m.reference())
    m.close()


@pytest.mark.parametrize("q_len,hist", [(1024, 3008), (512, 3520), (100, 4000), (32, 4000), (300, 0)])
def test_prompt_only_launches_of_one_work_group_per_cu(q_len, hist):
    """A prompt-only launch of at most one work-group per CU: each tile's keys
    are split between two wave groups of one work-group and merged in LDS;
    tiles cut into pieces (as far as that work-group count allows) write
    records that the merge kernel combines."""
    m = Mixed([q_len], [hist], seed=160 + q_len)
    out, plan = m.run()
    assert plan.info.num_items == 0 and plan.info.num_prefill_items * 8 <= 256
    report(f"prompt only {q_len} after {hist}", items=plan.info.num_prefill_items, merges=plan.info.num_merges)
    compare(f"prompt only {q_len} after {hist}", out, m.reference())
    m.close()


@pytest.mark.parametrize("hkv", [1, 2, 16])
def test_mixed_step_with_other_kv_head_counts(hkv):
    m = Mixed([40, 1, 100, 1, 33], [10, 300, 50, 2000, 0], seed=150 + hkv, hkv=hkv)
    out, plan = m.run()
    assert plan.info.num_prefill_items > 0 and plan.info.num_items > 0
    compare(f"mixed step, {hkv} kv heads", out, m.reference())
    m.close()


FP8 = pa.PA_FP8_E4M3
# non-power-of-two scales: fl32(1/scale) is inexact and the codes span most
# of the format's range
FP8_SCALES = (0.1, 0.0173)


@pytest.mark.parametrize("q_lens,hist", [
    ([1, 2, 15, 16, 17, 63, 64, 65, 100, 1, 0, 255], [100, 0, 17, 5, 0, 64, 1, 33, 4000, 4095, 9, 2000]),
    ([40, 1, 1], [10, 30, 300]),
])
def test_fp8_mixed_step_ragged(q_lens, hist):
    """FP8 pools: decode rows and prefill tiles in one launch; slots past each
    sequence's length hold NaN codes."""
    m = Mixed(q_lens, hist, seed=110 + len(q_lens), dtype=FP8, kv_scales=FP8_SCALES)
    out, plan = m.run()
    report("fp8 mixed ragged", rows=len(m.q), decode_items=plan.info.num_items,
           prefill_items=plan.info.num_prefill_items, merges=plan.info.num_merges, poisoned=m.poisoned)
    compare("fp8 mixed ragged", out, m.reference())
    m.close()


def test_fp8_prompt_rows_with_a_score_scale_past_one():
    """K's scale folded into the score scale takes it past 1 (10 * log2(e) * 0.1)."""
    m = Mixed([40, 100, 1], [10, 300, 50], seed=141, dtype=FP8, kv_scales=FP8_SCALES)
    m.scale = 10.0
    out, _ = m.run()
    compare("fp8 prompt rows at scale 10", out, m.reference())
    m.close()


@pytest.mark.parametrize("q_len,hist", [(1024, 3008), (512, 3520), (32, 4000)])
def test_fp8_prompt_only_launches_of_one_work_group_per_cu(q_len, hist):
    """FP8 pools: each tile's keys split between two wave groups of one
    work-group per CU, merged in LDS; cut tiles write value-domain records."""
    m = Mixed([q_len], [hist], seed=170 + q_len, dtype=FP8, kv_scales=FP8_SCALES)
    out, plan = m.run()
    assert plan.info.num_items == 0 and plan.info.num_prefill_items * 8 <= 256
    compare(f"fp8 prompt only {q_len} after {hist}", out, m.reference())
    m.close()


def test_fp8_prompt_chunk_alone_sampled():
    """The 2016-token chunk at position 2016 on an FP8 pool: 63 tiles, one
    round of prompt-only work-groups (more than one per CU).  Rows are
    sampled."""
    m = Mixed([2016], [2016], seed=133, dtype=FP8, kv_scales=FP8_SCALES)
    out, plan = m.run()
    assert plan.info.num_items == 0 and plan.info.num_prefill_items == 63 and plan.info.num_merges == 0
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 1000, 1983, 1984, 2015],
                                     rng.choice(2016, 24, replace=False)])).astype(np.int64)
    compare("fp8 chunk alone sampled", out[torch.from_numpy(rows).cuda()], m.reference(rows))
    m.close()


@pytest.mark.parametrize("n", [1, 17, 300])
def test_fp8_whole_prompt_prefill(n):
    m = Mixed([n], [0], seed=120 + n, dtype=FP8, kv_scales=FP8_SCALES)
    out, _ = m.run()
    compare(f"fp8 whole prompt {n}", out, m.reference())
    # the first token sees only itself: its value codes times V's scale,
    # rounded once to fp32 and once to F16
    codes = m.st.pool.v[0, int(m.st.host[0][1][0, 0]), :, 0, :].cpu().numpy()
    lut = np.array([oracle.e4m3_to_f64(c) for c in range(256)], np.float32)
    want = (lut[codes] * np.float32(FP8_SCALES[1])).astype(np.float16)
    assert np.array_equal(out[0].cpu().numpy(), np.repeat(want, 4, axis=0))
    m.close()


def test_fp8_long_chunk_split_into_merged_pieces():
    """Cut tiles write value-domain records (V's scale applied) that the
    merge combines with each other."""
    m = Mixed([300, 1, 1], [3000, 5000, 10], seed=130, dtype=FP8, kv_scales=FP8_SCALES)
    out, plan = m.run()
    report("fp8 split pieces", prefill_items=plan.info.num_prefill_items, merges=plan.info.num_merges)
    assert plan.info.num_merges > 0 and plan.info.num_prefill_items > 5
    compare("fp8 split pieces", out, m.reference())
    m.close()


def test_fp8_one_token_rows_equal_the_planned_decode_bitwise():
    lens = [1, 17, 300, 4097, 64]
    m = Mixed([1] * len(lens), [x - 1 for x in lens], seed=131, dtype=FP8, kv_scales=FP8_SCALES)
    out, _ = m.run()
    plan = m.st.pool.plan(np.array(lens, np.int32))
    out2 = torch.empty_like(m.qd)
    m.st.pool.run(0, plan, m.qd, out2, m.st.dev[0][1], m.w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    compare("fp8 decode rows", out, m.reference())
    m.close()


def test_fp8_value_scale_is_linear_in_prefill_rows():
    """Doubling V's scale (codes unchanged) doubles every prefill row exactly,
    for whole tiles and for cut (merged) tiles."""
    m = Mixed([50, 200], [0, 4000], seed=132, dtype=FP8, kv_scales=FP8_SCALES)
    a, plan = m.run()
    assert plan.info.num_merges > 0
    m.st.pool.set_scales(0, FP8_SCALES[0], 2 * FP8_SCALES[1])
    b, _ = m.run()
    a2, b = 2 * a.float(), b.float()
    normal = a.float().abs() > 2.0 ** -14       # values at 2^-14 may be rounded subnormals
    assert torch.equal(b[normal], a2[normal])
    assert float((b - a2).abs().max()) <= 2.0 ** -24
    m.close()


@pytest.mark.parametrize("case", range(24))
def test_random_steps_against_the_oracle(case):
    """Seeded random steps over the planner's paths: prompt-only launches
    (split kernels, cut tiles), mixed launches with decode rows, and several
    KV-head counts and pool types, each checked against the oracle in full."""
    rng = np.random.default_rng(1000 + case)
    hkv = int(rng.choice([1, 2, 4, 8]))
    batch = int(rng.integers(1, 6))
    q_lens = [int(x) for x in rng.choice([1, 1, 2, 17, 40, 100, 257], size=batch)]
    if case % 2 == 0:                       # prompt-only steps on even cases
        q_lens = [max(q, 2) for q in q_lens]
    hist = [int(x) for x in rng.integers(0, 1500, size=batch)]
    fp8 = case % 3 == 2
    kw = dict(dtype=FP8, kv_scales=FP8_SCALES) if fp8 else {}
    m = Mixed(q_lens, hist, seed=2000 + case, hkv=hkv, **kw)
    out, plan = m.run()
    report(f"random step {case}", hkv=hkv, fp8=fp8, q_lens=q_lens, hist=hist,
           decode_items=plan.info.num_items, prefill_items=plan.info.num_prefill_items,
           merges=plan.info.num_merges)
    compare(f"random step {case}", out, m.reference())
    m.close()
