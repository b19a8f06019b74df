"""GPU parity at the limits of the shapes, against the fp64 oracle:
  - a 131,072-token context (8,192 blocks in one table row; 32 pieces in the
    fixed split, cut and merged in the planned one);
  - a batch of 8,192 sequences of 0 .. 48 tokens;
  - pools whose tile offsets pass 2^32 bytes (F16 and FP8), so that every
    address computed from a block id needs 64-bit arithmetic: the writes of
    pa_write_kv, the decode, the planned decode and a mixed prefill step.
Tolerance as for the other parity tests: max |err| <= 2e-3, rel L2 <= 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import paged_kv_cache_64_amd as pa
from tests.gpu_harness import Staged, compare, report
from tests.test_parity_gpu import _poison_tails

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_overrides(monkeypatch):
    monkeypatch.delenv("PA_SPLIT_TOKENS", raising=False)


def _planned(st, layer=0):
    plan = st.pool.plan(st.w.ctx_lens)
    q, tables = st.dev[layer]
    out = torch.empty_like(q)
    st.pool.run(layer, plan, q, out, tables, st.w.scale)
    torch.cuda.synchronize()
    return out, plan


def test_long_context_fixed_and_planned():
    lens = [131072, 1, 5000, 17]
    w = workloads.custom(lens, seed=160)
    st = Staged(w)
    npois = _poison_tails(st)
    ref = st.reference(0)
    fixed = st.decode(0)
    report("long context", poisoned=npois, split=st.pool.split_tokens(w.batch, 32, w.max_context_len))
    compare("long context fixed", fixed, ref)
    planned, plan = _planned(st)
    report("long context planned", items=plan.info.num_items, merges=plan.info.num_merges,
           longest=plan.info.max_piece_tokens)
    assert plan.info.num_merges > 0
    compare("long context planned", planned, ref)
    st.close()


def test_large_batch_of_short_contexts():
    rng = np.random.default_rng(161)
    lens = rng.integers(0, 49, size=8192).astype(np.int32)
    lens[:4] = [0, 1, 16, 48]
    w = workloads.custom(lens, seed=161)
    st = Staged(w)
    _poison_tails(st)
    ref = st.reference(0)
    compare("batch 8192 fixed", st.decode(0), ref)
    planned, plan = _planned(st)
    report("batch 8192 planned", items=plan.info.num_items, merges=plan.info.num_merges)
    compare("batch 8192 planned", planned, ref)
    st.close()


@pytest.mark.parametrize("fp8", [False, True])
def test_pool_offsets_beyond_4_gib(fp8):
    """About 304,000 blocks per layer: K tiles of high block ids start past
    2^32 bytes (F16: block 131,072 and up; FP8: 262,144 and up)."""
    lens = [3000, 700, 16, 1, 2500]
    w = workloads.custom(lens, seed=162 + fp8, pool_factor=1300)
    tile_bytes = 16 * 128 * (1 if fp8 else 2)
    scales = (0.1, 0.0173)
    st = Staged(w, dtype=pa.PA_FP8_E4M3 if fp8 else pa.PA_F16, kv_scales=scales)
    tables = st.host[0][1]
    held = -(-w.ctx_lens.astype(np.int64) // 16)
    used = np.concatenate([tables[s, :held[s]] for s in range(w.batch)]).astype(np.int64)
    far = int(((used * w.num_kv_heads + w.num_kv_heads - 1) * tile_bytes >= 2 ** 32).sum())
    report("pool offsets", pool_blocks=w.pool_blocks, max_block=int(used.max()), blocks_past_4GiB=far)
    assert far > 20
    _poison_tails_any(st)
    ref = st.reference(0)
    compare(f"offsets>4GiB fixed fp8={fp8}", st.decode(0), ref)
    planned, _ = _planned(st)
    compare(f"offsets>4GiB planned fp8={fp8}", planned, ref)
    # a mixed step on the same pool: the last 200 tokens of sequence 0 and of
    # sequence 4 as prompt chunks, the others as decode rows
    q_lens = [200, 1, 1, 1, 200]
    starts = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    qrows = w.q_rows(int(starts[-1]))
    plan = st.pool.prefill_plan(starts, lens)
    out = torch.empty((int(starts[-1]), 32, 128), dtype=torch.float16, device="cuda")
    st.pool.prefill_run(0, plan, torch.from_numpy(qrows).cuda(), out, st.dev[0][1], w.scale)
    torch.cuda.synchronize()
    q, tbl, ids, k, v = st.host[0]
    kc, vc, t2 = oracle.relabelled_cache(ids, k, v, tbl, w.ctx_lens, 16)
    if fp8:
        mref = oracle.prefill_e4m3(qrows, oracle.quantize_e4m3(kc, scales[0]), oracle.quantize_e4m3(vc, scales[1]),
                                   t2, starts, lens, w.scale, 16, *scales)
    else:
        mref = oracle.prefill(qrows, kc, vc, t2, starts, lens, w.scale, 16)
    compare(f"offsets>4GiB mixed fp8={fp8}", out, mref)
    st.close()


def _poison_tails_any(st, layer=0):
    """NaN past each context in its last block (F16 NaN or the FP8 NaN code)."""
    w = st.w
    tables = st.host[layer][1]
    for s, ctx in enumerate(w.ctx_lens):
        ctx = int(ctx)
        if ctx == 0 or ctx % 16 == 0:
            continue
        blk = int(tables[s, (ctx - 1) // 16])
        if st.fp8:
            st.pool.k[layer, blk, :, ctx % 16:, :] = 0x7F
            st.pool.v[layer, blk, :, ctx % 16:, :] = 0x7F
        else:
            st.pool.k[layer, blk, :, ctx % 16:, :] = float("nan")
            st.pool.v[layer, blk, :, ctx % 16:, :] = float("nan")
    torch.cuda.synchronize()
