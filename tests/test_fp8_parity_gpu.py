"""GPU parity of FP8 (E4M3) pools: libpa through the C ABI against the fp64
oracle's E4M3 path.

The oracle quantises the host F16 values itself (oracle.quantize_e4m3) and
decodes the codes in fp64; the library encodes in pa_write_kv / the
appending decode.  Stored codes are compared bit-exactly; outputs to the F16
tolerance (max |err| <= 2e-3, relative L2 <= 1e-3), since both sides attend
over the same dequantised values and the kernel's arithmetic is the F16
path's (F16 keys, fp32 accumulation).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
import paged_kv_cache_64_amd as pa
from tests.gpu_harness import Staged, compare, report

pytestmark = pytest.mark.gpu

FP8 = pa.PA_FP8_E4M3
NAN_CODE = 0x7F
RAGGED = [1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 100, 255, 256, 257, 1000, 4097]
# non-power-of-two scales, so that fl32(1/scale) is inexact and the values span
# most of the format's range (N(0,1) values, keys up to x8)
SCALES = (0.1, 0.0173)


@pytest.fixture(autouse=True)
def _no_split_override(monkeypatch):
    monkeypatch.delenv("PA_SPLIT_TOKENS", raising=False)


def _poison_tails(st, layer=0):
    """Sets the codes of each sequence's last-block slots past its context to NaN."""
    w = st.w
    tables = st.host[layer][1]
    n = 0
    for s, ctx in enumerate(w.ctx_lens):
        ctx = int(ctx)
        if ctx == 0 or ctx % w.block_size == 0:
            continue
        blk = int(tables[s, (ctx - 1) // w.block_size])
        off = ctx % w.block_size
        st.pool.k[layer, blk, :, off:, :] = NAN_CODE
        st.pool.v[layer, blk, :, off:, :] = NAN_CODE
        n += w.block_size - off
    torch.cuda.synchronize()
    return n


def _planned(st, layer=0, k_new=None, v_new=None, wave_heads=None):
    plan = st.pool.plan(st.w.ctx_lens)
    if wave_heads is not None:  # override the planner's choice of per-wave KV heads
        plan.info.decode_wave_heads = wave_heads
    q, tables = st.dev[layer]
    out = torch.empty_like(q)
    st.pool.run(layer, plan, q, out, tables, st.w.scale, k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    return out, plan


def test_fp8_write_kv_stores_the_oracle_codes():
    """Codes per layer with that layer's scales; skipped slots untouched;
    out-of-range values saturate; infinities clamp; NaN stays NaN."""
    report("fp8 write_kv codes")
    pool = pa.Pool(2, 8, dtype=FP8, fill=0.0)
    scales = {0: (1.0 / 64, 3.0), 1: SCALES}
    for layer, (ks, vs) in scales.items():
        pool.set_scales(layer, ks, vs)
    rng = np.random.default_rng(3)
    n = 48
    slots = rng.choice(8 * 16, size=n, replace=False).astype(np.int32)
    slots[5] = -1
    slots[9] = 8 * 16
    want_k = np.zeros(tuple(pool.k.shape), np.uint8)
    want_v = np.zeros(tuple(pool.v.shape), np.uint8)
    for layer, (ks, vs) in scales.items():
        k = (rng.standard_normal((n, 8, 128)) * 8).astype(np.float16)
        v = (rng.standard_normal((n, 8, 128)) * 400).astype(np.float16)  # many saturate
        k[0, 0, :4] = [np.inf, -np.inf, 60000.0, -0.0]
        k[1, 1, 0] = np.nan
        pool.write(layer, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                   torch.from_numpy(slots).cuda())
        qk = oracle.quantize_e4m3(k, ks)
        qv = oracle.quantize_e4m3(v, vs)
        for i, sl in enumerate(slots):
            if 0 <= sl < 8 * 16:
                want_k[layer, sl // 16, :, sl % 16, :] = qk[i]
                want_v[layer, sl // 16, :, sl % 16, :] = qv[i]
    torch.cuda.synchronize()
    kp, vp = pool.k.cpu().numpy(), pool.v.cpu().numpy()
    # the NaN inputs: any NaN code (the sign of a NaN is not pinned)
    for layer in scales:
        nan_at = (layer, slots[1] // 16, 1, slots[1] % 16, 0)
        assert kp[nan_at] & 0x7F == 0x7F
        kp[nan_at] = want_k[nan_at]
    assert np.array_equal(kp, want_k)
    assert np.array_equal(vp, want_v)
    assert (vp == 0x7E).any() and (vp == 0xFE).any()   # saturation was exercised
    pool.close()


def test_fp8_ragged_batch_fixed_phases_and_planned():
    w = workloads.custom(RAGGED, seed=61)
    st = Staged(w, dtype=FP8, kv_scales=SCALES)
    npois = _poison_tails(st)
    ref = st.reference(0)
    report("fp8 ragged", poisoned_slots=npois)
    out = st.decode(0)
    compare("fp8 ragged", out, ref)
    compare("fp8 ragged phases", st.decode(0, phases=True), ref)
    planned, plan = _planned(st)
    report("fp8 planned", items=plan.info.num_items, merges=plan.info.num_merges)
    compare("fp8 ragged planned", planned, ref)
    assert plan.info.max_piece_tokens <= 1024
    compare("fp8 ragged planned, wave heads", _planned(st, wave_heads=1)[0], ref)
    st.close()


@pytest.mark.parametrize("split", [64, 256, 4096])
def test_fp8_split_lengths(monkeypatch, split):
    monkeypatch.setenv("PA_SPLIT_TOKENS", str(split))
    w = workloads.custom([3, 64, 129, 700, 2048, 5000], seed=62 + split)
    st = Staged(w, dtype=FP8, kv_scales=SCALES)
    _poison_tails(st)
    compare(f"fp8 split={split}", st.decode(0), st.reference(0))
    st.close()


def test_fp8_empty_and_single_token_contexts():
    w = workloads.custom([0, 1, 0, 2], seed=63)
    st = Staged(w, dtype=FP8, kv_scales=SCALES)
    out = st.decode(0).cpu().numpy()
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    compare("fp8 ctx 0/1/2", out.astype(np.float64), st.reference(0))
    st.close()


def test_fp8_value_scale_is_linear():
    """Doubling v_scale (codes unchanged) doubles the output exactly; the
    output is the code-domain attention times v_scale."""
    w = workloads.custom([5, 40, 300], seed=64)
    st = Staged(w, dtype=FP8, kv_scales=SCALES)
    a = st.decode(0)
    st.pool.set_scales(0, SCALES[0], 2 * SCALES[1])
    b = st.decode(0).float()
    a2 = 2 * a.float()
    normal = a.float().abs() > 2.0 ** -14       # values at 2^-14 may be rounded subnormals
    assert torch.equal(b[normal], a2[normal])
    assert float((b - a2).abs().max()) <= 2.0 ** -24
    st.close()


def test_fp8_extreme_scales_saturate_and_underflow():
    """A value scale that saturates most V codes and a key scale that flushes
    small keys to subnormal or zero codes: the oracle sees the same codes."""
    w = workloads.custom([17, 250, 1100], seed=65, key_boost_prob=0.05)
    st = Staged(w, dtype=FP8, kv_scales=(4.0, 1.0 / 512))
    _poison_tails(st)
    vp = st.pool.v[0].cpu().numpy()[st.host[0][2]]        # referenced blocks
    assert ((vp & 0x7F) == 0x7E).mean() > 0.3
    compare("fp8 extreme scales", st.decode(0), st.reference(0))
    st.close()


@pytest.mark.parametrize("k", [1, 2, 4, 9])
def test_fp8_config_full_parity(k):
    w = workloads.config(k)
    st = Staged(w, dtype=FP8, kv_scales=SCALES)
    compare(f"fp8 config{k}", st.decode(0), st.reference(0))
    planned, _ = _planned(st)
    compare(f"fp8 config{k} planned", planned, st.reference(0))
    st.close()


@pytest.mark.parametrize("planned", [False, True, "wave_heads"])
def test_fp8_append_encodes_the_newest_token_and_attends_to_it(planned):
    lens = [1, 16, 17, 100, 257, 1000, 0, 4097]
    w = workloads.custom(lens, seed=66)
    st = Staged(w, dtype=FP8, kv_scales=SCALES)
    _poison_tails(st)
    q, tables, ids, k, v = st.host[0]
    rng = np.random.default_rng(8)
    k_new = (rng.standard_normal((w.batch, 8, 128)) * 3).astype(np.float16)
    v_new = rng.standard_normal((w.batch, 8, 128)).astype(np.float16)
    kd, vd = torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda()
    qd, td = st.dev[0]
    wh = 1 if planned == "wave_heads" else None
    if planned:
        out, plan = _planned(st, k_new=kd, v_new=vd, wave_heads=wh)
        assert plan.info.max_piece_tokens <= 1024
    else:
        out = torch.empty_like(qd)
        st.pool.decode(0, qd, out, td, st.lens, w.max_context_len, w.scale, k_new=kd, v_new=vd)
        torch.cuda.synchronize()
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
    compare(f"fp8 append planned={planned}", out, st.reference(0))
    kp, vp = st.pool.k[0].cpu().numpy(), st.pool.v[0].cpu().numpy()
    qk, qv = oracle.quantize_e4m3(k_new, SCALES[0]), oracle.quantize_e4m3(v_new, SCALES[1])
    for s, blk, off in newest:
        assert np.array_equal(kp[blk, :, off, :], qk[s])
        assert np.array_equal(vp[blk, :, off, :], qv[s])
    # a read-only decode of the same schedule afterwards gives the same bits
    again = _planned(st, wave_heads=wh)[0] if planned else st.decode(0)
    assert torch.equal(again.view(torch.int16), out.view(torch.int16))
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
                                                        (3, 16, 40, [int(x) for x in np.arange(48) * 37 % 900])])
def test_fp8_cascade_matches_oracle(groups, gsize, pblocks, extra):
    """Shared-prefix pieces over FP8 tiles: value-domain records merged with
    the members' own suffix pieces; NaN codes past every context."""
    lens = [pblocks * 16 + e for e in extra]
    w = workloads.custom(lens, seed=140 + groups, prefix_groups=(groups, gsize, pblocks))
    st = Staged(w, dtype=FP8, kv_scales=SCALES)
    _poison_tails(st)
    group = np.repeat(np.arange(groups), gsize).astype(np.int32)
    plen = np.full(groups, pblocks * 16, np.int32)
    out, plan = _cascade(st, group, plen)
    report("fp8 cascade", groups=groups, members=gsize, prefix_items=plan.info.num_prefix_items,
           merges=plan.info.num_merges)
    assert plan.info.num_prefix_items > 0
    compare(f"fp8 cascade g{groups}x{gsize}", out, st.reference(0))
    plain, _ = _planned(st)
    compare(f"fp8 cascade vs planned g{groups}x{gsize}", out, plain.cpu().numpy().astype(np.float64))
    st.close()


def test_fp8_cascade_with_ungrouped_sequences_and_append():
    lens = [64 + 3, 64 + 100, 64 + 17, 64 + 1, 500, 0]
    w = workloads.custom(lens, seed=150, prefix_groups=(1, 4, 4))
    st = Staged(w, dtype=FP8, kv_scales=SCALES)
    _poison_tails(st)
    group = np.array([0, 0, 0, 0, -1, -1], np.int32)
    plen = np.array([64], np.int32)
    q, tables, ids, k, v = st.host[0]
    rng = np.random.default_rng(12)
    k_new = rng.standard_normal((w.batch, 8, 128)).astype(np.float16)
    v_new = rng.standard_normal((w.batch, 8, 128)).astype(np.float16)
    out, plan = _cascade(st, group, plen, torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda())
    assert plan.info.shared_newest == 0 and plan.info.num_prefix_items > 0
    k2, v2 = k.copy(), v.copy()
    for s, c in enumerate(w.ctx_lens):
        if c:
            r = np.searchsorted(ids, tables[s, (c - 1) // 16])
            k2[r, (c - 1) % 16] = k_new[s]
            v2[r, (c - 1) % 16] = v_new[s]
    st.host[0] = (q, tables, ids, k2, v2)
    compare("fp8 cascade append", out, st.reference(0))
    st.close()


def test_fp8_cascade_value_scale_is_linear():
    w = workloads.custom([80 + e for e in (0, 7, 30, 100)], seed=151, prefix_groups=(1, 4, 5))
    st = Staged(w, dtype=FP8, kv_scales=SCALES)
    group, plen = np.zeros(4, np.int32), np.array([80], np.int32)
    a, _ = _cascade(st, group, plen)
    st.pool.set_scales(0, SCALES[0], 2 * SCALES[1])
    b, _ = _cascade(st, group, plen)
    a2, b = 2 * a.float(), b.float()
    normal = a.float().abs() > 2.0 ** -14       # values at 2^-14 may be rounded subnormals
    assert torch.equal(b[normal], a2[normal])
    assert float((b - a2).abs().max()) <= 2.0 ** -24
    st.close()


def test_fp8_cascade_prefix_workload_full():
    w = workloads.config(5)
    st = Staged(w, dtype=FP8, kv_scales=SCALES)
    group = np.repeat(np.arange(16), 16).astype(np.int32)
    plen = np.full(16, 2048, np.int32)
    out, plan = _cascade(st, group, plen)
    report("fp8 cascade config5", prefix_items=plan.info.num_prefix_items, items=plan.info.num_items,
           merges=plan.info.num_merges)
    compare("fp8 cascade config5", out, st.reference(0))
    st.close()
