"""Pins for the oracle's chunked-prefill / mixed step (oracle.prefill), each
against something other than itself: the pinned decode oracle (one-token
chunks; every query row as a decode with a shorter context), torch's
scaled_dot_product_attention in fp64 with an explicit causal mask, the
invariance of causal attention under chunking, a closed form, and brute
force on a tiny case."""
import math

import numpy as np
import pytest
import torch

import oracle


def _cache(rng, lens, hkv, d, bs, pool_factor=2):
    """Random F16 slot caches and tables for sequences of the given lengths;
    blocks are distinct and randomly placed."""
    held = [-(-int(n) // bs) for n in lens]
    width = max(1, max(held) if held else 1)
    nb = pool_factor * max(1, sum(held))
    ids = rng.permutation(nb)
    tables = np.zeros((len(lens), width), np.int32)
    at = 0
    for s, h in enumerate(held):
        tables[s, :h] = ids[at:at + h]
        at += h
    k = rng.standard_normal((nb * bs, hkv, d)).astype(np.float16)
    v = rng.standard_normal((nb * bs, hkv, d)).astype(np.float16)
    return k, v, tables


def _starts(q_lens):
    return np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)


def test_one_token_chunks_equal_the_decode_oracle():
    rng = np.random.default_rng(1)
    lens = [1, 5, 16, 17, 40]
    k, v, t = _cache(rng, lens, 2, 16, 4)
    q = rng.standard_normal((len(lens), 8, 16)).astype(np.float16)
    a = oracle.prefill(q, k, v, t, _starts([1] * len(lens)), lens, 0.25, 4)
    b = oracle.decode(q, k, v, t, lens, 0.25, 4)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-14)


def test_each_query_row_is_a_decode_with_a_shorter_context():
    """Query j of a q_len chunk of a seq_len sequence attends exactly like a
    decode of context seq_len - q_len + j + 1 over the same table."""
    rng = np.random.default_rng(2)
    q_lens = [1, 2, 5, 16, 17, 0, 9]
    hist = [0, 7, 3, 0, 30, 12, 64]
    lens = [h + n for h, n in zip(hist, q_lens)]
    k, v, t = _cache(rng, lens, 2, 16, 4)
    total = sum(q_lens)
    q = rng.standard_normal((total, 8, 16)).astype(np.float16)
    got = oracle.prefill(q, k, v, t, _starts(q_lens), lens, 0.3, 4)
    rows_t, ctx = [], []
    for s, (n, L) in enumerate(zip(q_lens, lens)):
        for j in range(n):
            rows_t.append(t[s])
            ctx.append(L - n + j + 1)
    want = oracle.decode(q, k, v, np.array(rows_t, np.int32), np.array(ctx, np.int32), 0.3, 4)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (16, 2)])
def test_matches_torch_sdpa_with_a_causal_mask(hq, hkv):
    rng = np.random.default_rng(3 + hq)
    d, bs = 32, 8
    q_lens = [3, 1, 24, 0, 11]
    hist = [5, 40, 0, 9, 16]
    lens = [h + n for h, n in zip(hist, q_lens)]
    k, v, t = _cache(rng, lens, hkv, d, bs)
    q = rng.standard_normal((sum(q_lens), hq, d)).astype(np.float16)
    scale = 1.0 / math.sqrt(d)
    got = oracle.prefill(q, k, v, t, _starts(q_lens), lens, scale, bs)
    starts = _starts(q_lens)
    for s, (n, L) in enumerate(zip(q_lens, lens)):
        if n == 0:
            continue
        slots = [int(t[s, p // bs]) * bs + p % bs for p in range(L)]
        ks = torch.from_numpy(k[slots].astype(np.float64)).permute(1, 0, 2)   # [hkv, L, d]
        vs = torch.from_numpy(v[slots].astype(np.float64)).permute(1, 0, 2)
        ks = ks.repeat_interleave(hq // hkv, dim=0).contiguous()
        vs = vs.repeat_interleave(hq // hkv, dim=0).contiguous()
        qs = torch.from_numpy(q[starts[s]:starts[s + 1]].astype(np.float64)).permute(1, 0, 2)
        j = torch.arange(n)[:, None]
        tt = torch.arange(L)[None, :]
        mask = tt <= (L - n + j)                                               # bottom-right causal
        ref = torch.nn.functional.scaled_dot_product_attention(qs.contiguous(), ks, vs,
                                                               attn_mask=mask, scale=scale)
        np.testing.assert_allclose(got[starts[s]:starts[s + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)


def test_chunking_does_not_change_the_rows():
    """A prompt processed in one chunk or in several (each chunk's sequence
    length being the tokens stored so far) gives the same rows, bit for bit."""
    rng = np.random.default_rng(4)
    P = 37
    k, v, t = _cache(rng, [P], 2, 16, 4)
    q = rng.standard_normal((P, 8, 16)).astype(np.float16)
    whole = oracle.prefill(q, k, v, t, [0, P], [P], 0.2, 4)
    cuts = [0, 5, 6, 20, 37]
    parts = [oracle.prefill(q[a:b], k, v, t, [0, b - a], [b], 0.2, 4) for a, b in zip(cuts, cuts[1:])]
    assert np.array_equal(np.concatenate(parts), whole)


def test_first_token_of_a_prompt_returns_its_value():
    rng = np.random.default_rng(5)
    k, v, t = _cache(rng, [9], 2, 16, 4)
    q = rng.standard_normal((9, 8, 16)).astype(np.float16)
    out = oracle.prefill(q, k, v, t, [0, 9], [9], 0.5, 4)
    slot0 = int(t[0, 0]) * 4
    for h in range(8):
        assert np.array_equal(out[0, h], v[slot0, h // 4].astype(np.float64))


def test_brute_force_tiny():
    rng = np.random.default_rng(6)
    q_lens, lens, bs, hq, hkv, d = [2, 3], [3, 5], 2, 2, 1, 3
    k, v, t = _cache(rng, lens, hkv, d, bs)
    q = rng.standard_normal((5, hq, d)).astype(np.float16)
    got = oracle.prefill(q, k, v, t, _starts(q_lens), lens, 0.7, bs)
    row = 0
    for s, (n, L) in enumerate(zip(q_lens, lens)):
        for j in range(n):
            vis = L - n + j + 1
            for h in range(hq):
                zs = []
                for p in range(vis):
                    sl = int(t[s][p // bs]) * bs + p % bs
                    zs.append(0.7 * sum(float(q[row, h, i]) * float(k[sl, 0, i]) for i in range(d)))
                m = max(zs)
                w = [math.exp(z - m) for z in zs]
                for i in range(d):
                    acc = 0.0
                    for p in range(vis):
                        sl = int(t[s][p // bs]) * bs + p % bs
                        acc += w[p] * float(v[sl, 0, i])
                    assert abs(got[row, h, i] - acc / sum(w)) < 1e-12
            row += 1


def test_rejects_inconsistent_offsets():
    rng = np.random.default_rng(7)
    k, v, t = _cache(rng, [8, 8], 1, 4, 4)
    q = rng.standard_normal((4, 1, 4)).astype(np.float16)
    with pytest.raises(ValueError):        # a chunk longer than its sequence
        oracle.prefill(q, k, v, t, [0, 1, 4], [8, 2], 1.0, 4)
    with pytest.raises(ValueError):        # a sequence past its table
        oracle.prefill(q, k, v, t, [0, 2, 4], [8, 9], 1.0, 4)
    with pytest.raises(ValueError):        # decreasing offsets
        oracle.prefill(q, k, v, t, [0, 5, 4], [8, 8], 1.0, 4)
