"""Seeded synthetic inputs for one batched decode step of paged attention.

This module feeds both the HIP library and the oracle.  It holds none of the
method's arithmetic: it only draws random numbers and arranges them as the
pages describe the inputs -- per-sequence context lengths, per-sequence block
tables that name physical blocks scattered through a shared pool ("vLLM
Architecture and Installation", Example 3), and the F16 contents of those
blocks, laid out per block as [block_size, kv_heads, head_dim].

Streams.  Every array comes from its own counter-addressed numpy stream,
``SeedSequence(entropy=seed, spawn_key=(purpose, layer, chunk))``, so a value
never depends on the number of threads or on which other arrays were drawn.
Values are N(0, 1) drawn in float32 and rounded to F16 (round to nearest
even).

The five workloads (all with 32 query heads, 8 KV heads, head_dim 128,
block_size 16, scale 1/sqrt(128)):
  1  one layer, batch 1, context 256; the table is the first 16 ids of a
     random permutation of a 64-block pool
  2  one layer, batch 8, every context 4096; pool of 2x the needed blocks
  3  32 layers, batch 32, every context 4096; a fresh random table per layer
  4  one layer, 64 sequences, context uniform in [1, 8192]; 1 % of the
     (slot, kv head) key vectors are scaled by 8 in float32 before rounding
  5  one layer, 256 sequences in 16 groups of 16; each group shares 128
     physical prefix blocks (2048 tokens, reference count 16) and each
     sequence adds a private suffix of uniform [0, 6144] tokens
Two mixed steps (chunked prefill under a token budget, "vLLM Architecture
and Installation", Example 5; "Batching and Scheduling", Example 5): each
sequence brings q_lens[s] new tokens, already stored, and ctx_lens[s] counts
every token in the cache.
  6  32 layers; 32 decoding sequences at 4096 tokens plus the second
     2016-token chunk of a 4032-token prompt: 2048 tokens, the default budget
     of GPUs under 70 GiB
  7  8 layers; 32 decoding sequences at 4096 tokens plus the second
     16,352-token chunk of a 32,704-token prompt: 16,384 tokens, the default
     budget of GPUs with 160 GiB or more (MI355X has 288 GB)
One launch-bound step (the case a captured whole-step graph is for):
  8  32 layers, batch 1, context 256; per layer the table is the first 16
     ids of a random permutation of a 64-block pool (workload 1 on every layer)
Many short contexts (the case per-wave KV heads are for):
  9  one layer, batch 1024, every context 128; pool of 2x the needed blocks
"""
from __future__ import annotations

import math
import os
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# stream purposes
_META, _TABLE, _Q, _K, _V, _BOOST, _QROWS = range(7)
# blocks drawn per stream chunk (fixed, so results do not depend on threads)
_CHUNK_BLOCKS = 256


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(entropy=seed, spawn_key=tuple(key)))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


_scratch = threading.local()


def _normal_f16(rng: np.random.Generator, shape, boost=None, out=None) -> np.ndarray:
    """N(0, 1) drawn in float32 (optionally some rows scaled), rounded to F16."""
    n = int(np.prod(shape))
    buf = getattr(_scratch, "buf", None)
    if buf is None or buf.size < n:
        buf = _scratch.buf = np.empty(n, dtype=np.float32)
    view = buf[:n].reshape(shape)
    rng.standard_normal(out=view, dtype=np.float32)
    if boost is not None:
        mask, factor = boost
        view[mask] *= np.float32(factor)
    if out is None:
        return view.astype(np.float16)
    np.copyto(out, view, casting="same_kind")
    return out


@dataclass
class Workload:
    name: str
    seed: int
    layers: int
    ctx_lens: np.ndarray                 # int32 [batch]
    num_q_heads: int = 32
    num_kv_heads: int = 8
    head_dim: int = 128
    block_size: int = 16
    pool_blocks: int = 0                 # physical blocks per layer pool
    max_blocks: int = 0                  # table width
    prefix_groups: tuple | None = None   # (groups, group_size, prefix_blocks)
    key_boost_prob: float = 0.0
    key_boost: float = 8.0
    fresh_tables_per_layer: bool = True
    q_lens: np.ndarray | None = None     # int32 [batch]: new tokens per sequence (None: one each)
    description: str = ""
    _table_cache: dict = field(default_factory=dict, repr=False)

    # -- shapes -------------------------------------------------------------
    @property
    def batch(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def max_context_len(self) -> int:
        return int(self.ctx_lens.max()) if self.batch else 0

    def blocks_held(self) -> np.ndarray:
        """Blocks each sequence holds: whole blocks covering its context."""
        return -(-self.ctx_lens.astype(np.int64) // self.block_size)

    # -- metadata -----------------------------------------------------------
    def tables(self, layer: int = 0) -> np.ndarray:
        """int32 [batch, max_blocks]; entries past a sequence's blocks are 0."""
        key = layer if self.fresh_tables_per_layer else 0
        if key in self._table_cache:
            return self._table_cache[key]
        rng = _rng(self.seed, _TABLE, key)
        held = self.blocks_held()
        perm = rng.permutation(self.pool_blocks).astype(np.int32)
        tables = np.zeros((self.batch, self.max_blocks), dtype=np.int32)
        nxt = 0
        shared = 0
        if self.prefix_groups is not None:
            groups, gsize, pblocks = self.prefix_groups
            shared = pblocks
            for grp in range(groups):
                ids = perm[nxt:nxt + pblocks]
                nxt += pblocks
                tables[grp * gsize:(grp + 1) * gsize, :pblocks] = ids
        for s in range(self.batch):
            own = int(held[s]) - shared
            tables[s, shared:shared + own] = perm[nxt:nxt + own]
            nxt += own
        assert nxt <= self.pool_blocks
        if len(self._table_cache) > 4:
            self._table_cache.clear()
        self._table_cache[key] = tables
        return tables

    def referenced_blocks(self, layer: int = 0) -> np.ndarray:
        """Sorted unique physical block ids that some table names."""
        t = self.tables(layer)
        held = self.blocks_held()
        ids = [t[s, :held[s]] for s in range(self.batch)]
        if not ids:
            return np.zeros(0, dtype=np.int32)
        return np.unique(np.concatenate(ids)).astype(np.int32)

    # -- values -------------------------------------------------------------
    def q(self, layer: int = 0) -> np.ndarray:
        """F16 [batch, num_q_heads, head_dim]."""
        return _normal_f16(_rng(self.seed, _Q, layer),
                           (self.batch, self.num_q_heads, self.head_dim))

    @property
    def query_start(self) -> np.ndarray:
        """int32 [batch + 1]: first packed query row of each sequence."""
        q = self.q_lens if self.q_lens is not None else np.ones(self.batch, np.int32)
        return np.concatenate([[0], np.cumsum(q)]).astype(np.int32)

    def q_rows(self, n_rows: int, layer: int = 0) -> np.ndarray:
        """F16 [n_rows, num_q_heads, head_dim]: the packed query rows of a step
        in which sequences bring several new tokens (chunked prefill)."""
        return _normal_f16(_rng(self.seed, _QROWS, layer), (n_rows, self.num_q_heads, self.head_dim))

    def kv_blocks(self, layer: int = 0, ids: np.ndarray | None = None):
        """Contents of the referenced physical blocks of one layer.

        Returns (ids int32 [n], K F16 [n, B, Hkv, d], V F16 [n, B, Hkv, d]).
        Block i's values come from the chunk streams of its rank among the
        sorted referenced ids, so any subset `ids` is drawn consistently.
        """
        all_ids = self.referenced_blocks(layer)
        if ids is None:
            ids = all_ids
        ids = np.asarray(ids, dtype=np.int32)
        rank = np.searchsorted(all_ids, ids)
        assert np.all(all_ids[rank] == ids), "block not referenced by any table"
        shape = (self.block_size, self.num_kv_heads, self.head_dim)
        n = ids.shape[0]
        k = np.empty((n,) + shape, dtype=np.float16)
        v = np.empty((n,) + shape, dtype=np.float16)
        chunks = np.unique(rank // _CHUNK_BLOCKS)
        full = n == all_ids.shape[0]

        def fill(c):
            lo = c * _CHUNK_BLOCKS
            cnt = min(_CHUNK_BLOCKS, all_ids.shape[0] - lo)
            boost = None
            if self.key_boost_prob > 0.0:
                mask = _rng(self.seed, _BOOST, layer, c).random(
                    (cnt, self.block_size, self.num_kv_heads)) < self.key_boost_prob
                boost = (mask, self.key_boost)
            if full:
                _normal_f16(_rng(self.seed, _K, layer, c), (cnt,) + shape, boost, k[lo:lo + cnt])
                _normal_f16(_rng(self.seed, _V, layer, c), (cnt,) + shape, None, v[lo:lo + cnt])
                return
            kc = _normal_f16(_rng(self.seed, _K, layer, c), (cnt,) + shape, boost)
            vc = _normal_f16(_rng(self.seed, _V, layer, c), (cnt,) + shape)
            sel = np.nonzero((rank >= lo) & (rank < lo + cnt))[0]
            k[sel] = kc[rank[sel] - lo]
            v[sel] = vc[rank[sel] - lo]

        if len(chunks) > 1:
            with ThreadPoolExecutor(_threads()) as ex:
                list(ex.map(fill, chunks))
        else:
            for c in chunks:
                fill(c)
        return ids, k, v

    # -- accounting (what the step must read; used for reporting) -----------
    def kv_unique_bytes(self, elem_bytes: int = 2) -> int:
        """K+V bytes of the distinct (block, offset) slots the step reads, over all
        layers: shared prefix blocks count once."""
        per_token = self.num_kv_heads * self.head_dim * 2 * elem_bytes
        total = 0
        held = self.blocks_held()
        for layer in range(self.layers if self.fresh_tables_per_layer else 1):
            t = self.tables(layer)
            used = {}
            for s in range(self.batch):
                ctx = int(self.ctx_lens[s])
                for j in range(int(held[s])):
                    n = min(self.block_size, ctx - j * self.block_size)
                    b = int(t[s, j])
                    used[b] = max(used.get(b, 0), n)
            total += sum(used.values()) * per_token
        if not self.fresh_tables_per_layer:
            total *= self.layers
        return total

    def kv_bytes(self, layers: int | None = None, elem_bytes: int = 2) -> int:
        """K+V bytes every sequence reads once per layer (logical); elem_bytes 2
        for F16 storage, 1 for FP8."""
        per_token = self.num_kv_heads * self.head_dim * 2 * elem_bytes
        return int(self.ctx_lens.astype(np.int64).sum()) * per_token * (layers or self.layers)


def block_slot_mapping(block_ids, block_size: int = 16) -> np.ndarray:
    """int32 slot list that writes whole physical blocks: block_ids[i]'s tokens
    go to slots block_ids[i] * block_size + 0 .. block_size - 1, in that order.

    This is the caller's side of the pool write: an engine's model runner
    builds slot_mapping from its block tables ("vLLM Architecture and
    Installation", Example 3) and hands it to the write entry point, which only
    scatters rows to the slots it is given.  Rows of a [n, block_size, Hkv, d]
    block array reshaped to [n * block_size, Hkv, d] line up with these slots.
    """
    ids = np.asarray(block_ids, dtype=np.int64).reshape(-1)
    slots = ids[:, None] * block_size + np.arange(block_size, dtype=np.int64)[None, :]
    assert slots.size == 0 or int(slots.max()) < 2 ** 31
    return slots.reshape(-1).astype(np.int32)


def _uniform_ints(seed, purpose, lo, hi, n):
    return _rng(seed, _META, purpose).integers(lo, hi + 1, size=n).astype(np.int32)


def config(k: int, seed: int | None = None) -> Workload:
    """The workloads, numbered 1..9 as in the module docstring."""
    seed = k if seed is None else seed
    if k == 1:
        return Workload("paged decode, 1 layer, batch 1, ctx 256", seed, layers=1,
                        ctx_lens=np.array([256], np.int32), pool_blocks=64, max_blocks=16,
                        description="table = first 16 ids of a random permutation of 64 blocks")
    if k == 2:
        return Workload("paged decode, 1 layer, batch 8, ctx 4096", seed, layers=1,
                        ctx_lens=np.full(8, 4096, np.int32), pool_blocks=2 * 8 * 256,
                        max_blocks=256)
    if k == 3:
        return Workload("paged decode step, 32 layers, batch 32, ctx 4096", seed, layers=32,
                        ctx_lens=np.full(32, 4096, np.int32), pool_blocks=2 * 32 * 256,
                        max_blocks=256, fresh_tables_per_layer=True)
    if k == 4:
        lens = _uniform_ints(seed, 0, 1, 8192, 64)
        need = int((-(-lens.astype(np.int64) // 16)).sum())
        return Workload("paged decode, 1 layer, 64 ragged sequences, ctx U[1,8192]", seed,
                        layers=1, ctx_lens=lens, pool_blocks=2 * need, max_blocks=512,
                        key_boost_prob=0.01, key_boost=8.0)
    if k == 5:
        groups, gsize, pblocks = 16, 16, 128
        suffix = _uniform_ints(seed, 1, 0, 6144, groups * gsize)
        lens = (pblocks * 16 + suffix).astype(np.int32)
        need = groups * pblocks + int((-(-suffix.astype(np.int64) // 16)).sum())
        return Workload("paged decode, 1 layer, 256 sequences, 16 shared 2048-token prefixes",
                        seed, layers=1, ctx_lens=lens, pool_blocks=2 * need, max_blocks=512,
                        prefix_groups=(groups, gsize, pblocks))
    if k == 8:
        return Workload("paged decode step, 32 layers, batch 1, ctx 256 (launch-bound)", seed, layers=32,
                        ctx_lens=np.array([256], np.int32), pool_blocks=64, max_blocks=16,
                        fresh_tables_per_layer=True,
                        description="per layer: first 16 ids of a random permutation of 64 blocks")
    if k == 9:
        return Workload("paged decode, 1 layer, batch 1024, ctx 128", seed, layers=1,
                        ctx_lens=np.full(1024, 128, np.int32), pool_blocks=2 * 1024 * 8,
                        max_blocks=8)
    if k in (6, 7):
        chunk, hist, layers = (2016, 2016, 32) if k == 6 else (16352, 16352, 8)
        lens = np.array([hist + chunk] + [4096] * 32, np.int32)
        need = int((-(-lens.astype(np.int64) // 16)).sum())
        return Workload(f"mixed step, {layers} layers, 32 decodes at ctx 4096 + a {chunk}-token "
                        f"prompt chunk at position {hist}", seed, layers=layers, ctx_lens=lens,
                        pool_blocks=2 * need, max_blocks=int(-(-lens.max() // 16)),
                        q_lens=np.array([chunk] + [1] * 32, np.int32))
    raise ValueError(f"unknown workload {k}")


def custom(ctx_lens, *, seed=1234, layers=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
           block_size=16, pool_factor=2, max_blocks=None, prefix_groups=None,
           key_boost_prob=0.0, name="custom") -> Workload:
    """A small workload of the same structure, for tests."""
    lens = np.asarray(ctx_lens, dtype=np.int32)
    held = -(-lens.astype(np.int64) // block_size)
    if prefix_groups is not None:
        groups, gsize, pblocks = prefix_groups
        need = groups * pblocks + int((held - pblocks).sum())
    else:
        need = int(held.sum())
    if max_blocks is None:
        max_blocks = max(1, int(held.max()) if lens.size else 1)
    return Workload(name, seed, layers=layers, ctx_lens=lens, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                    pool_blocks=max(1, pool_factor * need), max_blocks=max_blocks,
                    prefix_groups=prefix_groups, key_boost_prob=key_boost_prob)
