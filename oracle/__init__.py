"""fp64 CPU oracle for one decode step of paged attention.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  The product library
(paged_kv_cache_64_amd) never imports it, and it never imports the product.

The arithmetic lives in pa_oracle.c; this module only marshals numpy arrays
into it and builds the oracle's own slot-indexed host cache from the seeded
generator's block contents (no device layout is involved).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("PA_ORACLE_LIB") or _build.LIB
        if os.path.abspath(path) == _build.DEFAULT_LIB and not _build.is_current(path):
            _build.build(lib=path)   # missing, or built from other sources
        lib = ctypes.CDLL(path)
        lib.pa_oracle_f16_to_f64.restype = ctypes.c_double
        lib.pa_oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.pa_oracle_slot.restype = ctypes.c_int64
        lib.pa_oracle_slot.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64]
        lib.pa_oracle_kv_bytes_per_token.restype = ctypes.c_int64
        lib.pa_oracle_kv_bytes_per_token.argtypes = [ctypes.c_int32] * 4
        lib.pa_oracle_page_bytes.restype = ctypes.c_int64
        lib.pa_oracle_page_bytes.argtypes = [ctypes.c_int32] * 5
        lib.pa_oracle_e4m3_to_f64.restype = ctypes.c_double
        lib.pa_oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.pa_oracle_f64_to_e4m3.restype = ctypes.c_uint8
        lib.pa_oracle_f64_to_e4m3.argtypes = [ctypes.c_double]
        lib.pa_oracle_quantize_e4m3.restype = ctypes.c_uint8
        lib.pa_oracle_quantize_e4m3.argtypes = [ctypes.c_uint16, ctypes.c_float]
        lib.pa_oracle_decode_e4m3.restype = ctypes.c_int
        lib.pa_oracle_decode_e4m3.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_void_p, ctypes.c_int32]
        lib.pa_oracle_prefill.restype = ctypes.c_int
        lib.pa_oracle_prefill.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_double, ctypes.c_void_p, ctypes.c_int32]
        lib.pa_oracle_decode.restype = ctypes.c_int
        lib.pa_oracle_decode.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_double, ctypes.c_void_p, ctypes.c_int32]
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def f16_to_f64(bits: int) -> float:
    """binary16 bit pattern -> exact double (the oracle's own decoder)."""
    return _load().pa_oracle_f16_to_f64(int(bits) & 0xFFFF)


def slot(table_row, block_size: int, pos: int) -> int:
    row = np.ascontiguousarray(table_row, dtype=np.int32)
    return int(_load().pa_oracle_slot(_ptr(row), block_size, pos))


def kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_value) -> int:
    return int(_load().pa_oracle_kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_value))


def page_bytes(block_size, kv_heads, key_dim, value_dim, bytes_per_value) -> int:
    return int(_load().pa_oracle_page_bytes(block_size, kv_heads, key_dim, value_dim,
                                            bytes_per_value))


def host_cache(num_blocks, block_size, block_ids, blocks, fill=np.nan):
    """Slot-indexed host cache [num_blocks*block_size, kv_heads, head_dim] (F16).

    `blocks` holds the contents of the physical blocks named by `block_ids`,
    shaped [n, block_size, kv_heads, head_dim]; every other slot gets `fill`.
    """
    blocks = np.asarray(blocks, dtype=np.float16)
    n, b, hkv, d = blocks.shape
    assert b == block_size
    cache = np.full((num_blocks, block_size, hkv, d), fill, dtype=np.float16)
    cache[np.asarray(block_ids, dtype=np.int64)] = blocks
    return cache.reshape(num_blocks * block_size, hkv, d)


def decode(q, k_slots, v_slots, block_tables, ctx_lens, scale, block_size, threads=0):
    """fp64 attention output [batch, num_q_heads, head_dim] for one layer.

    q: F16 [batch, Hq, d]; k_slots/v_slots: F16 [num_slots, Hkv, d];
    block_tables: int32 [batch, max_blocks]; ctx_lens: int32 [batch].
    """
    q = np.ascontiguousarray(q, dtype=np.float16)
    k_slots = np.ascontiguousarray(k_slots, dtype=np.float16)
    v_slots = np.ascontiguousarray(v_slots, dtype=np.float16)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    batch, hq, d = q.shape
    num_slots, hkv, d2 = k_slots.shape
    assert d2 == d and v_slots.shape == k_slots.shape
    assert tables.ndim == 2 and tables.shape[0] == batch and lens.shape == (batch,)
    out = np.empty((batch, hq, d), dtype=np.float64)
    rc = _load().pa_oracle_decode(
        _ptr(q.view(np.uint16)), _ptr(k_slots.view(np.uint16)), _ptr(v_slots.view(np.uint16)),
        num_slots, _ptr(tables), tables.shape[1], _ptr(lens), batch, hq, hkv, d, block_size,
        float(scale), _ptr(out), int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected its inputs (code {rc})")
    return out


def prefill(q, k_slots, v_slots, block_tables, query_start, seq_lens, scale, block_size,
            threads=0):
    """fp64 output [total_q, num_q_heads, head_dim] of a chunked-prefill / mixed
    step: sequence s owns packed query rows query_start[s] .. query_start[s+1]-1
    (its last q_len positions, already in the cache) and query j sees positions
    0 .. seq_lens[s] - q_len + j.

    q: F16 [total_q, Hq, d]; k_slots/v_slots: F16 [num_slots, Hkv, d];
    block_tables: int32 [batch, max_blocks]; query_start: int32 [batch + 1];
    seq_lens: int32 [batch].
    """
    q = np.ascontiguousarray(q, dtype=np.float16)
    k_slots = np.ascontiguousarray(k_slots, dtype=np.float16)
    v_slots = np.ascontiguousarray(v_slots, dtype=np.float16)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    starts = np.ascontiguousarray(query_start, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    batch = lens.shape[0]
    total_q, hq, d = q.shape
    num_slots, hkv, d2 = k_slots.shape
    assert d2 == d and v_slots.shape == k_slots.shape
    assert tables.ndim == 2 and tables.shape[0] == batch and starts.shape == (batch + 1,)
    assert int(starts[-1]) == total_q
    out = np.empty((total_q, hq, d), dtype=np.float64)
    rc = _load().pa_oracle_prefill(
        _ptr(q.view(np.uint16)), _ptr(k_slots.view(np.uint16)), _ptr(v_slots.view(np.uint16)),
        num_slots, _ptr(tables), tables.shape[1], _ptr(starts), _ptr(lens), batch, hq, hkv, d,
        block_size, float(scale), _ptr(out), int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected its inputs (code {rc})")
    return out


def relabelled_cache(ids, k_blocks, v_blocks, tables, ctx_lens, block_size):
    """Compact slot-indexed caches for the oracle plus tables rewritten to match.

    Block ids[i] becomes block i, so the caches are the block contents
    themselves ([n*B, Hkv, d], no copy).  Relabelling physical blocks does not
    change the result (a pinned invariance).  Table entries past a sequence's
    context are left as 0.
    """
    ids = np.asarray(ids, dtype=np.int64)
    tables = np.asarray(tables)
    held = -(-np.asarray(ctx_lens, dtype=np.int64) // block_size)
    order = np.argsort(ids, kind="stable")
    sorted_ids = ids[order]
    out_tables = np.zeros_like(tables, dtype=np.int32)
    for s in range(tables.shape[0]):
        row = tables[s, :held[s]]
        pos = np.minimum(np.searchsorted(sorted_ids, row), max(len(ids) - 1, 0))
        if row.size and not np.all(sorted_ids[pos] == row):
            raise ValueError(f"sequence {s} names a block that is not among ids")
        out_tables[s, :held[s]] = order[pos]
    n, b, hkv, d = k_blocks.shape
    return k_blocks.reshape(n * b, hkv, d), v_blocks.reshape(n * b, hkv, d), out_tables


def e4m3_to_f64(code: int) -> float:
    """E4M3 code -> exact double (the oracle's own decoder)."""
    return _load().pa_oracle_e4m3_to_f64(int(code) & 0xFF)


def f64_to_e4m3(x: float) -> int:
    """double -> E4M3 code: nearest, ties to even, saturating at 448."""
    return int(_load().pa_oracle_f64_to_e4m3(float(x)))


def quantize_e4m3(values_f16, scale: float) -> np.ndarray:
    """Codes an FP8 pool holds for F16 values written with this scale:
    fl32(fl32(x) * fl32(1/scale)) rounded to nearest even, saturating."""
    v = np.ascontiguousarray(values_f16, dtype=np.float16)
    inv = float(np.float32(1.0 / scale))
    lib = _load()
    # one call of the oracle's routine per F16 bit pattern, then a lookup
    table = np.fromiter((lib.pa_oracle_quantize_e4m3(b, inv) for b in range(1 << 16)),
                        dtype=np.uint8, count=1 << 16)
    out = table[v.reshape(-1).view(np.uint16)]
    return out.reshape(v.shape)


def decode_e4m3(q, k_codes, v_codes, block_tables, ctx_lens, scale, block_size, k_scale, v_scale,
                threads=0):
    """fp64 attention over FP8 (E4M3) slot caches [num_slots, Hkv, d] of codes."""
    q = np.ascontiguousarray(q, dtype=np.float16)
    k_codes = np.ascontiguousarray(k_codes, dtype=np.uint8)
    v_codes = np.ascontiguousarray(v_codes, dtype=np.uint8)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    batch, hq, d = q.shape
    num_slots, hkv, d2 = k_codes.shape
    assert d2 == d and v_codes.shape == k_codes.shape
    out = np.empty((batch, hq, d), dtype=np.float64)
    rc = _load().pa_oracle_decode_e4m3(
        _ptr(q.view(np.uint16)), _ptr(k_codes), _ptr(v_codes), num_slots, _ptr(tables),
        tables.shape[1], _ptr(lens), batch, hq, hkv, d, block_size, float(scale), float(k_scale),
        float(v_scale), _ptr(out), int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected its inputs (code {rc})")
    return out


def prefill_e4m3(q, k_codes, v_codes, block_tables, query_start, seq_lens, scale, block_size,
                 k_scale, v_scale, threads=0):
    """fp64 output of a chunked-prefill / mixed step over FP8 (E4M3) slot caches.

    Query j of sequence s's q_len-token chunk attends exactly as a one-token
    decode whose context is the positions it sees, 0 .. seq_len - q_len + j
    (the identity the F16 prefill oracle is pinned to), so every packed row is
    handed to decode_e4m3 with its own context length and its sequence's table.
    """
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    starts = np.asarray(query_start, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    batch = lens.shape[0]
    assert starts.shape == (batch + 1,) and starts[0] == 0
    q_lens = np.diff(starts)
    if np.any(q_lens < 0) or np.any(lens < q_lens):
        raise ValueError("query offsets do not fit the sequence lengths")
    owner = np.repeat(np.arange(batch), q_lens)
    j = np.arange(int(starts[-1])) - starts[owner]
    ctx = (lens[owner] - q_lens[owner] + j + 1).astype(np.int32)
    return decode_e4m3(q, k_codes, v_codes, tables[owner], ctx, scale, block_size, k_scale,
                       v_scale, threads)
