"""Helpers shared by the GPU tests: put a seeded workload into a device pool
through pa_write_kv, run the library, and compare with the oracle.

Both sides draw from workloads.py; the GPU side sees the values only through
pa_write_kv, the oracle only through its own slot-indexed host cache.
"""
import math

import numpy as np
import torch

import oracle
import paged_kv_cache_64_amd as pa
import workloads

# Tolerance for F16 outputs against the fp64 oracle.
MAX_ABS = 2e-3
REL_L2 = 1e-3


def report(name, **kw):
    print(f"[gpu-test] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


class Staged:
    """A workload's layers written into a device pool, plus host copies for the oracle."""

    def __init__(self, w, layers=(0,), pool_layers=None, fill=float("nan"), keep_host=True,
                 dtype=pa.PA_F16, kv_scales=(1.0, 1.0)):
        """dtype PA_FP8_E4M3 stores codes; kv_scales = (k_scale, v_scale) for every layer."""
        self.w = w
        self.layers = tuple(layers)
        nl = pool_layers if pool_layers is not None else max(self.layers) + 1
        self.pool = pa.Pool(nl, w.pool_blocks, w.num_kv_heads, w.head_dim, w.block_size,
                            fill=fill, dtype=dtype)
        self.fp8 = dtype == pa.PA_FP8_E4M3
        self.kv_scales = tuple(float(x) for x in kv_scales)
        self.lens = torch.from_numpy(w.ctx_lens.copy()).cuda()
        self.host = {}
        self.dev = {}
        for layer in self.layers:
            if self.fp8:
                self.pool.set_scales(layer, *self.kv_scales)
            ids, k, v = w.kv_blocks(layer)
            write_blocks(self.pool, layer, ids, k, v)
            q = w.q(layer)
            tables = w.tables(layer)
            self.dev[layer] = (torch.from_numpy(q).cuda(), torch.from_numpy(tables).cuda())
            if keep_host:
                self.host[layer] = (q, tables, ids, k, v)
        torch.cuda.synchronize()

    def decode(self, layer, phases=False, max_context_len=None, workspace=None, scale=None):
        q, tables = self.dev[layer]
        out = torch.empty_like(q)
        mcl = self.w.max_context_len if max_context_len is None else max_context_len
        self.pool.decode(layer, q, out, tables, self.lens, mcl,
                         self.w.scale if scale is None else scale, workspace=workspace,
                         phases=phases)
        torch.cuda.synchronize()
        return out

    def reference(self, layer, seqs=None, scale=None):
        q, tables, ids, k, v = self.host[layer]
        lens = self.w.ctx_lens
        if seqs is not None:
            seqs = np.asarray(seqs)
            q, tables, lens = q[seqs], tables[seqs], lens[seqs]
        kc, vc, tables = oracle.relabelled_cache(ids, k, v, tables, lens, self.w.block_size)
        scale = self.w.scale if scale is None else scale
        if self.fp8:
            ks, vs = self.kv_scales
            return oracle.decode_e4m3(q, oracle.quantize_e4m3(kc, ks), oracle.quantize_e4m3(vc, vs),
                                      tables, lens, scale, self.w.block_size, ks, vs)
        return oracle.decode(q, kc, vc, tables, lens, scale, self.w.block_size)

    def close(self):
        self.pool.close()


def write_blocks(pool, layer, ids, k_blocks, v_blocks):
    """Stores whole physical blocks through pa_write_kv: k_blocks[i] ([B, Hkv, d],
    host F16) goes to block ids[i]."""
    n = int(np.asarray(ids).shape[0]) * pool.block_size
    slots = workloads.block_slot_mapping(ids, pool.block_size)
    rows = lambda x: torch.from_numpy(np.ascontiguousarray(x).reshape(n, pool.num_kv_heads,
                                                                     pool.head_dim)).cuda()
    pool.write(layer, rows(k_blocks), rows(v_blocks), torch.from_numpy(slots).cuda())


def compare(name, gpu_out, ref, max_abs=MAX_ABS, rel_l2=REL_L2):
    """Element-by-element comparison in fp64; returns (max_abs, rel_l2)."""
    g = gpu_out.detach().cpu().numpy().astype(np.float64) if torch.is_tensor(gpu_out) else gpu_out
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite output"
    err = np.abs(g - ref)
    mx = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(g - ref) / denom) if denom > 0 else float(np.linalg.norm(g))
    if err.size:
        worst = np.unravel_index(int(err.argmax()), err.shape)
    else:
        worst = ()
    report(name, max_abs=f"{mx:.3e}", rel_l2=f"{rel:.3e}", worst=worst)
    assert mx <= max_abs, f"{name}: max |err| {mx:.3e} > {max_abs} at {worst}"
    assert rel <= rel_l2, f"{name}: rel L2 {rel:.3e} > {rel_l2}"
    return mx, rel


def slots_of(table_row, positions, block_size):
    """Slots of logical positions of one sequence (host side of the caller)."""
    return [int(table_row[p // block_size]) * block_size + p % block_size for p in positions]


def scale_of(d):
    return 1.0 / math.sqrt(d)
