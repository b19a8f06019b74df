"""Byte and time models used for reporting.

decode_step_model restates the pages' modelled decode step ("Batching and
Scheduling", Example 1): a step reads the weights once plus every sequence's
own KV cache, does 2 x params flops per sequence, and takes the larger of
bytes / bandwidth and flops / peak.

The algorithmic byte counts below are what one decode step of attention
must move per layer: every sequence reads its whole context of K and V
(kv_heads x head_dim x 2 x 2 bytes per token), its F16 query, its block
table entries, and writes its F16 output.
"""
from __future__ import annotations

import math

MI355X_HBM_BYTES_PER_S = 8.0e12       # AMD published peak
MI355X_F16_DENSE_FLOPS = 2.5e15       # AMD published dense MFMA peak (no sparsity)


def decode_step_model(params, bits_per_weight, peak_flops, bandwidth, context,
                      kv_bytes_per_token, batch):
    weight_bytes = params * bits_per_weight / 8
    step_bytes = weight_bytes + batch * context * kv_bytes_per_token
    flops = 2 * params * batch
    step = max(step_bytes / bandwidth, flops / peak_flops)
    return {
        "batch": batch,
        "bytes_per_step_GB": step_bytes / 1e9,
        "step_ms": step * 1e3,
        "tok_s_total": batch / step,
        "tok_s_per_seq": 1 / step,
        "flop_util_pct": 100 * flops / step / peak_flops,
        "kv_GB": batch * context * kv_bytes_per_token / 1e9,
    }


def sequences_that_fit(params, bits_per_weight, vram_bytes, context, kv_bytes_per_token):
    return math.floor((vram_bytes - params * bits_per_weight / 8) / (context * kv_bytes_per_token))


def kv_bytes_per_token_layer(num_kv_heads, head_dim, elem_bytes=2):
    return num_kv_heads * head_dim * 2 * elem_bytes


def split_kernel_bytes(ctx_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                       kv_elem_bytes=2):
    """Algorithmic bytes of one partial-attention launch (one layer): all K/V of
    every context (kv_elem_bytes per value: 2 for F16, 1 for FP8), each F16
    query once, each table entry read once."""
    kv = 0
    table = 0
    for c in ctx_lens:
        c = int(c)
        kv += c * kv_bytes_per_token_layer(num_kv_heads, head_dim, kv_elem_bytes)
        table += 4 * (-(-c // block_size))
    q = len(ctx_lens) * num_q_heads * head_dim * 2
    return {"kv": kv, "q": q, "table": table, "total": kv + q + table}


def step_bytes(ctx_lens, num_q_heads, num_kv_heads, head_dim, block_size, layers,
               kv_elem_bytes=2):
    """Algorithmic bytes of a whole decode step: per layer the split-kernel bytes
    plus the F16 output, plus the new token's K/V written per sequence."""
    per = split_kernel_bytes(ctx_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                             kv_elem_bytes)
    out = len(ctx_lens) * num_q_heads * head_dim * 2
    new_kv = len(ctx_lens) * kv_bytes_per_token_layer(num_kv_heads, head_dim, kv_elem_bytes)
    return layers * (per["total"] + out + new_kv)
