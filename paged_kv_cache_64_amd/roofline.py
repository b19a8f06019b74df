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
    """Algorithmic bytes of one decode-attention launch (one layer): all K/V of
    every context (kv_elem_bytes per value: 2 for F16, 1 for FP8), each F16
    query read once, each table entry read once, and each F16 output row
    written once."""
    kv = 0
    table = 0
    for c in ctx_lens:
        c = int(c)
        kv += c * kv_bytes_per_token_layer(num_kv_heads, head_dim, kv_elem_bytes)
        table += 4 * (-(-c // block_size))
    q = len(ctx_lens) * num_q_heads * head_dim * 2
    out = len(ctx_lens) * num_q_heads * head_dim * 2
    return {"kv": kv, "q": q, "table": table, "out": out, "total": kv + q + table + out}


def step_bytes(ctx_lens, num_q_heads, num_kv_heads, head_dim, block_size, layers,
               kv_elem_bytes=2):
    """Algorithmic bytes of a whole decode step: per layer the launch bytes above
    plus the new token's K/V written per sequence."""
    per = split_kernel_bytes(ctx_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                             kv_elem_bytes)
    new_kv = len(ctx_lens) * kv_bytes_per_token_layer(num_kv_heads, head_dim, kv_elem_bytes)
    return layers * (per["total"] + new_kv)


# The pages' modelled decode step ("Batching and Scheduling", Example 1): an
# 8.03 B-parameter model at 4.5 bits per weight on an RTX 4090 (1,008 GB/s,
# 165.2 TFLOP/s F16 tensor), every sequence at 4,096 tokens of 128 KiB F16 KV.
PAGES_MODEL = {"params": 8.03e9, "bits_per_weight": 4.5, "peak_flops": 165.2e12,
               "bandwidth": 1008e9, "context": 4096, "kv_bytes_per_token": 131072}


def pages_context(batches=(1, 8, 16, 32)):
    """The pages' modelled rows (context only, not a target), and the same model
    evaluated at MI355X's published peaks for comparison."""
    m = PAGES_MODEL
    rows = []
    for b in batches:
        r = decode_step_model(m["params"], m["bits_per_weight"], m["peak_flops"], m["bandwidth"],
                              m["context"], m["kv_bytes_per_token"], b)
        x = decode_step_model(m["params"], m["bits_per_weight"], MI355X_F16_DENSE_FLOPS,
                              MI355X_HBM_BYTES_PER_S, m["context"], m["kv_bytes_per_token"], b)
        rows.append({"batch": b, "bytes_per_step_GB": round(r["bytes_per_step_GB"], 2),
                     "kv_GB": round(r["kv_GB"], 2), "rtx4090_step_ms": round(r["step_ms"], 2),
                     "rtx4090_tok_s": round(r["tok_s_total"], 1),
                     "mi355x_peak_step_ms": round(x["step_ms"], 3),
                     "mi355x_peak_tok_s": round(x["tok_s_total"], 1)})
    return {"source": "Batching and Scheduling, Example 1: a modelled whole-model decode step "
                      "(weights read once + every sequence's KV), max(bytes / bandwidth, flops / peak)",
            "model": dict(m), "rows": rows,
            "note": "context only: the pages model the whole model's step on an RTX 4090; "
                    "this bench times attention alone, whose KV share at batch 32 is kv_GB"}
