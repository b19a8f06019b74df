/*
 * pa_oracle.c -- TEST INFRASTRUCTURE, not part of the product.
 *
 * A plain, slow, fp64 CPU reference for one batched decode step of attention
 * over a paged KV cache.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or constant with the HIP library under paged_kv_cache_64_amd/.
 *
 * What it follows (the pages are named by title and section):
 *  - "vLLM Architecture and Installation", Example 3 (paged KV cache block
 *    tables): a request's block table lists the physical blocks holding its
 *    tokens in order; the slot of logical position p is
 *    table[p / block_size] * block_size + p % block_size, and the attention
 *    kernel gathers every earlier key and value of the request by that map.
 *  - "Reading Inference Engine Codebases", Example 2: the attention scale is
 *    1/sqrt(head dimension) unless the model overrides it, so the scale is an
 *    argument; KV heads may be shared by several query heads (grouped-query
 *    attention).
 *  - "Reading Inference Engine Codebases", Example 6: softmax is computed in
 *    its max-shifted form exp(x - max) / sum.
 *  - "vLLM Architecture and Installation", Example 6 and "Batching and
 *    Scheduling", Example 1: page size = block size x KV heads x (key dim +
 *    value dim) x bytes per value; 128 KiB of F16 KV per token for the 8B
 *    shape.
 *
 * Readings where the pages are silent (each is a stated choice):
 *  - query head h uses KV head h / (num_q_heads / num_kv_heads) (contiguous
 *    groups);
 *  - the context of sequence s is exactly its positions [0, ctx_s); the
 *    newest token is already stored, so no causal mask is needed;
 *  - table entries at or past ceil(ctx_s / block_size) and slots past ctx_s in
 *    the last block are never read;
 *  - ctx_s == 0 gives an all-zero output row;
 *  - the same physical block may appear in several tables (and twice in one
 *    table); each occurrence is simply read;
 *  - in a chunked-prefill step (pa_oracle_prefill) the chunk's keys and
 *    values are already stored and query j of a q_len-token chunk sees
 *    positions 0 .. seq_len - q_len + j.
 *
 * Parity pins (tests/test_oracle_pins.py, tests/test_oracle_fp8.py,
 * tests/test_oracle_prefill.py): brute
 * force over a contiguous cache, torch's scaled_dot_product_attention in fp64,
 * permutation of block ids, ctx = 1, identical keys, the two-token sigmoid
 * form, V scaling, the pages' slot example and sizing figures; the E4M3
 * decoder and encoder against the format's closed forms and torch's
 * float8_e4m3fn.  No function here is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef PA_ORACLE_SOURCE_SHA256
#define PA_ORACLE_SOURCE_SHA256 "unknown"
#endif
/* sha256 of this file and the build flags (oracle/build.py); the loader reads
 * it from the library file and rebuilds a library made from other sources. */
__attribute__((used, visibility("default"))) const char pa_oracle_build_source[] =
    "pa-oracle-source-sha256:" PA_ORACLE_SOURCE_SHA256;

/* IEEE 754 binary16 -> double, written from the format's definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 *   e == 0      : subnormal, value = frac * 2^-24
 *   e == 31     : infinity (frac == 0) or NaN
 *   otherwise   : value = (1024 + frac) * 2^(e - 25)
 * Every binary16 value is exactly representable as a double. */
double pa_oracle_f16_to_f64(uint16_t bits)
{
    const int sign = (bits >> 15) & 1;
    const int e = (bits >> 10) & 0x1f;
    const int frac = bits & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)frac, -24);
    else if (e == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), e - 25);
    return sign ? -v : v;
}

/* Slot of logical position `pos` for one request ("vLLM Architecture and
 * Installation", Example 3): the table entry at pos / block_size names the
 * physical block, pos % block_size is the offset inside it. */
int64_t pa_oracle_slot(const int32_t *table_row, int32_t block_size, int64_t pos)
{
    return (int64_t)table_row[pos / block_size] * block_size + pos % block_size;
}

/* Bytes of K plus V for one token over all layers ("Batching and Scheduling",
 * Example 1: 128 KiB per token for 32 layers x 8 KV heads x 128 dims in F16). */
int64_t pa_oracle_kv_bytes_per_token(int32_t layers, int32_t kv_heads, int32_t head_dim,
                                     int32_t bytes_per_value)
{
    return (int64_t)layers * kv_heads * head_dim * 2 /* K and V */ * bytes_per_value;
}

/* Page size of one block in one layer ("vLLM Architecture and Installation",
 * Example 6): block size x KV heads x (key dim + value dim) x bytes. */
int64_t pa_oracle_page_bytes(int32_t block_size, int32_t kv_heads, int32_t key_dim,
                             int32_t value_dim, int32_t bytes_per_value)
{
    return (int64_t)block_size * kv_heads * (key_dim + value_dim) * bytes_per_value;
}

/*
 * One decode step of attention, one layer.
 *
 *   q            F16 bits [batch][num_q_heads][head_dim]
 *   k_slots      F16 bits [num_slots][num_kv_heads][head_dim]  (slot-indexed cache)
 *   v_slots      F16 bits [num_slots][num_kv_heads][head_dim]
 *   block_tables int32    [batch][max_blocks]
 *   ctx_lens     int32    [batch]
 *   out          double   [batch][num_q_heads][head_dim]
 *
 * For each sequence s and query head h (g = h / (num_q_heads/num_kv_heads)):
 *   z[t]  = scale * sum_i q[s][h][i] * K[slot(s,t)][g][i]      t = 0 .. ctx_s-1
 *   M     = max_t z[t]
 *   w[t]  = exp(z[t] - M),  L = sum_t w[t]
 *   out[s][h][i] = sum_t w[t] * V[slot(s,t)][g][i] / L
 * all in double, sums taken in increasing t.
 *
 * Returns 0 on success, 1 on a bad geometry, 2 when a table entry or a
 * context length points outside the given arrays, 3 on allocation failure.
 */
int pa_oracle_decode(const uint16_t *q, const uint16_t *k_slots, const uint16_t *v_slots,
                     int64_t num_slots, const int32_t *block_tables, int32_t max_blocks,
                     const int32_t *ctx_lens, int32_t batch, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, double scale,
                     double *out, int32_t num_threads)
{
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks < 0 || num_q_heads % num_kv_heads != 0)
        return 1;

    /* Every table entry that will be read must name a slot inside the arrays. */
    for (int32_t s = 0; s < batch; ++s) {
        const int64_t ctx = ctx_lens[s];
        if (ctx < 0 || ctx > (int64_t)max_blocks * block_size)
            return 2;
        const int32_t *row = block_tables + (int64_t)s * max_blocks;
        for (int64_t t = 0; t < ctx; ++t) {
            const int64_t slot = pa_oracle_slot(row, block_size, t);
            if (slot < 0 || slot >= num_slots)
                return 2;
        }
    }

    const int32_t group = num_q_heads / num_kv_heads;
    const int64_t rows = (int64_t)batch * num_q_heads;
    int failed = 0;

#ifdef _OPENMP
    if (num_threads <= 0)
        num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads) reduction(| : failed)
#endif
    for (int64_t r = 0; r < rows; ++r) {
        const int32_t s = (int32_t)(r / num_q_heads);
        const int32_t h = (int32_t)(r % num_q_heads);
        const int32_t g = h / group;
        const int64_t ctx = ctx_lens[s];
        const int32_t *row = block_tables + (int64_t)s * max_blocks;
        const uint16_t *qh = q + r * head_dim;
        double *o = out + r * head_dim;

        for (int32_t i = 0; i < head_dim; ++i)
            o[i] = 0.0;
        if (ctx == 0)
            continue;

        double *z = (double *)malloc(sizeof(double) * (size_t)ctx);
        double *qd = (double *)malloc(sizeof(double) * (size_t)head_dim);
        if (!z || !qd) {
            free(z);
            free(qd);
            failed |= 1;
            continue;
        }
        for (int32_t i = 0; i < head_dim; ++i)
            qd[i] = pa_oracle_f16_to_f64(qh[i]);

        /* scores, gathered through the block table */
        double m = -INFINITY;
        for (int64_t t = 0; t < ctx; ++t) {
            const int64_t slot = pa_oracle_slot(row, block_size, t);
            const uint16_t *kr = k_slots + (slot * num_kv_heads + g) * head_dim;
            double dot = 0.0;
            for (int32_t i = 0; i < head_dim; ++i)
                dot += qd[i] * pa_oracle_f16_to_f64(kr[i]);
            z[t] = scale * dot;
            if (z[t] > m)
                m = z[t];
        }

        /* max-shifted softmax weights and their sum */
        double l = 0.0;
        for (int64_t t = 0; t < ctx; ++t) {
            z[t] = exp(z[t] - m);
            l += z[t];
        }

        /* weighted sum of values */
        for (int64_t t = 0; t < ctx; ++t) {
            const int64_t slot = pa_oracle_slot(row, block_size, t);
            const uint16_t *vr = v_slots + (slot * num_kv_heads + g) * head_dim;
            for (int32_t i = 0; i < head_dim; ++i)
                o[i] += z[t] * pa_oracle_f16_to_f64(vr[i]);
        }
        for (int32_t i = 0; i < head_dim; ++i)
            o[i] /= l;

        free(z);
        free(qd);
    }
    return failed ? 3 : 0;
}

/*
 * Chunked prefill / mixed step of attention, one layer.
 *
 * "Batching and Scheduling", Example 5, and "vLLM Architecture and
 * Installation", Example 5: a step gives each request some number of new
 * tokens under a token budget -- one for a decoding request, a chunk of the
 * prompt for a prefilling one -- and there is no separate prefill or decode
 * phase.  Reading (stated): the new tokens' keys and values are already in
 * the cache when attention runs (as for the decode step), the chunk of
 * sequence s holds its last q_len_s positions, and query j of the chunk
 * (position p = seq_len_s - q_len_s + j) attends to positions 0 .. p of its
 * own sequence (causal attention over the paged history and the chunk).
 *
 *   q            F16 bits [total_q][num_q_heads][head_dim], the chunks packed
 *                in sequence order; sequence s owns rows
 *                query_start[s] .. query_start[s+1]-1
 *   k_slots      F16 bits [num_slots][num_kv_heads][head_dim]
 *   v_slots      F16 bits [num_slots][num_kv_heads][head_dim]
 *   block_tables int32    [batch][max_blocks]
 *   query_start  int32    [batch + 1], query_start[0] == 0, nondecreasing
 *   seq_lens     int32    [batch], seq_lens[s] >= q_len_s (tokens in the
 *                cache after this step's writes)
 *   out          double   [total_q][num_q_heads][head_dim]
 *
 * Row (j, h) of sequence s, with n = seq_len_s - q_len_s + j + 1 visible
 * positions and g = h / (num_q_heads/num_kv_heads):
 *   z[t] = scale * sum_i q[row][h][i] * K[slot(s,t)][g][i]     t = 0 .. n-1
 *   out[row][h][i] = sum_t exp(z[t] - max z) * V[slot(s,t)][g][i] / sum_t exp(z[t] - max z)
 * in double, sums in increasing t.
 *
 * Returns 0 on success, 1 on a bad geometry, 2 when the query offsets,
 * lengths or table entries do not fit the arrays, 3 on allocation failure.
 */
int pa_oracle_prefill(const uint16_t *q, const uint16_t *k_slots, const uint16_t *v_slots,
                      int64_t num_slots, const int32_t *block_tables, int32_t max_blocks,
                      const int32_t *query_start, const int32_t *seq_lens, int32_t batch,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, double scale, double *out, int32_t num_threads)
{
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks < 0 || num_q_heads % num_kv_heads != 0)
        return 1;
    if (query_start[0] != 0)
        return 2;
    for (int32_t s = 0; s < batch; ++s) {
        const int64_t q_len = (int64_t)query_start[s + 1] - query_start[s];
        const int64_t len = seq_lens[s];
        if (q_len < 0 || len < q_len || len > (int64_t)max_blocks * block_size)
            return 2;
        const int32_t *row = block_tables + (int64_t)s * max_blocks;
        for (int64_t t = 0; t < len; ++t) {
            const int64_t slot = pa_oracle_slot(row, block_size, t);
            if (slot < 0 || slot >= num_slots)
                return 2;
        }
    }

    const int32_t group = num_q_heads / num_kv_heads;
    const int64_t total_q = query_start[batch];
    const int64_t rows = total_q * num_q_heads;
    int failed = 0;

#ifdef _OPENMP
    if (num_threads <= 0)
        num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads) reduction(| : failed)
#endif
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t qi = r / num_q_heads; /* packed query row */
        const int32_t h = (int32_t)(r % num_q_heads);
        const int32_t g = h / group;
        int32_t s = 0; /* the sequence owning query row qi */
        while (query_start[s + 1] <= qi)
            ++s;
        const int64_t q_len = (int64_t)query_start[s + 1] - query_start[s];
        const int64_t j = qi - query_start[s];
        const int64_t n = (int64_t)seq_lens[s] - q_len + j + 1; /* positions 0 .. n-1 */
        const int32_t *row = block_tables + (int64_t)s * max_blocks;
        const uint16_t *qh = q + r * head_dim;
        double *o = out + r * head_dim;

        for (int32_t i = 0; i < head_dim; ++i)
            o[i] = 0.0;
        double *z = (double *)malloc(sizeof(double) * (size_t)n);
        double *qd = (double *)malloc(sizeof(double) * (size_t)head_dim);
        if (!z || !qd) {
            free(z);
            free(qd);
            failed |= 1;
            continue;
        }
        for (int32_t i = 0; i < head_dim; ++i)
            qd[i] = pa_oracle_f16_to_f64(qh[i]);

        double m = -INFINITY;
        for (int64_t t = 0; t < n; ++t) {
            const int64_t slot = pa_oracle_slot(row, block_size, t);
            const uint16_t *kr = k_slots + (slot * num_kv_heads + g) * head_dim;
            double dot = 0.0;
            for (int32_t i = 0; i < head_dim; ++i)
                dot += qd[i] * pa_oracle_f16_to_f64(kr[i]);
            z[t] = scale * dot;
            if (z[t] > m)
                m = z[t];
        }
        double l = 0.0;
        for (int64_t t = 0; t < n; ++t) {
            z[t] = exp(z[t] - m);
            l += z[t];
        }
        for (int64_t t = 0; t < n; ++t) {
            const int64_t slot = pa_oracle_slot(row, block_size, t);
            const uint16_t *vr = v_slots + (slot * num_kv_heads + g) * head_dim;
            for (int32_t i = 0; i < head_dim; ++i)
                o[i] += z[t] * pa_oracle_f16_to_f64(vr[i]);
        }
        for (int32_t i = 0; i < head_dim; ++i)
            o[i] /= l;

        free(z);
        free(qd);
    }
    return failed ? 3 : 0;
}

/* ---- FP8 E4M3 (OCP "e4m3fn") key/value storage ---------------------------
 * The pages state only that an FP8 KV cache stores one byte per value and
 * halves the page ("vLLM Architecture and Installation", Example 6); the
 * format is read as OCP E4M3: 1 sign bit, 4 exponent bits (bias 7), 3
 * fraction bits, no infinities, S.1111.111 = NaN, largest finite 448.  A
 * stored code means code_value * scale for a per-layer scale of K or of V. */

/* code -> double, from the format definition:
 *   e == 0            : frac * 2^-9 (subnormal)
 *   e == 15, frac == 7: NaN
 *   otherwise         : (8 + frac) * 2^(e - 10) */
double pa_oracle_e4m3_to_f64(uint8_t code)
{
    const int sign = (code >> 7) & 1;
    const int e = (code >> 3) & 0xf;
    const int frac = code & 0x7;
    double v;
    if (e == 15 && frac == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)frac, -9);
    else
        v = ldexp((double)(8 + frac), e - 10);
    return sign ? -v : v;
}

/* double -> code: round to nearest, ties to even, magnitudes beyond 448
 * saturate to 448 (no infinities in the format); NaN -> 0x7f.  Written as a
 * search over the 127 non-negative finite codes, which are ordered by value. */
uint8_t pa_oracle_f64_to_e4m3(double x)
{
    if (isnan(x))
        return 0x7f;
    const int neg = signbit(x) ? 1 : 0;
    double a = fabs(x);
    uint8_t best = 0;
    if (a >= 448.0) {
        best = 0x7e;
    } else {
        /* the largest code whose value is <= a, then compare with the next */
        uint8_t lo = 0;
        for (uint8_t c = 0; c < 0x7f; ++c)
            if (pa_oracle_e4m3_to_f64(c) <= a)
                lo = c;
        const double vlo = pa_oracle_e4m3_to_f64(lo);
        if (lo == 0x7e || vlo == a) {
            best = lo;
        } else {
            const double vhi = pa_oracle_e4m3_to_f64((uint8_t)(lo + 1));
            const double dlo = a - vlo, dhi = vhi - a;
            if (dlo < dhi)
                best = lo;
            else if (dhi < dlo)
                best = (uint8_t)(lo + 1);
            else
                best = (lo & 1) ? (uint8_t)(lo + 1) : lo; /* tie: even code */
        }
    }
    return (uint8_t)(best | (neg << 7));
}

/* The stored code of an F16 value written into an FP8 pool with scale s:
 * the product fl32(fl32(x) * r), r = fl32(1 / s), rounded as above. */
uint8_t pa_oracle_quantize_e4m3(uint16_t f16_bits, float inv_scale)
{
    const float x = (float)pa_oracle_f16_to_f64(f16_bits);
    const float y = x * inv_scale;
    return pa_oracle_f64_to_e4m3((double)y);
}

/* Decode step over FP8 pools: identical to pa_oracle_decode except that a
 * key or value component is code_value * k_scale (or v_scale). */
int pa_oracle_decode_e4m3(const uint16_t *q, const uint8_t *k_slots, const uint8_t *v_slots,
                          int64_t num_slots, const int32_t *block_tables, int32_t max_blocks,
                          const int32_t *ctx_lens, int32_t batch, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size, double scale,
                          double k_scale, double v_scale, double *out, int32_t num_threads)
{
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks < 0 || num_q_heads % num_kv_heads != 0)
        return 1;
    for (int32_t s = 0; s < batch; ++s) {
        const int64_t ctx = ctx_lens[s];
        if (ctx < 0 || ctx > (int64_t)max_blocks * block_size)
            return 2;
        const int32_t *row = block_tables + (int64_t)s * max_blocks;
        for (int64_t t = 0; t < ctx; ++t) {
            const int64_t slot = pa_oracle_slot(row, block_size, t);
            if (slot < 0 || slot >= num_slots)
                return 2;
        }
    }
    const int32_t group = num_q_heads / num_kv_heads;
    const int64_t rows = (int64_t)batch * num_q_heads;
    int failed = 0;
#ifdef _OPENMP
    if (num_threads <= 0)
        num_threads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(num_threads) reduction(| : failed)
#endif
    for (int64_t r = 0; r < rows; ++r) {
        const int32_t s = (int32_t)(r / num_q_heads);
        const int32_t h = (int32_t)(r % num_q_heads);
        const int32_t g = h / group;
        const int64_t ctx = ctx_lens[s];
        const int32_t *row = block_tables + (int64_t)s * max_blocks;
        double *o = out + r * head_dim;
        for (int32_t i = 0; i < head_dim; ++i)
            o[i] = 0.0;
        if (ctx == 0)
            continue;
        double *z = (double *)malloc(sizeof(double) * (size_t)ctx);
        double *qd = (double *)malloc(sizeof(double) * (size_t)head_dim);
        if (!z || !qd) {
            free(z);
            free(qd);
            failed |= 1;
            continue;
        }
        for (int32_t i = 0; i < head_dim; ++i)
            qd[i] = pa_oracle_f16_to_f64(q[r * head_dim + i]);
        double m = -INFINITY;
        for (int64_t t = 0; t < ctx; ++t) {
            const int64_t slot = pa_oracle_slot(row, block_size, t);
            const uint8_t *kr = k_slots + (slot * num_kv_heads + g) * head_dim;
            double dot = 0.0;
            for (int32_t i = 0; i < head_dim; ++i)
                dot += qd[i] * (pa_oracle_e4m3_to_f64(kr[i]) * k_scale);
            z[t] = scale * dot;
            if (z[t] > m)
                m = z[t];
        }
        double l = 0.0;
        for (int64_t t = 0; t < ctx; ++t) {
            z[t] = exp(z[t] - m);
            l += z[t];
        }
        for (int64_t t = 0; t < ctx; ++t) {
            const int64_t slot = pa_oracle_slot(row, block_size, t);
            const uint8_t *vr = v_slots + (slot * num_kv_heads + g) * head_dim;
            for (int32_t i = 0; i < head_dim; ++i)
                o[i] += z[t] * (pa_oracle_e4m3_to_f64(vr[i]) * v_scale);
        }
        for (int32_t i = 0; i < head_dim; ++i)
            o[i] /= l;
        free(z);
        free(qd);
    }
    return failed ? 3 : 0;
}
