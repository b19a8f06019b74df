/*
 * pa.h -- paged decode attention for MI355X (gfx950), C ABI.
 *
 * One batched decode step of attention over a paged KV cache: each active
 * sequence contributes one query token; its keys and values live in
 * fixed-size blocks that a per-sequence block table scatters through a shared
 * pool ("vLLM Architecture and Installation", Example 3: a block table maps a
 * request's logical positions to physical blocks; new keys and values are
 * written to slot table[p / block_size] * block_size + p % block_size, and
 * attention gathers a sequence's earlier keys and values by the same map).
 *
 * For sequence s, query head h, with g = h / (num_q_heads / num_kv_heads)
 * (query heads share KV heads in contiguous groups; "Reading Inference Engine
 * Codebases", Example 2, and "Batching and Scheduling", Example 10) and
 * ctx = context_lens[s]:
 *     z_t = scale * <q[s][h], K[slot(s,t)][g]>            t in [0, ctx)
 *     out[s][h] = sum_t softmax(z)_t * V[slot(s,t)][g]
 * with the max-shifted softmax ("Reading Inference Engine Codebases",
 * Example 6) and scale usually 1/sqrt(head_dim) ("Reading Inference Engine
 * Codebases", Example 2).  Queries are F16; keys and values are F16, or FP8
 * E4M3 codes times a per-layer scale (pa_pool_set_scales); accumulation is
 * fp32; the output is rounded once to F16 (round to nearest even).  ctx == 0
 * gives zeros.
 *
 * Memory.  Every pointer argument named *_dev is a device pointer owned by
 * the caller (for example a torch tensor's data_ptr()).  The library never
 * allocates or frees device memory.  A pa_pool handle lives in host memory
 * and holds only the geometry and the two pool base pointers; the caller
 * keeps the pool buffers alive until all stream work using them completes.
 *
 * Streams.  Calls that take a hipStream_t only enqueue work on that stream
 * and return before the GPU finishes.  pa_decode calls may run concurrently
 * on different streams when they use distinct workspaces and outputs.
 *
 * Errors.  Every entry point returns a pa_status and never throws.  Host-side
 * checks run synchronously before anything is enqueued.  Values that live on
 * the device (table entries, context lengths, slots) are not validated, since
 * that would need a synchronisation: table entries must lie in
 * [0, num_blocks) and context lengths in [0, max_context_len].  The kernels
 * clamp them so that a bad value cannot make them read or write outside the
 * pool or the tables; the numbers produced from such a value are unspecified.
 *
 * Geometry supported by this build: head_dim 128, block_size 16, F16 or FP8
 * (E4M3) keys and values, F16 queries and outputs, num_q_heads = 4 *
 * num_kv_heads, contexts (max_context_len, host lengths) of at most 2^30
 * tokens and block tables at most 2^26 entries wide.  Other values return
 * PA_ERR_UNSUPPORTED.  Every schedule
 * (decode, shared-prefix cascade, chunked prefill / mixed) runs on both pool
 * types.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent geometry */
    PA_ERR_UNSUPPORTED = -2, /* geometry outside what this build supports */
    PA_ERR_WORKSPACE = -3,   /* workspace smaller than pa_decode_workspace_bytes() */
    PA_ERR_HIP = -4          /* a HIP runtime call or a kernel launch failed */
} pa_status;

typedef enum {
    PA_F16 = 1,      /* IEEE binary16 keys and values */
    PA_FP8_E4M3 = 2  /* one byte per key/value: OCP FP8 E4M3 code x a per-layer scale */
} pa_dtype;

/* Geometry of one KV pool.  The pool holds num_layers independent layers of
 * num_blocks physical blocks each; one block holds block_size tokens of every
 * KV head.  Page size per block per layer is block_size x num_kv_heads x
 * (2 x head_dim) x bytes per value ("vLLM Architecture and Installation",
 * Example 6): 65,536 B for block_size 16, 8 KV heads, head_dim 128 and F16
 * values; half that for FP8. */
typedef struct {
    int32_t num_layers;
    int32_t num_blocks;   /* per layer */
    int32_t block_size;   /* tokens per block; must be 16 */
    int32_t num_kv_heads;
    int32_t head_dim;     /* must be 128 */
    int32_t dtype;        /* a pa_dtype: PA_F16 or PA_FP8_E4M3 */
} pa_pool_desc;

/* Opaque host-side handle. */
typedef struct pa_pool pa_pool;

/* Bytes of ONE of the two pool buffers (K or V):
 * num_layers * num_blocks * block_size * num_kv_heads * head_dim * element
 * size (2 for PA_F16, 1 for PA_FP8_E4M3: an FP8 cache halves the page,
 * "vLLM Architecture and Installation", Example 6).
 * Both buffers have this size; 256-byte alignment is required.  Device layout
 * of each buffer (row-major; F16 values or FP8 codes):
 *     [num_layers][num_blocks][num_kv_heads][block_size][head_dim]
 * so the block_size x head_dim tile of one (block, KV head) is contiguous
 * (4 KiB F16, 2 KiB FP8 for the supported geometry).  Returns 0 for a null
 * or invalid desc. */
size_t pa_pool_bytes(const pa_pool_desc *desc);

/* Wraps two caller-allocated device buffers of pa_pool_bytes(desc) bytes each
 * into a handle.  Writes *out only on PA_OK.  Touches no device memory. */
pa_status pa_pool_create(const pa_pool_desc *desc, void *k_pool_dev, void *v_pool_dev,
                         pa_pool **out);

/* Per-layer scales of an FP8 pool (default 1).  An FP8 key/value cache
 * stores one byte per value, which halves the block size and doubles the
 * token capacity (vLLM architecture page, Example 6, the FP8 lever; the
 * batching-and-scheduling page repeats the 1 MiB FP8 block for the 8B
 * shape).  The pages fix neither the 8-bit format nor the scaling: this
 * library reads them as OCP E4M3 with one scale per layer for keys and one
 * for values.  A stored code c means
 * value(c) * k_scale (keys) or * v_scale (values).  pa_write_kv and the
 * appending decode store c = E4M3 round-to-nearest-even of fl32(x *
 * fl32(1/scale)), clamped to +-448 (the format has no infinities; NaN stays
 * NaN).  Scales must be finite and > 0; they are read when later calls are
 * enqueued.  For F16 pools they are stored and ignored. */
pa_status pa_pool_set_scales(pa_pool *pool, int32_t layer, float k_scale, float v_scale);

/* Frees the handle (host memory only); never frees the device buffers.
 * A null pool is accepted and ignored. */
pa_status pa_pool_destroy(pa_pool *pool);

/* Scatters n_tokens new keys and values into the pool of one layer:
 * token i goes to slot slot_mapping_dev[i], i.e. block slot / block_size,
 * offset slot % block_size ("vLLM Architecture and Installation", Example 3).
 *   k_new_dev, v_new_dev: F16 [n_tokens][num_kv_heads][head_dim] (an FP8 pool
 *                         stores their codes, see pa_pool_set_scales)
 *   slot_mapping_dev:     int32 [n_tokens]; a negative slot skips that token,
 *                         a slot >= num_blocks * block_size is skipped too.
 * n_tokens == 0 is a no-op.  Two tokens with the same slot race. */
pa_status pa_write_kv(pa_pool *pool, int32_t layer, const void *k_new_dev, const void *v_new_dev,
                      const int32_t *slot_mapping_dev, int32_t n_tokens, hipStream_t stream);

/* Length in tokens of one context split of pa_decode for this launch shape
 * (a multiple of block_size; a sequence of ctx tokens is handled by
 * ceil(ctx / split) work-groups per KV head).  Returns 0 on invalid input.
 * Splits are 256 to 4096 tokens long.  The environment variable
 * PA_SPLIT_TOKENS, when set to a multiple of 64 in [64, 4096], overrides the
 * choice (tuning only). */
int32_t pa_decode_split_tokens(const pa_pool *pool, int32_t batch, int32_t num_q_heads,
                               int32_t max_context_len);

/* Bytes of device workspace pa_decode needs for this launch shape (0 when a
 * single split covers max_context_len).  Returns 0 on invalid input too;
 * pa_decode then reports the error. */
size_t pa_decode_workspace_bytes(const pa_pool *pool, int32_t batch, int32_t num_q_heads,
                                 int32_t max_context_len);

/* One decode step of attention for one layer (see the formula at the top).
 *   q_dev:            F16 [batch][num_q_heads][head_dim]
 *   out_dev:          F16 [batch][num_q_heads][head_dim]
 *   block_tables_dev: int32 [batch][max_blocks_per_seq]; only the first
 *                     ceil(ctx/block_size) entries of a row are read
 *   context_lens_dev: int32 [batch]
 *   max_context_len:  host-side upper bound of context_lens (sizes the grid);
 *                     must be <= max_blocks_per_seq * block_size; tokens past
 *                     it are ignored
 *   scale:            logit scale, normally 1/sqrt(head_dim)
 *   workspace_dev:    >= pa_decode_workspace_bytes(...) bytes, 256-byte
 *                     aligned; may be null when that size is 0
 * batch == 0 is a no-op.  Equivalent to pa_decode_partial followed by
 * pa_decode_merge with the same arguments. */
pa_status pa_decode(pa_pool *pool, int32_t layer, const void *q_dev, void *out_dev,
                    const int32_t *block_tables_dev, int32_t max_blocks_per_seq,
                    const int32_t *context_lens_dev, int32_t batch, int32_t num_q_heads,
                    int32_t max_context_len, float scale, void *workspace_dev,
                    size_t workspace_bytes, hipStream_t stream);

/* One decode step of one layer that also stores this step's token: for each
 * sequence s with ctx = context_lens[s] >= 1, the K and V of its newest
 * position ctx - 1 are written to the slot its table gives for that position
 * (table[(ctx-1) / block_size] * block_size + (ctx-1) % block_size), and
 * attention then runs over positions [0, ctx) exactly as pa_decode does.
 * The result equals pa_write_kv of those slots followed by pa_decode, in one
 * launch fewer: the new values are used from registers, and the pool write
 * only serves later calls.  On the pages the attention kernel does both jobs
 * in one step: it stores the step's keys and values in their slots and reads
 * the earlier ones through the block table ("vLLM Architecture and
 * Installation", Example 3).
 *   k_new_dev, v_new_dev: F16 [batch][num_kv_heads][head_dim], 16-byte aligned
 * Other arguments as pa_decode.  The newest position's block must not be
 * shared with a sequence that is decoded concurrently. */
pa_status pa_append_decode(pa_pool *pool, int32_t layer, const void *q_dev, const void *k_new_dev,
                           const void *v_new_dev, void *out_dev, const int32_t *block_tables_dev,
                           int32_t max_blocks_per_seq, const int32_t *context_lens_dev, int32_t batch,
                           int32_t num_q_heads, int32_t max_context_len, float scale,
                           void *workspace_dev, size_t workspace_bytes, hipStream_t stream);

/* First phase of pa_decode (k_new_dev = v_new_dev = NULL) or of
 * pa_append_decode (both non-null): one work-group per (sequence, KV head,
 * context split) attends to its split and writes the unnormalised partial
 * output, running max and running sum (fp32) into the workspace.  When a
 * single split covers max_context_len it writes the final F16 output instead
 * and pa_decode_merge has nothing to do. */
pa_status pa_decode_partial(pa_pool *pool, int32_t layer, const void *q_dev, const void *k_new_dev,
                            const void *v_new_dev, void *out_dev, const int32_t *block_tables_dev,
                            int32_t max_blocks_per_seq, const int32_t *context_lens_dev, int32_t batch,
                            int32_t num_q_heads, int32_t max_context_len, float scale,
                            void *workspace_dev, size_t workspace_bytes, hipStream_t stream);

/* Second phase of pa_decode: merges the per-split partials of every
 * (sequence, query head) by their log-sum-exp weights, divides by the merged
 * sum and writes the F16 output.  Takes the same launch shape as the
 * pa_decode_partial call whose workspace it reads. */
pa_status pa_decode_merge(pa_pool *pool, void *out_dev, const int32_t *context_lens_dev,
                          int32_t batch, int32_t num_q_heads, int32_t max_context_len,
                          const void *workspace_dev, size_t workspace_bytes, hipStream_t stream);

/* ---- Planned decode: the schedule is built on the host ----------------
 * An engine's scheduler keeps every request's length on the host (the pages'
 * block-table program tracks `lengths` next to the tables: "vLLM
 * Architecture and Installation", Example 3).  From those lengths
 * pa_decode_plan cuts each sequence's context into pieces so that about 256
 * work-groups (one per MI355X compute unit) do near-equal work, orders the
 * pieces longest first, and lists the sequences that were cut (only those are
 * merged).  One plan serves every layer of a step.  For a batch of equal
 * lengths the plan is one piece per sequence and no merge. */
typedef struct {
    int32_t batch;
    int32_t num_q_heads;
    int32_t max_context_len;  /* largest context in the plan */
    int32_t num_items;        /* pieces (work-groups per KV head) */
    int32_t num_merges;       /* sequences cut into more than one piece */
    int32_t num_slots;        /* partial records per query head */
    int32_t max_piece_tokens; /* longest piece */
    int32_t num_prefix_items; /* shared-prefix pieces (pa_cascade_plan) */
    int32_t num_members;      /* member entries of the shared-prefix pieces */
    int32_t shared_newest;    /* members whose newest token lies in the shared prefix */
    int32_t num_prefill_items; /* chunked-prefill pieces (pa_prefill_plan) */
    int32_t num_q_rows;       /* rows of q and out: batch, or the step's query tokens */
    int32_t mixed_decode_waves; /* pa_prefill_plan with both kinds of pieces: waves per
                                   work-group that walk a decode piece (2 when the prompt
                                   tiles are the longer part, so they progress beside the
                                   decode streams; else 4); 4 in every other plan */
    int32_t decode_wave_heads; /* pa_decode_plan: 1 when its pieces are at most 1024
                                  tokens and the plan's dispatch model rates it faster
                                  for each of a work-group's four waves to take its own
                                  KV head and walk the whole piece, else 0.  The caller may
                                  clear or set it before pa_decode_run; it is ignored
                                  unless num_kv_heads is a multiple of 4 and
                                  max_piece_tokens <= 1024, and in every other plan. */
    size_t plan_bytes;        /* bytes of the serialised plan */
    size_t workspace_bytes;   /* device workspace pa_decode_run needs (0: none) */
} pa_plan_info;

/* Builds the schedule for host-side context lengths (int32 [batch], >= 0).
 * Always fills *info.  With plan_host == NULL it only sizes the plan; else it
 * writes info->plan_bytes bytes into plan_host (PA_ERR_WORKSPACE if
 * plan_host_bytes is smaller).  The caller copies those bytes to a 16-byte
 * aligned device buffer for pa_decode_run.  Host-only: enqueues nothing. */
pa_status pa_decode_plan(const pa_pool *pool, const int32_t *context_lens_host, int32_t batch,
                         int32_t num_q_heads, void *plan_host, size_t plan_host_bytes,
                         pa_plan_info *info);

/* Shared-prefix (cascade) schedule.  Sequences may be grouped: member s of
 * group G = prefix_group_host[s] (-1: none) shares the physical blocks of its
 * first prefix_len_host[G] tokens (a multiple of block_size, at most its
 * context) with every other member -- their table rows hold the same ids
 * there, as reference-counted prefix blocks do ("Reading Inference Engine
 * Codebases", Examples 3 and 12).  The prefix is then read once per group of
 * up to 16 members instead of once per member: its tiles feed the members'
 * stacked query heads (16 x 4 = 64 rows per KV head) through MFMA, and each
 * member's prefix and suffix results are merged by their log-sum-exp weights.
 * The result is the same attention as pa_decode_plan's.  The block ids of a
 * group's prefix are read from its first member's table row.  Other arguments
 * and the two-call sizing as pa_decode_plan. */
pa_status pa_cascade_plan(const pa_pool *pool, const int32_t *context_lens_host, int32_t batch,
                          const int32_t *prefix_group_host, const int32_t *prefix_len_host,
                          int32_t num_groups, int32_t num_q_heads, void *plan_host,
                          size_t plan_host_bytes, pa_plan_info *info);

/* One decode step of one layer on a planned schedule: the plan's pieces, then
 * the merge of the cut sequences.  k_new_dev/v_new_dev (both or neither)
 * append the newest token as pa_append_decode does (rejected with
 * PA_ERR_INVALID_ARG when info->shared_newest > 0: that token would land in
 * a shared block).  q, out, tables, scale and
 * stream as pa_decode; the context lengths come from the plan.
 *   info:           the pa_plan_info the plan builder filled in; its counts
 *                   must give exactly info->plan_bytes (else
 *                   PA_ERR_INVALID_ARG)
 *   plan_dev:       16-byte aligned device copy of the plan's bytes; it must
 *                   stay unchanged until the work completes
 *   plan_dev_bytes: size of the buffer at plan_dev; PA_ERR_WORKSPACE when it
 *                   is smaller than info->plan_bytes
 * A plan whose device bytes were damaged cannot make the kernels access
 * memory outside the given buffers (every entry is clamped), but its results
 * are unspecified. */
pa_status pa_decode_run(pa_pool *pool, int32_t layer, const pa_plan_info *info,
                        const void *plan_dev, size_t plan_dev_bytes, const void *q_dev,
                        const void *k_new_dev, const void *v_new_dev, void *out_dev,
                        const int32_t *block_tables_dev, int32_t max_blocks_per_seq, float scale,
                        void *workspace_dev, size_t workspace_bytes, hipStream_t stream);

/* ---- Chunked prefill / mixed step -------------------------------------
 * A step gives every scheduled request some number of new tokens under a
 * token budget: one for a decoding request, a chunk of its prompt for a
 * prefilling one, with no separate prefill and decode phases ("Batching and
 * Scheduling", Example 5; "vLLM Architecture and Installation", Example 5).
 * Sequence s brings q_len_s = query_start[s+1] - query_start[s] new tokens
 * (>= 0), whose keys and values are already stored in their slots
 * (pa_write_kv), and has seq_len_s >= q_len_s tokens in the cache in all.
 * Its query rows are q rows query_start[s] .. query_start[s+1]-1, packed in
 * sequence order ([num_q_rows][num_q_heads][head_dim] F16, num_q_rows =
 * query_start[batch]); query j of the chunk sits at position
 * p = seq_len_s - q_len_s + j and attends to positions 0 .. p of its own
 * sequence (causal attention through the block table).  Output rows match
 * the query rows.
 *
 * pa_prefill_plan builds the schedule on the host from query_start_host
 * (int32 [batch + 1], query_start_host[0] == 0, nondecreasing) and
 * seq_lens_host (int32 [batch]): one-token rows become decode pieces as in
 * pa_decode_plan; longer chunks are cut into tiles of 32 query tokens whose
 * causal key ranges are cut into near-equal pieces for the matrix-core
 * prefill kernel; rows cut into several pieces are merged.  Sizing, the
 * two-call protocol and the device copy as pa_decode_plan. */
pa_status pa_prefill_plan(const pa_pool *pool, const int32_t *query_start_host,
                          const int32_t *seq_lens_host, int32_t batch, int32_t num_q_heads,
                          void *plan_host, size_t plan_host_bytes, pa_plan_info *info);

/* One layer of a chunked-prefill / mixed step on a pa_prefill_plan schedule.
 * q_dev and out_dev hold info->num_q_rows packed rows (F16, for F16 and FP8
 * pools alike).  The plan (info, plan_dev, plan_dev_bytes), tables, scale,
 * workspace and stream as pa_decode_run. */
pa_status pa_prefill_run(pa_pool *pool, int32_t layer, const pa_plan_info *info,
                         const void *plan_dev, size_t plan_dev_bytes, const void *q_dev,
                         void *out_dev, const int32_t *block_tables_dev, int32_t max_blocks_per_seq,
                         float scale, void *workspace_dev, size_t workspace_bytes,
                         hipStream_t stream);

/* pa_decode without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments and result as pa_decode.  When the split
 * plan needs a workspace (pa_decode_workspace_bytes > 0) the partials go to
 * one fixed array of 32 MiB that the library keeps in each GPU's memory until
 * the process ends; a launch shape that would need more returns
 * PA_ERR_WORKSPACE.  The call itself allocates nothing: the array's address is
 * looked up once per device, on the first call on that device (the device of
 * `stream`).  Every call on one GPU shares that GPU's array, which keeps the
 * last call's partials (nothing in it has to start at zero: each call writes
 * every record it reads), so calls that overlap in time on one GPU -- on
 * different streams, or from different threads -- race and must be ordered
 * by the caller. */
pa_status pa_decode_noalloc(pa_pool *pool, int32_t layer, const void *q_dev, void *out_dev,
                            const int32_t *block_tables_dev, int32_t max_blocks_per_seq,
                            const int32_t *context_lens_dev, int32_t batch, int32_t num_q_heads,
                            int32_t max_context_len, float scale, hipStream_t stream);

/* Static English text for a status code. */
const char *pa_status_string(pa_status status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
