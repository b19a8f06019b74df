// pa_internal.h -- shared between the C-ABI layer (pa_api.cpp) and the HIP
// kernels (pa_kernels.hip).  Not installed; callers use include/pa.h.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace pa {

// Geometry this build's kernels are written for.
constexpr int kHeadDim = 128;     // elements per head
constexpr int kBlockSize = 16;    // tokens per block
constexpr int kGroup = 4;         // query heads per KV head
constexpr int kWaves = 4;         // waves per work-group of the split kernel
constexpr int kSplitQuantum = kWaves * kBlockSize;  // split lengths are multiples of this
constexpr int kMaxSplitTokens = kWaves * 64 * kBlockSize;  // a wave owns at most 64 blocks
constexpr int kMaxContextTokens = 1 << 30;  // longest context: token and block arithmetic stays in int32

// Device layout of one pool buffer (K or V), F16, row-major:
//   [num_layers][num_blocks][num_kv_heads][kBlockSize][kHeadDim]
// One (block, KV head) tile of kBlockSize x kHeadDim is contiguous.
// Elements are F16 (2 bytes) or FP8 E4M3 codes (1 byte).
__host__ __device__ inline size_t tile_elems() { return static_cast<size_t>(kBlockSize) * kHeadDim; }
__host__ __device__ inline size_t layer_bytes(int32_t num_blocks, int32_t num_kv_heads, int32_t elem_bytes) {
    return static_cast<size_t>(num_blocks) * num_kv_heads * tile_elems() * elem_bytes;
}

struct WriteKvArgs {
    char *k_layer;                // this layer's K base (bytes)
    char *v_layer;                // this layer's V base (bytes)
    int32_t elem_bytes;           // 2: F16 pool, 1: FP8 E4M3 pool
    float inv_k_scale;            // FP8: stored code = e4m3(x * inv_scale)
    float inv_v_scale;
    const uint16_t *k_new;        // [n_tokens][num_kv_heads][kHeadDim]
    const uint16_t *v_new;
    const int32_t *slot_mapping;  // [n_tokens]
    int32_t n_tokens;
    int32_t num_kv_heads;
    int64_t num_slots;            // num_blocks * kBlockSize
};

struct DecodeArgs {
    const char *k_layer;          // this layer's K base (bytes)
    const char *v_layer;          // this layer's V base (bytes)
    int32_t elem_bytes;           // 2: F16 pool, 1: FP8 E4M3 pool
    float v_scale;                // FP8: value = code * scale (K's scale is folded into scale_log2e)
    float inv_k_scale;
    float inv_v_scale;
    const uint16_t *q;            // [batch][num_q_heads][kHeadDim]
    const uint16_t *k_new;        // [batch][num_kv_heads][kHeadDim] newest token's K, or null
    const uint16_t *v_new;        // [batch][num_kv_heads][kHeadDim] newest token's V, or null
    const int32_t *tables;        // [batch][max_blocks]
    const int32_t *ctx_lens;      // [batch]
    uint16_t *out;                // [batch][num_q_heads][kHeadDim] (single-split launches)
    float *o_part;                // [batch][num_q_heads][max_splits][kHeadDim]
    float *ml_part;               // [batch][num_q_heads][max_splits][2]: running max (log2 units), sum
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_blocks;
    int32_t max_blocks;           // table row length
    int32_t max_ctx;              // host bound on context lengths
    int32_t split_tokens;         // multiple of kSplitQuantum
    int32_t max_splits;           // ceil(max_ctx / split_tokens)
    float scale_log2e;            // scale * log2(e)
    // Host-planned schedule (null for the fixed-split grid): items of 8 int32
    // {seq, t_begin, t_end, ctx, slot (-1: direct output), 0, 0, 0} and merges
    // of 4 int32 {seq, first slot, pieces, 0}; partial record of query head h
    // of a piece = slot * num_q_heads + h.
    const int32_t *items;
    const int32_t *merges;
    int32_t num_items;
    int32_t num_merges;
    int32_t num_slots;
    // Shared-prefix (cascade) pieces: 8 int32 {first member's seq, t_begin,
    // t_end, members (<= kMaxMembers), offset into the member list, 0, 0, 0};
    // member entries of 2 int32 {seq, slot}.
    const int32_t *prefix_items;
    const int32_t *members;
    int32_t num_prefix_items;
    int32_t num_members;
    // chunked-prefill pieces (prefill_kernel) and the packed query rows
    const int32_t *prefill_items;
    int32_t num_prefill_items;
    int32_t num_q_rows;  // rows of q / out: batch for a decode step, total query tokens for a mixed one
    // waves of a work-group that walk a decode piece in a mixed launch (2 or 4)
    int32_t mixed_decode_waves;
    // decode launches: 1 = four KV heads per work-group, one per wave, each
    // wave walking its head's whole piece (short pieces; Hkv a multiple of 4)
    int32_t decode_wave_heads;
};

// Serialised host plan: a header of kPlanHeader int32, then the decode items,
// the merges, the shared-prefix items, their members and the prefill items.
//   decode item  {s, t_begin, t_end, ctx, record slot or -1, q/out row, 0, 0}
//   merge        {s, first record slot, records, out row}
//   prefill item {s, first q/out row, query tokens (<= kPrefillTile), position
//                 of the first, key begin, key end, record base or -1,
//                 pieces of the tile, this piece, 0, 0, 0}
constexpr int kPlanHeader = 8;
constexpr int kItemInts = 8;
constexpr int kMergeInts = 4;
constexpr int kPrefillItemInts = 12;
constexpr int kPrefillTile = 32;             // query tokens per prefill work-group (16 per wave pair)
// Key blocks per prefill piece (the piece's table row is staged in LDS, 6 KiB).
// A 16,352-token chunk at position 16,352 has tiles of 1,022-2,044 blocks: cut
// into pieces of at most 256 blocks they wrote 1.8 GB of fp32 partial records
// per layer and the merge launch took 0.48 ms.  At most 1,024 blocks (0.5 GB)
// the chunk took 6.28-6.36 ms per layer, at most 1,536 (0.3 GB, the longer
// half of the tiles cut in two) 6.10 ms.
constexpr int kMaxPrefillPieceBlocks = 1536;
constexpr int kPrefixItemInts = 8;
constexpr int kMemberInts = 2;
constexpr int kMaxMembers = 16;        // 16 members x 4 query heads = 64 stacked rows
constexpr int kMaxPrefixPieceBlocks = 32;
constexpr int32_t kPlanMagic = 0x50414e31;  // "PAN1"


// The allocation-free decode (pa_decode_noalloc) keeps its split partials in
// one fixed device array of this many bytes per GPU.
constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;

// Device address of that array on the GPU that `stream` belongs to, looked
// up once per device (hipGetSymbolAddress) and kept.
hipError_t noalloc_scratch(hipStream_t stream, void **ptr);

hipError_t launch_write_kv(const WriteKvArgs &a, hipStream_t stream);
hipError_t launch_decode_partial(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_merge_planned(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_prefix(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_cascade(const DecodeArgs &a, hipStream_t stream);  // decode + shared-prefix pieces
hipError_t launch_prefill(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_mixed(const DecodeArgs &a, hipStream_t stream);  // decode + prefill pieces (F16)

}  // namespace pa
