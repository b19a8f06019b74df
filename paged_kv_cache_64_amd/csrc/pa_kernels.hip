// pa_kernels.hip -- HIP kernels of paged attention on gfx950 (CDNA4, wave64).
//
//   write_kv_kernel        scatter new K/V rows into pool slots (F16, or
//                          FP8 codes) ("vLLM Architecture and Installation",
//                          Example 3: slot = table[p / B] * B + p % B,
//                          computed by the caller and passed in as
//                          slot_mapping)
//   decode_partial_kernel  one work-group per (decode piece, KV head):
//                          gathers the piece's K/V tiles through the block
//                          table and runs an online, max-shifted softmax
//                          ("Reading Inference Engine Codebases", Example 6)
//                          for the four query heads that share the KV head
//   decode_merge_kernel,   merge per-piece partials by their log-sum-exp
//   decode_merge_planned_kernel   weights and write F16
//   decode_prefix_kernel   shared-prefix pieces: one read of a group's
//                          prefix tiles serves every member (MFMA)
//   prefill_dma_kernel,    chunked-prefill tiles of 32 query tokens, causal,
//   prefill_kernel         on the matrix cores ("Batching and Scheduling",
//                          Example 5); F16 pools copy K/V tiles straight
//                          into LDS, FP8 pools widen them through registers
//   mixed_kernel           decode and prefill pieces of one step in one
//                          launch
//   cascade_kernel         decode and shared-prefix pieces of one step in one
//                          launch
//
// A decode step is bound by HBM bandwidth: every sequence reads its own K/V
// once per step and nothing is shared between sequences ("Batching and
// Scheduling", Example 1), at about 4 flop per byte.  There what matters is
// keeping 16-byte loads in flight and the per-byte instruction count low;
// the dense tiles of shared prefixes and prompt chunks go to MFMA.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
// Raw tile data in native vectors (HIP's uint4/uint2 are classes, and arrays
// of them are not promoted to registers).
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((ext_vector_type(4)));

// Online-softmax bookkeeping: the running max m is only raised when a score
// exceeds it by more than kTau (log2 units), so most blocks skip the
// cross-lane max and the accumulator rescale.  Every weight is then at most
// 2^kTau, far from fp32 overflow, and the final division by the sum removes
// the common factor exactly.
constexpr float kTau = 8.0f;

__device__ __forceinline__ float shfl_xor(float v, int mask) {
    const int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

// Orders this wave's LDS traffic: stores issued before are visible to loads
// issued after, for every lane of the wave.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Buffer resource over one K or V tile (gfx9-family dword3).  A resource with
// zero records turns every load through it into a zero fill that moves no
// data, which lets the pipelined loop below issue loads unconditionally.
constexpr int kRsrcDword3 = 0x00020000;
// Cache-policy bits of the K/V loads.  Every K/V byte is read exactly once
// per step, so the loads are marked non-temporal (the nt bit, 2): measured
// 12 % faster than the default policy on the 32-layer batch-32 step.
#ifndef PA_KV_LOAD_AUX
#define PA_KV_LOAD_AUX 2
#endif
// Register buffers of the shared-prefix pipeline (each wave reads every
// block of its piece).
#ifndef PA_PREFIX_NBUF
#define PA_PREFIX_NBUF 2
#endif
// Register buffers of the decode pipeline (blocks in flight per wave).  F16
// at 2 / 3 / 4: 81.3 / 81.7 / 81.8 us per launch on the 32-layer batch-32
// step, but depth 2 (158 VGPRs, three waves per SIMD) took the ragged
// 64-sequence step from 184 to 191 us and the shared-prefix step from 580 to
// 595 us, so 3 is kept.
#ifndef PA_DECODE_NBUF
#define PA_DECODE_NBUF 3
#endif
// FP8 pools (tiles half the size): 2 / 3 / 4 / 5 measured 44.9 / 44.8 / 45.0
// / 45.4 us.
#ifndef PA_DECODE_NBUF_FP8
#define PA_DECODE_NBUF_FP8 3
#endif
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char *tile, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(tile), static_cast<short>(0), bytes, kRsrcDword3);
}
__device__ __forceinline__ u4 load_raw16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, PA_KV_LOAD_AUX));
}
// Tiles that are read more than once keep the default cache policy:
//  - shared-prefix pieces (every wave of the work-group reads each tile for
//    its own rows): with the streaming hint, lines left before the other waves
//    read them, and the prefix kernel fetched 1.28x its bytes (67.6 us per
//    layer on the 256-sequence shared-prefix step, against 50.3 us and 1.00x);
//  - prefill copies (every 32-token query tile of a prompt reads the same
//    keys): the 16,352-token chunk took 9.24 ms per layer with the hint and
//    7.78 ms without.
__device__ __forceinline__ h8 load_shared16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}
__device__ __forceinline__ u2 load_shared8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, 0));
}
__device__ __forceinline__ u2 load_raw8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, PA_KV_LOAD_AUX));
}

// ---- FP8 (OCP E4M3 on gfx950) storage --------------------------------------
// Codes are written as round-to-nearest-even of fl32(x * inv_scale) after a
// clamp to +-448 (the format has no infinities); NaN stays NaN.  Every code
// is exactly representable in F16 and fp32.
__device__ __forceinline__ float fp8_clamp(float x) {
    return __builtin_isnan(x) ? x : __builtin_amdgcn_fmed3f(x, 448.0f, -448.0f);
}
__device__ __forceinline__ uint32_t fp8_encode4(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(a), fp8_clamp(b), 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_clamp(c), fp8_clamp(d), r, true);
    return static_cast<uint32_t>(r);
}
// 8 F16 values -> 8 codes
__device__ __forceinline__ u2 fp8_encode8(h8 x, float inv) {
    u2 r;
    r.x = fp8_encode4(static_cast<float>(x[0]) * inv, static_cast<float>(x[1]) * inv, static_cast<float>(x[2]) * inv,
                      static_cast<float>(x[3]) * inv);
    r.y = fp8_encode4(static_cast<float>(x[4]) * inv, static_cast<float>(x[5]) * inv, static_cast<float>(x[6]) * inv,
                      static_cast<float>(x[7]) * inv);
    return r;
}
// Codes 0,1 (HI = false) or 2,3 (HI = true) of a word -> two F16 values.
// Every E4M3 value is exact in F16; at scale 1 the conversion is exact.
template <bool HI>
__device__ __forceinline__ h2 fp8_pair_f16(uint32_t word) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(word), 1.0f, HI);
}
// 8 codes (2 words) -> 8 F16 values in order
__device__ __forceinline__ h8 fp8_decode8_h(uint32_t w0, uint32_t w1) {
    const h2 a = fp8_pair_f16<false>(w0), b = fp8_pair_f16<true>(w0);
    const h2 c = fp8_pair_f16<false>(w1), d = fp8_pair_f16<true>(w1);
    return h8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ int clamp_ctx(int ctx, int max_ctx, int max_blocks) {
    ctx = ctx < 0 ? 0 : ctx;
    ctx = ctx > max_ctx ? max_ctx : ctx;
    const int cap = max_blocks * kBlockSize;
    return ctx > cap ? cap : ctx;
}

// ---------------------------------------------------------------------------
// write_kv: one thread per 16-byte chunk of a (token, KV head) row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void write_kv_kernel(WriteKvArgs a) {
    constexpr int kChunks = kHeadDim / 8;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t total = static_cast<int64_t>(a.n_tokens) * a.num_kv_heads * kChunks;
    if (idx >= total) return;
    const int chunk = static_cast<int>(idx % kChunks);
    const int64_t row = idx / kChunks;  // token * num_kv_heads + head
    const int head = static_cast<int>(row % a.num_kv_heads);
    const int64_t token = row / a.num_kv_heads;
    const int64_t slot = a.slot_mapping[token];
    if (slot < 0 || slot >= a.num_slots) return;
    const int64_t blk = slot / kBlockSize;
    const int64_t off = slot % kBlockSize;
    const int64_t dst = ((blk * a.num_kv_heads + head) * kBlockSize + off) * kHeadDim + chunk * 8;  // elements
    const int64_t src = row * kHeadDim + chunk * 8;
    if (a.elem_bytes == 1) {
        const h8 kx = *reinterpret_cast<const h8 *>(a.k_new + src);
        const h8 vx = *reinterpret_cast<const h8 *>(a.v_new + src);
        *reinterpret_cast<u2 *>(a.k_layer + dst) = fp8_encode8(kx, a.inv_k_scale);
        *reinterpret_cast<u2 *>(a.v_layer + dst) = fp8_encode8(vx, a.inv_v_scale);
    } else {
        *reinterpret_cast<uint4 *>(a.k_layer + 2 * dst) = *reinterpret_cast<const uint4 *>(a.k_new + src);
        *reinterpret_cast<uint4 *>(a.v_layer + 2 * dst) = *reinterpret_cast<const uint4 *>(a.v_new + src);
    }
}

// ---------------------------------------------------------------------------
// decode_partial: grid (split, KV head, sequence), 256 threads = 4 waves.
//
// Each wave walks its own contiguous run of the split's blocks and keeps its
// own running max, sum and output accumulator; the four waves are merged
// through LDS at the end.  A block is 16 tokens x 128 dims of one KV head:
// 4 KiB of K and 4 KiB of V (2 KiB each for FP8 codes).  With lane
// l = 16r + n (r = l/16, n = l%16), per block:
//
//   S^T = K Q^T   four v_mfma_f32_16x16x32_f16, 32 dims each:
//                 A = K: lane l holds MFMA row n, which is token
//                     4(n%4) + n/4 (the 4x4 transpose of the token index),
//                     at 8 dims per MFMA -- F16 pools: dims 32i + 8r .. +7
//                     of 16-byte load i < 4; FP8 pools: dims 64i + 16r .. +15
//                     of 16-byte load i < 2, widened to F16 (exact).  Each
//                     load instruction covers 64 contiguous bytes of each of
//                     16 token rows.
//                 B = Q^T: column n is query head n%4 of the group (columns
//                     4..15 repeat heads 0..3) at the same dims.
//                 D: lane l holds the scores of tokens 4c + r, c < 4, for
//                    head n%4.
//   softmax       on those four scores per lane (the lanes of one head hold
//                 equal values), with the lazily raised max; the weights are
//                 rounded to F16 (at most 2^kTau) and the running sum adds
//                 the rounded values.
//   O += P V      eight v_mfma_f32_16x16x16_f16, one per dim 8n + j, j < 8:
//                 A = P: lane l's four weights at k-slots 4r + c = token
//                     4c + r -- the D layout of S^T as it stands;
//                 B = V: load c < 4 of lane l holds token 4c + r, dims
//                     8n .. 8n+7 (each F16 load instruction is 1 KiB
//                     contiguous, each FP8 one 512 B); byte permutes gather
//                     dim 8n + j of the lane's four tokens;
//                 D: result element c of lane l is head c at dim 8n + j.
//   K's FP8 scale is folded into the score scale and V's into the output.
// ---------------------------------------------------------------------------
// MIXED: the decode pieces of a mixed launch, walked by a.mixed_decode_waves
// (2 or 4) of the work-group's waves; a wave then owns up to 128 blocks, its
// table entries in two registers.
// WH: each of the four waves takes its own KV head of the piece and walks all
// of the piece's blocks (at most 64), so no partial sums cross waves; the
// plan asks for this when its pieces are short (a work-group's fixed work is
// then spread over four times the blocks).
template <int NBUF, bool FP8, bool MIXED = false, bool WH = false>
__device__ __forceinline__ void decode_partial_body(const DecodeArgs &a, uint32_t bx, uint32_t by, uint32_t bz) {
    static_assert(!(WH && MIXED), "a mixed launch keeps one KV head per work-group");
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar register
    // Planned launches number work-groups item-major with the KV head fastest,
    // so the heads of one piece -- whose tiles share each 32 KiB block of
    // K and of V -- run side by side, as in the fixed-split grid.
    const int wg_heads = WH ? a.num_kv_heads / kWaves : a.num_kv_heads;  // work-groups per item
    const int g = a.items == nullptr ? static_cast<int>(by)
                  : WH               ? static_cast<int>(bx % wg_heads) * kWaves + w
                                     : static_cast<int>(bx % a.num_kv_heads);
    const int lane = tid & 63;
    const int r = lane >> 4, n = lane & 15;
    const int ktok = 4 * (n & 3) + (n >> 2);  // the token of this lane's MFMA row of K

    __shared__ float m_lds[kWaves][4];
    __shared__ float l_lds[kWaves][4];
    __shared__ float o_lds[kWaves][kGroup][kHeadDim];

    // This work-group's piece of one sequence: tokens [t_begin, t_end) of
    // sequence s (context ctx), and where its result goes -- the final F16
    // output (direct) or partial record rec_base + h * rec_stride of query
    // head h.
    int s, ctx, t_begin, t_end, qrow;  // qrow: this sequence's row of q and out
    bool direct;
    int64_t rec_base, rec_stride;
    if (a.items != nullptr) {
        // Plan entries are clamped so a damaged plan cannot index outside
        // q, out, the tables or the workspace.
        const int32_t *it = a.items + kItemInts * static_cast<size_t>(bx / wg_heads);
        s = min(max(it[0], 0), a.batch - 1);
        qrow = min(max(it[5], 0), a.num_q_rows - 1);
        ctx = min(max(it[3], 0), a.max_blocks * kBlockSize);
        t_begin = max(it[1], 0);
        t_end = min(it[2], ctx);
        const int slot = min(it[4], a.num_slots - 1);
        direct = slot < 0;
        rec_base = static_cast<int64_t>(slot) * a.num_q_heads;
        rec_stride = 1;
    } else {
        const int split = static_cast<int>(bx);
        s = static_cast<int>(bz);
        qrow = s;
        ctx = clamp_ctx(a.ctx_lens[s], a.max_ctx, a.max_blocks);
        t_begin = split * a.split_tokens;
        t_end = min(ctx, t_begin + a.split_tokens);
        direct = a.max_splits == 1;
        rec_base = static_cast<int64_t>(s) * a.num_q_heads * a.max_splits + split;
        rec_stride = a.max_splits;
    }
    const int head0 = g * kGroup;

    if (t_begin >= t_end) {
        // Nothing to attend to.  A direct piece that starts at 0 owns an
        // empty context, whose output row is zero.
        if (direct && t_begin == 0) {
            const int d0 = (tid & 63) * 2;
            if constexpr (WH) {  // the wave's own four heads
#pragma unroll
                for (int h = 0; h < kGroup; ++h) {
                    uint16_t *o = a.out + (static_cast<size_t>(qrow) * a.num_q_heads + head0 + h) * kHeadDim + d0;
                    *reinterpret_cast<uint32_t *>(o) = 0u;
                }
            } else {
                const int h = tid >> 6;
                uint16_t *o = a.out + (static_cast<size_t>(qrow) * a.num_q_heads + head0 + h) * kHeadDim + d0;
                *reinterpret_cast<uint32_t *>(o) = 0u;
            }
        }
        return;
    }
    const int b_begin = t_begin / kBlockSize;
    // A piece never spans more than kMaxSplitTokens / kBlockSize blocks (64 per
    // wave when four walk it, one per lane of a wave's table register); a
    // damaged plan entry is cut there too.
    // (WH: 64 blocks, as each wave walks the whole piece)
    const int b_end = min((t_end + kBlockSize - 1) / kBlockSize, b_begin + (WH ? 64 : kMaxSplitTokens / kBlockSize));
    t_end = min(t_end, b_end * kBlockSize);
    const int nw = MIXED && a.mixed_decode_waves == 2 ? 2 : kWaves;  // waves that walk blocks
    const int per_wave = WH ? b_end - b_begin : (b_end - b_begin + nw - 1) / nw;
    const int wb_begin = WH ? b_begin : w < nw ? min(b_end, b_begin + w * per_wave) : b_end;
    const int wb_end = min(b_end, wb_begin + per_wave);

    // Block-table entries of this wave's blocks are loaded up front, entry
    // wb_begin + i into lane i (a wave never owns more than 64 blocks), and
    // each block's entry is then read with v_readlane: no memory or LDS
    // access has to complete between a block's turn and the issue of its
    // K/V loads.  This load comes first: every K/V address depends on it.
    const int32_t *table = a.tables + static_cast<size_t>(s) * a.max_blocks;
    const int tbl_v = lane < wb_end - wb_begin ? table[wb_begin + lane] : 0;
    const int tbl_v1 = MIXED && lane + 64 < wb_end - wb_begin ? table[wb_begin + 64 + lane] : 0;

    // Q^T operands: qm[i] holds query head l%4 at the 8 dims of MFMA i in this
    // lane, chunk_dim(i) .. +7.
    auto chunk_dim = [&](int i) { return FP8 ? 64 * (i >> 1) + 16 * r + 8 * (i & 1) : 32 * i + 8 * r; };
    h8 qm[4];
    {
        const uint16_t *qh = a.q + (static_cast<size_t>(qrow) * a.num_q_heads + head0 + (lane & 3)) * kHeadDim;
#pragma unroll
        for (int i = 0; i < 4; ++i) qm[i] = *reinterpret_cast<const h8 *>(qh + chunk_dim(i));
    }

    // The newest token (position ctx-1) when this call also appends it: the
    // work-group whose split holds it stores its K/V row into the pool (for
    // later steps) and uses the new values straight from registers, so no
    // load in this launch depends on that store.  The values are loaded here
    // (F16, in this lane's K and V layout), encoded where they are used, and
    // the row is stored after the loop, so nothing waits for them before the
    // first K/V loads are issued.
    const int new_tok = ctx - 1;
    const bool owns_new = a.k_new != nullptr && new_tok >= t_begin && new_tok < t_end;
    const int new_blk = new_tok / kBlockSize;
    const int new_off = new_tok % kBlockSize;
    constexpr int kChunks = FP8 ? 8 : 16;  // 16-byte chunks of a stored K or V row
    const bool stores_new = owns_new && (WH || w == 0) && lane < 2 * kChunks;  // WH: each wave its own head
    u4 kn_raw[4], vn_raw;  // K: dims chunk_dim(i) .. +7; V: dims 8n .. 8n+7
    u4 st_raw[2];          // the stored row's chunk as F16: 16 values (FP8 pools) or 8
    uint32_t new_phys = 0;
    if (owns_new) {
        const size_t row = (static_cast<size_t>(s) * a.num_kv_heads + g) * kHeadDim;
#pragma unroll
        for (int i = 0; i < 4; ++i) kn_raw[i] = *reinterpret_cast<const u4 *>(a.k_new + row + chunk_dim(i));
        vn_raw = *reinterpret_cast<const u4 *>(a.v_new + row + 8 * n);
        if (stores_new) {
            const bool is_k = lane < kChunks;
            const int c = is_k ? lane : lane - kChunks;
            const uint16_t *src = (is_k ? a.k_new : a.v_new) + row + (FP8 ? 16 : 8) * c;
            st_raw[0] = *reinterpret_cast<const u4 *>(src);
            if (FP8) st_raw[1] = *reinterpret_cast<const u4 *>(src + 8);
            new_phys = static_cast<uint32_t>(table[new_blk]);
        }
    }

    const uint32_t last_block = static_cast<uint32_t>(a.num_blocks - 1);
    constexpr int kElem = FP8 ? 1 : 2;
    const size_t tile_bytes = tile_elems() * kElem;
    const char *k_layer = a.k_layer;
    const char *v_layer = a.v_layer;
    // per-lane byte offsets inside a tile
    const uint32_t k_off = static_cast<uint32_t>(ktok * kHeadDim * kElem + 16 * r);  // + 64 i
    const uint32_t v_off = static_cast<uint32_t>(lane * 8 * kElem);                 // + 512 kElem c

    float m_run = -INFINITY;  // running max of head n%4 (log2 units), equal in the lanes of that head
    float l_run = 0.0f;       // sum of this lane's weights (tokens 4c + r) of head n%4
    f4 oacc[8];               // MFMA j's result: oacc[j][c] = head c at dim 8n + j
#pragma unroll
    for (int j = 0; j < 8; ++j) oacc[j] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    // Registers of one block: K as 16-byte loads, V as 16-byte (F16) or
    // 8-byte (FP8) loads.
    constexpr int kKLoads = FP8 ? 2 : 4;
    using VReg = std::conditional_t<FP8, u2, u4>;
    u4 kb[NBUF][kKLoads];  // raw tile data
    VReg vb[NBUF][4];

    // Issues the loads of block b into register buffer buf.  Blocks past
    // the wave's run are issued through empty resources (no memory traffic),
    // so every pipeline step issues the same number of loads.
    auto issue = [&](int buf, int b) {
        const bool live = b < wb_end;
        const int ti = live ? b - wb_begin : 0;
        uint32_t phys = static_cast<uint32_t>(MIXED && ti >= 64 ? __builtin_amdgcn_readlane(tbl_v1, ti - 64)
                                                                : __builtin_amdgcn_readlane(tbl_v, ti));
        phys = phys > last_block ? last_block : phys;
        const size_t base = (static_cast<size_t>(phys) * a.num_kv_heads + g) * tile_bytes;
        const int bytes = live ? static_cast<int>(tile_bytes) : 0;
        // The V resource ends at the piece's last token: value rows past it
        // (slots past the sequence in its last block, which may hold
        // anything) load as zeros, so their zero weights cannot meet a NaN,
        // at no VALU cost.  Keys past it are masked to -inf in consume.
        const int vbytes = live ? min(t_end - b * kBlockSize, kBlockSize) * kHeadDim * kElem : 0;
        const __amdgpu_buffer_rsrc_t kr = tile_rsrc(k_layer + base, bytes);
        const __amdgpu_buffer_rsrc_t vr = tile_rsrc(v_layer + base, vbytes);
#pragma unroll
        for (int i = 0; i < kKLoads; ++i) kb[buf][i] = load_raw16(kr, k_off + 64u * i);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if constexpr (FP8)
                vb[buf][c] = load_raw8(vr, v_off + 512u * c);
            else
                vb[buf][c] = load_raw16(vr, v_off + 1024u * c);
        }
    };

    auto consume = [&](int buf, int b) {
        if (owns_new && b == new_blk) {
            // the pool may still hold the previous content of the newest slot
            u4 kn[kKLoads];
            VReg vn;
            if constexpr (FP8) {
#pragma unroll
                for (int i = 0; i < kKLoads; ++i) {
                    const u2 lo = fp8_encode8(__builtin_bit_cast(h8, kn_raw[2 * i]), a.inv_k_scale);
                    const u2 hi = fp8_encode8(__builtin_bit_cast(h8, kn_raw[2 * i + 1]), a.inv_k_scale);
                    kn[i] = u4{lo.x, lo.y, hi.x, hi.y};
                }
                vn = fp8_encode8(__builtin_bit_cast(h8, vn_raw), a.inv_v_scale);
            } else {
#pragma unroll
                for (int i = 0; i < kKLoads; ++i) kn[i] = kn_raw[i];
                vn = vn_raw;
            }
            const bool k_mine = ktok == new_off;
#pragma unroll
            for (int i = 0; i < kKLoads; ++i) kb[buf][i] = k_mine ? kn[i] : kb[buf][i];
#pragma unroll
            for (int c = 0; c < 4; ++c) vb[buf][c] = (4 * c + r == new_off) ? vn : vb[buf][c];
        }
        // ---- S^T = K Q^T ----
        h8 ka[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (FP8) {
                const u4 k2 = kb[buf][i >> 1];
                ka[i] = (i & 1) ? fp8_decode8_h(k2.z, k2.w) : fp8_decode8_h(k2.x, k2.y);
            } else {
                ka[i] = __builtin_bit_cast(h8, kb[buf][i]);
            }
        }
        f4 st = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) st = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[i], qm[i], st, 0, 0, 0);

        // ---- mask the tail of the sequence's last block ----
        // (its value rows past the end already loaded as zeros, see issue)
        const int valid = t_end - b * kBlockSize;  // >= 1; pieces end on block edges or at ctx
        const bool partial = valid < kBlockSize;
        float x[4];  // scores of tokens 4c + r in log2 units
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            x[c] = st[c] * a.scale_log2e;
            if (partial && 4 * c + r >= valid) x[c] = -INFINITY;
        }

        // ---- online softmax with a lazily raised max ----
        float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        if (__builtin_amdgcn_ballot_w64(bm > m_run + kTau) != 0) {
            bm = fmaxf(bm, shfl_xor(bm, 16));
            bm = fmaxf(bm, shfl_xor(bm, 32));
            const float m_new = fmaxf(m_run, bm);
            const float alpha = fast_exp2(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
            // lanes 0..3 hold heads 0..3, result element c is head c
            const f4 a4 = {__int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 0)),
                           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 1)),
                           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 2)),
                           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), 3))};
#pragma unroll
            for (int j = 0; j < 8; ++j) oacc[j] *= a4;
        }
        const h2 p01 = {static_cast<_Float16>(fast_exp2(x[0] - m_run)), static_cast<_Float16>(fast_exp2(x[1] - m_run))};
        const h2 p23 = {static_cast<_Float16>(fast_exp2(x[2] - m_run)), static_cast<_Float16>(fast_exp2(x[3] - m_run))};
        const h2 one2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
        l_run = __builtin_amdgcn_fdot2(p01, one2, __builtin_amdgcn_fdot2(p23, one2, l_run, false), false);
        const h4 pa = {p01.x, p01.y, p23.x, p23.y};

        // ---- O += P V ----
        if constexpr (FP8) {
            uint32_t vw[4][2];  // codes of token 4c + r (zero past the piece's end)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                vw[c][0] = vb[buf][c].x;
                vw[c][1] = vb[buf][c].y;
            }
#pragma unroll
            for (int jp = 0; jp < 4; ++jp) {
                // bytes {c0 dim j, c1 dim j, c0 dim j+1, c1 dim j+1}, j = 2 jp
                const uint32_t sel = (jp & 1) ? 0x07030602u : 0x05010400u;
                const int wd = jp >> 1;
                const uint32_t t01 = __builtin_amdgcn_perm(vw[1][wd], vw[0][wd], sel);
                const uint32_t t23 = __builtin_amdgcn_perm(vw[3][wd], vw[2][wd], sel);
                const h2 a01 = fp8_pair_f16<false>(t01), b01 = fp8_pair_f16<true>(t01);
                const h2 a23 = fp8_pair_f16<false>(t23), b23 = fp8_pair_f16<true>(t23);
                const h4 v0 = {a01.x, a01.y, a23.x, a23.y};  // dim 8n + 2jp of tokens c = 0..3
                const h4 v1 = {b01.x, b01.y, b23.x, b23.y};  // dim 8n + 2jp + 1
                oacc[2 * jp] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, v0, oacc[2 * jp], 0, 0, 0);
                oacc[2 * jp + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, v1, oacc[2 * jp + 1], 0, 0, 0);
            }
        } else {
            u4 vv[4];  // token 4c + r, dims 8n .. 8n+7 (zero past the piece's end)
#pragma unroll
            for (int c = 0; c < 4; ++c) vv[c] = vb[buf][c];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // half j of tokens c = 0, 1 and of tokens c = 2, 3
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                const int wd = j >> 1;
                const uint32_t t01 = __builtin_amdgcn_perm(vv[1][wd], vv[0][wd], sel);
                const uint32_t t23 = __builtin_amdgcn_perm(vv[3][wd], vv[2][wd], sel);
                oacc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, __builtin_bit_cast(h4, u2{t01, t23}), oacc[j], 0,
                                                                0, 0);
            }
        }
    };

    // Software pipeline over this wave's blocks with NBUF register buffers:
    // block b + NBUF - 1 is issued before block b is consumed.  The prologue
    // keeps its loads in issue order (K then V, block by block) as in the
    // loop: reordered, they left the loop entry with a merged wait count
    // that waited for two blocks where one was due.
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) {
        issue(i, wb_begin + i);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int base = wb_begin; base < wb_end; base += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
            issue((u + NBUF - 1) % NBUF, base + u + NBUF - 1);
            if (base + u < wb_end) consume(u, base + u);
        }
    }

    // ---- store the newest token's K/V row ----
    if (stores_new) {
        const uint32_t phys = new_phys > last_block ? last_block : new_phys;
        const bool is_k = lane < kChunks;
        const int c = is_k ? lane : lane - kChunks;
        const size_t elems = (static_cast<size_t>(phys) * a.num_kv_heads + g) * tile_elems() +
                             static_cast<size_t>(new_off) * kHeadDim;
        char *pool = const_cast<char *>(is_k ? a.k_layer : a.v_layer);
        if constexpr (FP8) {
            const float inv = is_k ? a.inv_k_scale : a.inv_v_scale;
            const u2 lo = fp8_encode8(__builtin_bit_cast(h8, st_raw[0]), inv);
            const u2 hi = fp8_encode8(__builtin_bit_cast(h8, st_raw[1]), inv);
            *reinterpret_cast<u4 *>(pool + elems + 16 * c) = u4{lo.x, lo.y, hi.x, hi.y};
        } else {
            *reinterpret_cast<u4 *>(pool + 2 * elems + 16 * c) = st_raw[0];
        }
    }

    // ---- per-wave totals: sum over the four lane groups r ----
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);
    if (lane < 4) {
        m_lds[w][lane] = m_run;
        l_lds[w][lane] = l_run;
    }
    {
        // every lane group holds all four heads: group r stores head r
        float ov[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ov[j] = r == 0 ? oacc[j][0] : r == 1 ? oacc[j][1] : r == 2 ? oacc[j][2] : oacc[j][3];
        float4 *dst = reinterpret_cast<float4 *>(&o_lds[w][r][8 * n]);
        dst[0] = make_float4(ov[0], ov[1], ov[2], ov[3]);
        dst[1] = make_float4(ov[4], ov[5], ov[6], ov[7]);
    }
    if constexpr (WH) {
        // the wave's own four heads, each finished by this wave alone
        wave_lds_sync();
        const int d0 = lane * 2;
#pragma unroll
        for (int h = 0; h < kGroup; ++h) {
            const float M = m_lds[w][h], L = l_lds[w][h];
            const float2 v = *reinterpret_cast<const float2 *>(&o_lds[w][h][d0]);
            const float O0 = FP8 ? v.x * a.v_scale : v.x, O1 = FP8 ? v.y * a.v_scale : v.y;
            const size_t row = static_cast<size_t>(qrow) * a.num_q_heads + head0 + h;
            if (direct) {
                h2 pr = {static_cast<_Float16>(O0 / L), static_cast<_Float16>(O1 / L)};
                *reinterpret_cast<h2 *>(a.out + row * kHeadDim + d0) = pr;
            } else {
                const size_t slot = static_cast<size_t>(rec_base + static_cast<int64_t>(head0 + h) * rec_stride);
                *reinterpret_cast<float2 *>(a.o_part + slot * kHeadDim + d0) = make_float2(O0, O1);
                if (d0 == 0) *reinterpret_cast<float2 *>(a.ml_part + slot * 2) = make_float2(M, L);
            }
        }
        return;
    }
    __syncthreads();

    // ---- merge the four waves: thread -> (head, 2 dims) ----
    const int h = tid >> 6;
    const int d0 = (tid & 63) * 2;
    float mw[kWaves], M = -INFINITY;
#pragma unroll
    for (int x = 0; x < kWaves; ++x) {
        mw[x] = m_lds[x][h];
        M = fmaxf(M, mw[x]);
    }
    float L = 0.0f, O0 = 0.0f, O1 = 0.0f;
#pragma unroll
    for (int x = 0; x < kWaves; ++x) {
        const float wgt = mw[x] == -INFINITY ? 0.0f : fast_exp2(mw[x] - M);
        const float2 v = *reinterpret_cast<const float2 *>(&o_lds[x][h][d0]);
        L += wgt * l_lds[x][h];
        O0 += wgt * v.x;
        O1 += wgt * v.y;
    }
    if (FP8) {  // V's scale
        O0 *= a.v_scale;
        O1 *= a.v_scale;
    }
    const size_t row = static_cast<size_t>(qrow) * a.num_q_heads + head0 + h;
    if (direct) {
        const _Float16 r0 = static_cast<_Float16>(O0 / L);
        const _Float16 r1 = static_cast<_Float16>(O1 / L);
        h2 pr = {r0, r1};
        *reinterpret_cast<h2 *>(a.out + row * kHeadDim + d0) = pr;
    } else {
        const size_t slot = static_cast<size_t>(rec_base + static_cast<int64_t>(head0 + h) * rec_stride);
        *reinterpret_cast<float2 *>(a.o_part + slot * kHeadDim + d0) = make_float2(O0, O1);
        if (d0 == 0) *reinterpret_cast<float2 *>(a.ml_part + slot * 2) = make_float2(M, L);
    }
}

template <int NBUF, bool FP8>
__global__ __launch_bounds__(256, 2) void decode_partial_kernel(DecodeArgs a) {
    decode_partial_body<NBUF, FP8>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Per-wave KV heads: a wave walks at most 64 blocks, so two blocks in
// flight and three work-groups per CU (157 VGPRs), which overlap one
// another's start and end, beat three blocks at two per CU: 1,024 x 128
// tokens (the newest token appended, cold) 107.3-108.6 -> 104.3-104.6 us
// F16, 60.7-61.9 -> 58.6-59.2 us FP8; 512 x 256 tokens 94.1-94.6 -> 92.0-92.5
// us F16, 52.2-52.7 -> 50.5-51.0 us FP8; 256 x 1,024 tokens unchanged.
template <bool FP8>
__global__ __launch_bounds__(256, 3) void decode_wave_heads_kernel(DecodeArgs a) {
    decode_partial_body<2, FP8, false, true>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Records a merge loads in one round (the merges are latency-bound).
constexpr int kMergeBatch = 8;

// Log-sum-exp merge of n partial records at one output element:
//   M = max_i m_i,  L = sum_i 2^(m_i - M) l_i,  O = sum_i 2^(m_i - M) o_i
// load(i, ml, o) fetches record i's (m, l) and o.  Records come kMergeBatch
// at a time with all their loads in flight together; a later round that
// raises M rescales the running sums once.  For n <= kMergeBatch this is one
// round: M over all records, then the sums in record order.  A record with
// m = -inf (a piece that saw no key) adds nothing.  Returns O / L.
template <class Load>
__device__ __forceinline__ float merge_records(int n, Load load) {
    float M = -INFINITY, L = 0.0f, O = 0.0f;
    for (int i0 = 0; i0 < n; i0 += kMergeBatch) {
        float2 ml[kMergeBatch];
        float o[kMergeBatch];
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i)
            if (i0 + i < n) load(i0 + i, ml[i], o[i]);
        float Mc = M;
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i)
            if (i0 + i < n) Mc = fmaxf(Mc, ml[i].x);
        if (Mc != M) {
            const float sc = M == -INFINITY ? 0.0f : fast_exp2(M - Mc);
            L *= sc;
            O *= sc;
            M = Mc;
        }
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) {
            if (i0 + i < n) {
                const float wgt = ml[i].x == -INFINITY ? 0.0f : fast_exp2(ml[i].x - M);
                L += wgt * ml[i].y;
                O += wgt * o[i];
            }
        }
    }
    return O / L;
}

// ---------------------------------------------------------------------------
// decode_merge: 256 threads = two (sequence, query head) rows of 128 dims;
// merges the row's split records and writes F16.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 2 + (threadIdx.x >> 7);
    const int d = threadIdx.x & 127;
    if (row >= static_cast<int64_t>(a.batch) * a.num_q_heads) return;
    const int s = static_cast<int>(row / a.num_q_heads);
    const int ctx = clamp_ctx(a.ctx_lens[s], a.max_ctx, a.max_blocks);
    const int ns = (ctx + a.split_tokens - 1) / a.split_tokens;
    uint16_t *out = a.out + row * kHeadDim + d;
    if (ns == 0) {
        *out = 0;
        return;
    }
    const float *ml = a.ml_part + row * a.max_splits * 2;
    const float *op = a.o_part + row * a.max_splits * kHeadDim + d;
    const float r = merge_records(ns, [&](int i, float2 &mlv, float &ov) {
        mlv = *reinterpret_cast<const float2 *>(ml + 2 * i);
        ov = op[static_cast<int64_t>(i) * kHeadDim];
    });
    *reinterpret_cast<_Float16 *>(out) = static_cast<_Float16>(r);
}

// ---------------------------------------------------------------------------
// decode_merge_planned: grid (merge entry, group of HPW query heads); the
// pieces of sequence s are records first .. first + n - 1.  A merge's records
// of HPW consecutive heads are HPW x 128 contiguous floats; thread t merges
// elements t, t + 256, ... of them (HPW / 2 each).  Few merges (decode
// steps) keep two heads per work-group for parallelism; many (cut prompt
// tiles, one merge per query token) take more heads per work-group rather
// than launch tens of thousands of tiny ones.
// ---------------------------------------------------------------------------
// N records (N <= kMergeBatch) of E elements per thread, every load issued
// before any arithmetic: the same sums in the same order as merge_records.
template <int N, int E, typename Ptr>
__device__ __forceinline__ void merge_records_n(const Ptr &ptrs, float (&res)[E]) {
    float2 ml[E][N];
    float o[E][N];
#pragma unroll
    for (int k = 0; k < E; ++k)
#pragma unroll
        for (int i = 0; i < N; ++i) ptrs(k, i, ml[k][i], o[k][i]);
#pragma unroll
    for (int k = 0; k < E; ++k) {
        float M = -INFINITY;
#pragma unroll
        for (int i = 0; i < N; ++i) M = fmaxf(M, ml[k][i].x);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const float wgt = ml[k][i].x == -INFINITY ? 0.0f : fast_exp2(ml[k][i].x - M);
            L += wgt * ml[k][i].y;
            O += wgt * o[k][i];
        }
        res[k] = O / L;
    }
}

template <int HPW>
__global__ __launch_bounds__(256) void decode_merge_planned_kernel(DecodeArgs a) {
    static_assert(HPW % 2 == 0 && HPW <= 32, "heads per work-group");
    constexpr int E = HPW / 2;  // elements per thread
    const int32_t *m = a.merges + kMergeInts * static_cast<size_t>(blockIdx.x);
    const int row = min(max(m[3], 0), a.num_q_rows - 1);  // the output row
    const int first = max(m[1], 0);
    const int n = min(m[2], a.num_slots - first);
    const int d = static_cast<int>(threadIdx.x) % kHeadDim;
    const int h0 = static_cast<int>(blockIdx.y) * HPW + static_cast<int>(threadIdx.x) / kHeadDim;  // + 2k
    // 2 to 4 records (cut prompt tiles, most decode merges): straight-line
    if (n >= 2 && n <= 4 && static_cast<int>(blockIdx.y) * HPW + HPW <= a.num_q_heads) {
        auto ptrs = [&](int k, int i, float2 &mlv, float &ov) {
            const size_t rec = static_cast<size_t>(first + i) * a.num_q_heads + h0 + 2 * k;
            mlv = *reinterpret_cast<const float2 *>(a.ml_part + rec * 2);
            ov = a.o_part[rec * kHeadDim + d];
        };
        float res[E];
        if (n == 2) merge_records_n<2, E>(ptrs, res);
        else if (n == 3) merge_records_n<3, E>(ptrs, res);
        else merge_records_n<4, E>(ptrs, res);
#pragma unroll
        for (int k = 0; k < E; ++k)
            *reinterpret_cast<_Float16 *>(a.out + (static_cast<size_t>(row) * a.num_q_heads + h0 + 2 * k) * kHeadDim +
                                          d) = static_cast<_Float16>(res[k]);
        return;
    }
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int e = static_cast<int>(threadIdx.x) + 256 * k;
        const int h = static_cast<int>(blockIdx.y) * HPW + e / kHeadDim;
        const int d = e % kHeadDim;
        if (h >= a.num_q_heads) break;
        uint16_t *out = a.out + (static_cast<size_t>(row) * a.num_q_heads + h) * kHeadDim + d;
        if (n <= 0) {
            *out = 0;
            continue;
        }
        const float r = merge_records(n, [&](int i, float2 &mlv, float &ov) {
            const size_t rec = static_cast<size_t>(first + i) * a.num_q_heads + h;
            mlv = *reinterpret_cast<const float2 *>(a.ml_part + rec * 2);
            ov = a.o_part[rec * kHeadDim + d];
        });
        *reinterpret_cast<_Float16 *>(out) = static_cast<_Float16>(r);
    }
}

// ---------------------------------------------------------------------------
// decode_prefix: shared-prefix (cascade) pieces.  Sequences of a group share
// the physical blocks of a common prefix (reference-counted blocks, "Reading
// Inference Engine Codebases", Examples 3 and 12); one work-group per (piece,
// KV head) reads each prefix K/V tile once for all members.  Up to 16
// members x 4 query heads = 64 stacked query rows make Q K^T and P V real
// dense tiles, computed with v_mfma_f32_16x16x16_f16:
//   wave w owns rows 16w .. 16w+15: row 16w + 4r + j is member 4w + r, query
//   head 4g + j.  In the lane layout of the MFMA (lane l, n = l % 16,
//   r = l / 16):
//   S^T = K . Q^T   A = K tile   (lane: MFMA row n = token 4(n%4) + n/4,
//                                 dims {32i + 8r + 4u + c})
//                   B = Q^T      (lane: row n, the same dims)
//                   D = S^T      (lane: tokens 4c + r of row n)
//   O   = P . V     A = P        (lane: row n, k-slot 4r + c = token 4c + r)
//                                 -- D of S^T as is
//                   B = V        (lane: tokens 4c + r at dim 8n + j, MFMA j:
//                                 byte permutes of the lane's V registers,
//                                 token 4c + r, dims 8n .. 8n+7)
//                   D = O        (lane: rows 4r + c, dim 8n + j)
// Each member's result is a partial record (o, m, l), merged with the
// member's own suffix pieces by decode_merge_planned.  FP8 pools: each lane
// loads the same tokens and dims as 8-byte code groups and widens them to
// F16 in registers; K's scale is folded into the score scale and V's
// multiplies the records, which then hold values like every other piece's.
// ---------------------------------------------------------------------------
struct h4x2 {
    h4 v[2];
};
__device__ __forceinline__ h4x2 quads(h8 x) { return __builtin_bit_cast(h4x2, x); }


template <bool FP8>
__device__ __forceinline__ void prefix_body(const DecodeArgs &a, uint32_t bx) {
    const int g = static_cast<int>(bx % a.num_kv_heads);
    const int32_t *it = a.prefix_items + kPrefixItemInts * static_cast<size_t>(bx / a.num_kv_heads);
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int n = lane & 15, r = lane >> 4;

    __shared__ int tbl_lds[kMaxPrefixPieceBlocks];
    __shared__ float alpha_lds[kWaves][16];
    __shared__ float ml_lds[kWaves][16][2];

    // Plan entries are clamped so a damaged plan cannot index outside the
    // buffers.
    const int first_seq = min(max(it[0], 0), a.batch - 1);
    const int b_begin = max(it[1], 0) / kBlockSize;
    const int t_end = min(it[2], a.max_blocks * kBlockSize);
    const int b_end = min((t_end + kBlockSize - 1) / kBlockSize, b_begin + kMaxPrefixPieceBlocks);
    const int n_members = min(min(max(it[3], 0), kMaxMembers), a.num_members);
    const int moff = min(max(it[4], 0), max(a.num_members - n_members, 0));
    if (b_begin >= b_end || a.num_slots <= 0) return;

    // this lane's query row (as the B operand) and its member
    const int member = 4 * w + (n >> 2);
    const bool row_valid = member < n_members;
    h8 qv[4];
    if (row_valid) {
        const int sq = min(max(a.members[kMemberInts * (moff + member)], 0), a.batch - 1);
        const uint16_t *qrow = a.q + (static_cast<size_t>(sq) * a.num_q_heads + g * kGroup + (n & 3)) * kHeadDim;
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[i] = *reinterpret_cast<const h8 *>(qrow + 32 * i + 8 * r);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[i] = h8(0);
    }

    // the prefix's block ids, from the first member's table row
    const int32_t *table = a.tables + static_cast<size_t>(first_seq) * a.max_blocks;
    if (tid < b_end - b_begin) tbl_lds[tid] = table[b_begin + tid];
    __syncthreads();

    const uint32_t last_block = static_cast<uint32_t>(a.num_blocks - 1);
    constexpr int kElem = FP8 ? 1 : 2;
    const size_t tile_bytes = tile_elems() * kElem;
    const char *k_layer = a.k_layer;
    const char *v_layer = a.v_layer;
    // K: MFMA row n is token 4(n%4) + n/4, dims 32i + 8r .. +7, so S^T gives
    // lane (r, n) the scores of tokens 4c + r -- the tokens of its V registers:
    // V: token 4c + r, dims 8n .. +7
    const int ktok = 4 * (n & 3) + (n >> 2);
    const uint32_t k_off = static_cast<uint32_t>((ktok * kHeadDim + 8 * r) * kElem);  // + 32 i elements
    const uint32_t v_off = static_cast<uint32_t>((r * kHeadDim + 8 * n) * kElem);  // + 4 c rows

    float m_run = -INFINITY;  // running max of row n (log2 units)
    float l_run = 0.0f;       // this lane's share of row n's running sum
    f4 acc[8];  // MFMA j's result: acc[j][c] = row 4r + c at dim 8n + j
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[dt] = f4{0.f, 0.f, 0.f, 0.f};

    h8 kb[PA_PREFIX_NBUF][4], vb[PA_PREFIX_NBUF][4];
    u2 kr8[PA_PREFIX_NBUF][4], vr8[PA_PREFIX_NBUF][4];  // FP8 pools: raw codes until consumed
    auto issue = [&](int buf, int b) {
        const bool live = b < b_end;
        uint32_t phys = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(tbl_lds[live ? b - b_begin : 0]));
        phys = phys > last_block ? last_block : phys;
        const size_t base = (static_cast<size_t>(phys) * a.num_kv_heads + g) * tile_bytes;
        const int bytes = live ? static_cast<int>(tile_bytes) : 0;
        const __amdgpu_buffer_rsrc_t kr = tile_rsrc(k_layer + base, bytes);
        const __amdgpu_buffer_rsrc_t vr = tile_rsrc(v_layer + base, bytes);
        if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) kr8[buf][i] = load_shared8(kr, k_off + 32u * i);
#pragma unroll
            for (int c = 0; c < 4; ++c) vr8[buf][c] = load_shared8(vr, v_off + 512u * c);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) kb[buf][i] = load_shared16(kr, k_off + 64u * i);
#pragma unroll
            for (int c = 0; c < 4; ++c) vb[buf][c] = load_shared16(vr, v_off + 1024u * c);
        }
    };
    auto widen = [&](int buf) {  // FP8: the buffer's codes to F16
        if constexpr (FP8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) kb[buf][i] = fp8_decode8_h(kr8[buf][i].x, kr8[buf][i].y);
#pragma unroll
            for (int c = 0; c < 4; ++c) vb[buf][c] = fp8_decode8_h(vr8[buf][c].x, vr8[buf][c].y);
        }
    };

    auto consume = [&](int buf, int b) {
        widen(buf);
        // S^T for this wave's 16 rows
        f4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const h4x2 kk = quads(kb[buf][i]);
            const h4x2 qq = quads(qv[i]);
            st = __builtin_amdgcn_mfma_f32_16x16x16f16(kk.v[0], qq.v[0], st, 0, 0, 0);
            st = __builtin_amdgcn_mfma_f32_16x16x16f16(kk.v[1], qq.v[1], st, 0, 0, 0);
        }
        const int valid = min(kBlockSize, t_end - b * kBlockSize);
        float sc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) sc[c] = (4 * c + r < valid) ? st[c] * a.scale_log2e : -INFINITY;
        const float bmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        if (__builtin_amdgcn_ballot_w64(bmax > m_run + kTau) != 0) {
            float bm = bmax;
            bm = fmaxf(bm, shfl_xor(bm, 16));
            bm = fmaxf(bm, shfl_xor(bm, 32));
            const float m_new = fmaxf(m_run, bm);
            const float alpha = fast_exp2(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
            if (r == 0) alpha_lds[w][n] = alpha;
            wave_lds_sync();
            const float4 al = *reinterpret_cast<const float4 *>(&alpha_lds[w][4 * r]);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                acc[dt][0] *= al.x;
                acc[dt][1] *= al.y;
                acc[dt][2] *= al.z;
                acc[dt][3] *= al.w;
            }
        }
        // weights enter P V as F16; the running sum adds the same rounded
        // values, so numerator and denominator use identical weights
        h4 pa;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pa[c] = static_cast<_Float16>(fast_exp2(sc[c] - m_run));
            l_run += static_cast<float>(pa[c]);
        }
        // P V, one MFMA per dim 8n + j: byte permutes gather dim 8n + j of the
        // lane's four tokens (stale slots past the context are zeroed)
        u4 vv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) vv[c] = (4 * c + r >= valid) ? u4(0u) : __builtin_bit_cast(u4, vb[buf][c]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t t01 = __builtin_amdgcn_perm(vv[1][j >> 1], vv[0][j >> 1], sel);
            const uint32_t t23 = __builtin_amdgcn_perm(vv[3][j >> 1], vv[2][j >> 1], sel);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, __builtin_bit_cast(h4, u2{t01, t23}), acc[j], 0, 0, 0);
        }
    };

    // Software pipeline as in decode_partial: block b + NBUF - 1 is issued
    // before block b is consumed, the prologue's loads in issue order.
    constexpr int NBUF = PA_PREFIX_NBUF;
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i) {
        issue(i, b_begin + i);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int base = b_begin; base < b_end; base += NBUF) {
#pragma unroll
        for (int u = 0; u < NBUF; ++u) {
            issue((u + NBUF - 1) % NBUF, base + u + NBUF - 1);
            if (base + u < b_end) consume(u, base + u);
        }
    }

    // row sums over the four lane groups; (m, l) of rows 4r + c via LDS
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);
    if (r == 0) {
        ml_lds[w][n][0] = m_run;
        ml_lds[w][n][1] = l_run;
    }
    wave_lds_sync();
    const int my_member = 4 * w + r;  // rows 4r + c of the O layout
    if (my_member < n_members) {
        const int32_t *mem = a.members + kMemberInts * (moff + my_member);
        const int slot = min(max(mem[1], 0), a.num_slots - 1);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const size_t rec = static_cast<size_t>(slot) * a.num_q_heads + g * kGroup + c;
            const float vs = FP8 ? a.v_scale : 1.0f;
            float4 *dst = reinterpret_cast<float4 *>(a.o_part + rec * kHeadDim + 8 * n);
            dst[0] = make_float4(acc[0][c] * vs, acc[1][c] * vs, acc[2][c] * vs, acc[3][c] * vs);
            dst[1] = make_float4(acc[4][c] * vs, acc[5][c] * vs, acc[6][c] * vs, acc[7][c] * vs);
            if (n == 0) {
                a.ml_part[rec * 2] = ml_lds[w][4 * r + c][0];
                a.ml_part[rec * 2 + 1] = ml_lds[w][4 * r + c][1];
            }
        }
    }
}

template <bool FP8>
__global__ __launch_bounds__(256) void decode_prefix_kernel(DecodeArgs a) {
    prefix_body<FP8>(a, blockIdx.x);
}

// A shared-prefix (cascade) step in one launch: work-groups
// [0, decode items x Hkv) run ordinary pieces (whole contexts and the
// members' suffixes), the rest the shared-prefix pieces, so the prefix tiles
// stream beside the suffixes instead of in a launch of their own.
template <bool FP8>
__global__ __launch_bounds__(256, 2) void cascade_kernel(DecodeArgs a) {
    const uint32_t nd = static_cast<uint32_t>(a.num_items) * static_cast<uint32_t>(a.num_kv_heads);
    if (blockIdx.x < nd)
        decode_partial_body<FP8 ? PA_DECODE_NBUF_FP8 : PA_DECODE_NBUF, FP8>(a, blockIdx.x, 0, 0);
    else
        prefix_body<FP8>(a, blockIdx.x - nd);
}

// ---------------------------------------------------------------------------
// prefill: chunked-prefill pieces of a mixed step ("Batching and Scheduling",
// Example 5).  One work-group per (piece, KV head); a piece is a
// tile of up to kPrefillTile query tokens of one sequence against a range of
// its key blocks.  The tile's queries sit at positions pos0 .. pos0+n_q-1 and
// query t sees keys 0 .. pos0 + t (causal).  Wave w owns query tokens
// 16(w/2) .. +15 and query heads 4g + 2(w%2) + rt, rt < 2: two 16-row tiles
// whose row n is token 16(w/2) + n.
// Key blocks come kStageBlocks at a time: the work-group copies the stage's
// K and V tiles into LDS once -- each wave a quarter, 1 KiB per load
// instruction -- double-buffered, one barrier per stage (FP8 pools: the
// codes are widened to F16 on the way into LDS, so the arithmetic below is
// the F16 path's; K's scale is folded into the score scale and V's applied
// to the result); each wave then works
// through the stage two blocks at a time, reading its MFMA operands once per
// pair.
//   S^T = K . Q^T  v_mfma_f32_16x16x32_f16 per 32 dims and block:
//                  A = K   (lane l: token l%16 of the block, 8 dims)
//                  B = Q^T (lane l: row l%16, the same 8 dims)
//                  D = S^T (lane l: tokens 4(l/16) + c, c < 4, of row l%16)
//   O  += P . V    v_mfma_f32_16x16x32_f16 per 16 dims 16j .. 16j+15 and
//                  block pair:
//                  A = P   (lane l: row l%16, tokens 4(l/16) + c of both
//                           blocks -- D of S^T as is, rounded to F16)
//                  B = V   (lane l: the same 8 tokens at dim 16j + l%16, two
//                           LDS transpose reads, one per block)
//                  D = O   (lane l: rows 4(l/16) + c, dim 16j + l%16)
//   l  += P . 1    (F16 pools) one more such MFMA per row tile and pair with
//                  B all ones: the row sums of the same F16 weights, in D's
//                  row layout (FP8 pools add them with v_dot2 per lane and
//                  reduce across lanes at the end)
// Each wave computes only up to its last query's position, and masks only
// the pairs that reach past its first query's position or its last key.
// The softmax max is raised lazily as in the decode kernel (the comparison
// runs on raw scores, the scale enters once through the exponent's FMA); a
// row that sees no key of the piece keeps (m, l) = (-inf, 0).  A tile cut
// into several pieces writes partial records (token k of piece p at record
// base + k * pieces + p) for decode_merge_planned; a single piece writes F16
// rows.
// ---------------------------------------------------------------------------
// Maximum of three scores in one v_max3_f32.  fmaxf on values the compiler
// cannot prove canonical (matrix-core results, masked selects) first passes
// each through v_max_f32 x, x to quiet signalling NaNs, as IEEE mode asks:
// 6 extra instructions per 8 scores here.  Scores are finite or -inf, so the
// plain instruction gives the same maximum.  Measured on the 2016-token
// chunk: 125.3-126.0 -> 123.1-123.2 us per layer.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
    float d;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}
// LDS layouts of the K/V tiles, chosen by measuring SQ_LDS_BANK_CONFLICT
// for each access pattern alone on gfx950.  A key operand read takes one
// 16-byte chunk of each of 16 rows per 16-lane group; a value transpose read
// takes 32 bytes of each of 4 rows per 16-lane group; the register-staged
// copy writes one whole row per 16 lanes.
//  - Padded rows (register-staged copy): a row stride that is an odd
//    multiple of 8 dwords (72, 88, 104, 120) is conflict-free for both
//    reads; 68, 76, 80 or 84 dwords conflicted 2-way, 96 dwords 4-way.  The
//    reads keep one base address per lane and immediate offsets.  Writes of
//    one row per 16 lanes are conflict-free; two rows per 16 lanes were not.
//  - Unpadded 256-byte rows (copy straight into LDS, 1 KiB per
//    instruction): 16-byte chunk c of key row t at c ^ k_swz(t), of value
//    row t at c ^ v_swz(t), conflict-free; XORs over 8 (K) and 4 (V) rows
//    conflicted 2-way, unswizzled K rows 8-way.
// The F16 prompt chunk went from 12.3 M conflict cycles per launch to none.
constexpr int kPadRow = kHeadDim + 16;  // halves: 72 dwords
__device__ __forceinline__ int k_swz(int t) { return t & 15; }
__device__ __forceinline__ int v_swz(int t) { return 2 * (t & 7); }

// ds_read_b64_tr_b16: within each 16-lane group, lane 4a + b receives half b
// of the 8-byte chunks addressed by lanes a, a + 4, a + 8, a + 12 (in that
// order); p must point into LDS
typedef __attribute__((address_space(3))) s4 lds_s4;
__device__ __forceinline__ h4 lds_read_tr16(const _Float16 *p) {
    return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(p)));
}
#ifndef PA_PREFILL_STAGE_BLOCKS
#define PA_PREFILL_STAGE_BLOCKS 2
#endif
constexpr int kStageBlocks = PA_PREFILL_STAGE_BLOCKS;  // key blocks per LDS stage (even)
static_assert(kStageBlocks % 2 == 0 && kStageBlocks >= 2, "stages hold whole pairs");

// Prompt-chunk pieces over an FP8 pool: the codes go through registers, one
// stage ahead, and are widened to F16 on their way into LDS (F16 pools take
// prefill_body_dma below, which copies straight into LDS).
// SPLIT: as in prefill_body_dma, eight waves in two groups over the same
// rows, each group half of the piece's stages in its own buffers, merged
// through LDS at the end.
template <bool SPLIT = false>
__device__ __forceinline__ void prefill_body_fp8(const DecodeArgs &a, uint32_t bx) {
    constexpr int kGroups = SPLIT ? 2 : 1;
    constexpr int kThreads = 256 * kGroups;
    const int g = static_cast<int>(bx % a.num_kv_heads);
    const int32_t *it = a.prefill_items + kPrefillItemInts * static_cast<size_t>(bx / a.num_kv_heads);
    const int tid = threadIdx.x;
    const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave of the work-group
    const int grp = SPLIT ? w8 >> 2 : 0;                      // its group
    const int w = SPLIT ? w8 & 3 : w8;                        // its wave within the group
    const int lane = tid & 63;
    const int n = lane & 15, r = lane >> 4;

    __shared__ int tbl_lds[kMaxPrefillPieceBlocks];
    // [group][buffer][block][row][dim]
    __shared__ __attribute__((aligned(16))) _Float16 k_lds_g[kGroups][2][kStageBlocks][kBlockSize][kPadRow];
    __shared__ __attribute__((aligned(16))) _Float16 v_lds_g[kGroups][2][kStageBlocks][kBlockSize][kPadRow];
    auto &k_lds = k_lds_g[grp];
    auto &v_lds = v_lds_g[grp];
    // the tile row r of tensor t (0: K, 1: V) in stage buffer buf
    auto kv_row = [&](int buf, int t, int blk, int row) -> _Float16 * {
        return t ? &v_lds[buf][blk][row][0] : &k_lds[buf][blk][row][0];
    };
    __shared__ float alpha_lds[kGroups * kWaves][2][16];
    __shared__ float ml_lds[kGroups * kWaves][2][16][2];

    // Plan entries are clamped so a damaged plan cannot index outside q, out,
    // the tables, the pool or the workspace.
    const int s = min(max(it[0], 0), a.batch - 1);
    const int row0 = max(it[1], 0);
    const int n_q = min(max(it[2], 0), kPrefillTile);
    const int pos0 = max(it[3], 0);
    const int cap = a.max_blocks * kBlockSize;
    const int t_lo = min(max(it[4], 0), cap) & ~(kBlockSize - 1);
    const int t_hi = min(min(it[5], cap), pos0 + n_q);
    const int base_slot = it[6];
    const int np = max(it[7], 1);
    const int piece = min(max(it[8], 0), np - 1);
    const bool direct = base_slot < 0;
    if (!direct && a.num_slots <= 0) return;
    const int b_lo = t_lo / kBlockSize;
    const int b_hi = max(b_lo, min((t_hi + kBlockSize - 1) / kBlockSize, b_lo + kMaxPrefillPieceBlocks));

    const int32_t *table = a.tables + static_cast<size_t>(s) * a.max_blocks;
    for (int i = tid; i < b_hi - b_lo; i += kThreads) tbl_lds[i] = table[b_lo + i];
    __syncthreads();

    // this wave's query tokens and heads, and the keys its rows can see
    const int tok0 = 16 * (w >> 1);
    const int head0 = g * kGroup + 2 * (w & 1);
    const int rows_w = min(16, n_q - tok0);  // may be <= 0: the wave then only helps with the copies
    const int w_end = rows_w > 0 ? min(t_hi, pos0 + tok0 + rows_w) : t_lo;
    const int qp = pos0 + tok0 + n;  // position of row n

    // Q of the two row tiles, as the B operand of S^T: dims 32kk + 8r .. +7
    h8 qv[2][4];
    {
        const bool row_ok = n < rows_w;
        const size_t qr = static_cast<size_t>(min(max(row0 + tok0 + n, 0), a.num_q_rows - 1));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const uint16_t *qrow = a.q + (qr * a.num_q_heads + head0 + rt) * kHeadDim + 8 * r;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const h8 x = *reinterpret_cast<const h8 *>(qrow + 32 * kk);
                qv[rt][kk] = row_ok ? x : h8(0);
            }
        }
    }

    f4 oacc[2][8];
    float m_run[2], l_run[2];  // row n of each tile, log2 units (l: this lane's share)
    float negm[2];             // the weights' offset: -m_run, 0 while m_run = -inf
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        m_run[rt] = -INFINITY;
        negm[rt] = 0.0f;
        l_run[rt] = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) oacc[rt][j] = f4{0.f, 0.f, 0.f, 0.f};
    }
    const float c_scale = a.scale_log2e;
    const h2 ones = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};

    // copies: wave w moves tensor w/2 (K, V) of block w%2 of the pair: lane l
    // takes row l/16 + 4i, codes 8(l%16) .. +7, so each 16-lane pass of the
    // LDS writes covers one whole row
    const uint32_t last_block = static_cast<uint32_t>(a.num_blocks - 1);
    const size_t tile_bytes = tile_elems();        // one byte per code
    constexpr int kCopyBlocks = kStageBlocks / 2;  // blocks of one tensor each wave copies per stage
    constexpr int kLoads = 4;                      // 8-byte loads per lane and tile
    const int cp_tensor = w >> 1, cp_blk0 = (w & 1) * kCopyBlocks;
    const char *cp_layer = cp_tensor ? a.v_layer : a.k_layer;
    u2 stg8[kCopyBlocks][kLoads];  // raw codes of the next stage, widened at commit
    // Value rows at or past the piece's last key (t_hi) may hold anything
    // (slots past the sequence in its last block): the V resource ends at the
    // last row below t_hi, so those rows load as zeros and their zero weights
    // cannot meet a NaN.  Keys below t_hi are stored tokens, finite like every
    // key the rows see.
    auto fetch = [&](int b) {  // stage starting at block b, into the staging registers
#pragma unroll
        for (int x = 0; x < kCopyBlocks; ++x) {
            const int bb = b + cp_blk0 + x;
            const bool live = bb < b_hi;
            uint32_t phys = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(tbl_lds[live ? bb - b_lo : 0]));
            phys = phys > last_block ? last_block : phys;
            const size_t base = (static_cast<size_t>(phys) * a.num_kv_heads + g) * tile_bytes;
            // a live block holds at least one key (bb < b_hi), so only the
            // upper clamp is needed for its value rows; all of it in scalar
            // registers (wave-uniform, so no per-lane loop around the loads)
            const int rows = cp_tensor ? min(t_hi - bb * kBlockSize, kBlockSize) : kBlockSize;
            const int bytes = live ? rows * kHeadDim : 0;
            const __amdgpu_buffer_rsrc_t rs = tile_rsrc(cp_layer + base, bytes);
#pragma unroll
            for (int i = 0; i < kLoads; ++i) stg8[x][i] = load_shared8(rs, static_cast<uint32_t>(8 * lane + 512 * i));
        }
    };
    auto commit = [&](int buf) {  // the staging registers, widened, into LDS buffer buf
#pragma unroll
        for (int x = 0; x < kCopyBlocks; ++x)
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
                _Float16 *dst = kv_row(buf, cp_tensor, cp_blk0 + x, (lane >> 4) + 4 * i) + 8 * n;
                *reinterpret_cast<h8 *>(dst) = fp8_decode8_h(stg8[x][i].x, stg8[x][i].y);
            }
    };

    // transpose reads: lane l addresses token 4(l/16) + (l/4)%4, dims 4(l%4) .. +3
    // of a 16-dim slice, so that lane (r, n) receives tokens 4r .. 4r+3 at dim n
    const int tr_row = 4 * r + ((lane >> 2) & 3), tr_col = 4 * (lane & 3);
    auto compute = [&](int buf, int sb, int b) {  // blocks sb, sb+1 of the stage = key blocks b, b+1
        // the pair's K operands, read once for both row tiles
        h8 kx[2][4];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                kx[blk][kk] = *reinterpret_cast<const h8 *>(&k_lds[buf][sb + blk][n][32 * kk + 8 * r]);
        f4 st[2][2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) st[rt][blk] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
                    st[rt][blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kx[blk][kk], qv[rt][kk], st[rt][blk], 0, 0, 0);
        // masks, only where the pair reaches past the first row's position or
        // the last key this wave sees
        const int k_last = b * kBlockSize + 2 * kBlockSize - 1;
        const bool tail = k_last >= w_end;
        if (k_last > pos0 + tok0 || tail) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int kp = (b + blk) * kBlockSize + 4 * r + c;
                    const bool vis = kp < w_end && kp <= qp;
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) st[rt][blk][c] = vis ? st[rt][blk][c] : -INFINITY;
                }
        }
        h8 pw[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const float m1 = max3_raw(st[rt][0][0], st[rt][0][1], st[rt][0][2]);
            const float m2 = max3_raw(st[rt][0][3], st[rt][1][0], st[rt][1][1]);
            const float m3 = max3_raw(st[rt][1][2], st[rt][1][3], m1);
            const float bmax = max3_raw(m2, m3, m3);
            const float mb = bmax * c_scale;
            if (__builtin_amdgcn_ballot_w64(mb > m_run[rt] + kTau) != 0) {
                float bm = mb;
                bm = fmaxf(bm, shfl_xor(bm, 16));
                bm = fmaxf(bm, shfl_xor(bm, 32));
                const float m_new = fmaxf(m_run[rt], bm);
                // a row that has seen no key yet keeps m = -inf (and alpha 1)
                const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_run[rt] - m_new);
                l_run[rt] *= alpha;
                m_run[rt] = m_new;
                negm[rt] = m_new == -INFINITY ? 0.0f : -m_new;
                if (r == 0) alpha_lds[w8][rt][n] = alpha;
                wave_lds_sync();
                const float4 al = *reinterpret_cast<const float4 *>(&alpha_lds[w8][rt][4 * r]);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    oacc[rt][j][0] *= al.x;
                    oacc[rt][j][1] *= al.y;
                    oacc[rt][j][2] *= al.z;
                    oacc[rt][j][3] *= al.w;
                }
            }
            // weights exp2(s * scale - m) enter P V as F16; the running sum
            // adds the same rounded values (masked scores give exp2(-inf) = 0)
            const float neg_m = negm[rt];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int c = 0; c < 4; c += 2) {
                    const float p0 = fast_exp2(fmaf(st[rt][blk][c], c_scale, neg_m));
                    const float p1 = fast_exp2(fmaf(st[rt][blk][c + 1], c_scale, neg_m));
                    const h2 pp = {static_cast<_Float16>(p0), static_cast<_Float16>(p1)};
                    pw[rt][4 * blk + c] = pp.x;
                    pw[rt][4 * blk + c + 1] = pp.y;
                    l_run[rt] = __builtin_amdgcn_fdot2(pp, ones, l_run[rt], false);
                }
        }
        // P V over dims 16j .. 16j+15: lane (r, n) gets tokens 4r .. 4r+3 of
        // each block at dim 16j + n straight from the transpose reads
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            h4 t[2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) t[blk] = lds_read_tr16(&v_lds[buf][sb + blk][tr_row][16 * j + tr_col]);
            const h8 bv = {t[0][0], t[0][1], t[0][2], t[0][3], t[1][0], t[1][1], t[1][2], t[1][3]};
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                oacc[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pw[rt], bv, oacc[rt][j], 0, 0, 0);
        }
    };

    // the work-group walks every pair of the piece; a wave computes the pairs
    // below its last query's position
    const int n_stages = (b_hi - b_lo + kStageBlocks - 1) / kStageBlocks;
    const int w_blocks = w_end > t_lo ? (w_end + kBlockSize - 1) / kBlockSize - b_lo : 0;  // blocks this wave needs
    const int half = (n_stages + 1) / 2;
    const int my_first = SPLIT && grp ? half : 0;                            // first stage of this group
    const int my_count = SPLIT ? (grp ? n_stages - half : half) : n_stages;  // its stages
    const int rounds = SPLIT ? half : n_stages;  // barrier rounds, the same for both groups
    if (rounds > 0) {
        if (!SPLIT || my_count > 0) {
            fetch(b_lo + kStageBlocks * my_first);
            commit(0);
        }
        __syncthreads();
    }
    // this group's stage st reads its LDS buffer st % 2; meanwhile stage st+1
    // is loaded into the staging registers and, at the end, goes into LDS
    // buffer (st+1) % 2, which stage st-1 read before the last barrier
    auto stage = [&](int st, auto bufc) {
        constexpr int S = decltype(bufc)::value;  // == st % 2
        const int gst = my_first + st;            // the stage within the piece
        const int b0 = b_lo + kStageBlocks * gst;
        if (st + 1 < my_count) fetch(b0 + kStageBlocks);
        if (!SPLIT || st < my_count) {
#pragma unroll
            for (int sb = 0; sb < kStageBlocks; sb += 2)
                if (kStageBlocks * gst + sb < w_blocks) compute(S, sb, b0 + sb);
        }
        if (st + 1 < my_count) commit(S ^ 1);
        __syncthreads();
    };
    for (int st = 0; st < rounds; st += 2) {
        stage(st, std::integral_constant<int, 0>{});
        if (st + 1 < rounds) stage(st + 1, std::integral_constant<int, 1>{});
    }
    float mm[2][4], ll[2][4];  // SPLIT: the merged max and sum of rows 4r + c
    if constexpr (SPLIT) {
        // both groups' (max, sum) of every row to LDS; group 1 hands its
        // outputs to group 0 through the free key buffers, one row tile at
        // a time (32 values per lane), and group 0 merges
        float *mrg = reinterpret_cast<float *>(&k_lds_g[0][0][0][0][0]);  // [wave][32][64]
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float l = l_run[rt];
            l += shfl_xor(l, 16);
            l += shfl_xor(l, 32);
            if (r == 0) {
                ml_lds[w8][rt][n][0] = m_run[rt];
                ml_lds[w8][rt][n][1] = l;
            }
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            if (grp == 1) {
                float *dst = mrg + w * 32 * 64 + lane;
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) dst[(j * 4 + c) * 64] = oacc[rt][j][c];
            }
            __syncthreads();
            if (grp == 0 && rows_w > 0) {
                const float *src = mrg + w * 32 * 64 + lane;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int t = 4 * r + c;
                    const float m0 = ml_lds[w][rt][t][0], l0 = ml_lds[w][rt][t][1];
                    const float m1 = ml_lds[4 + w][rt][t][0], l1 = ml_lds[4 + w][rt][t][1];
                    const float M = fmaxf(m0, m1);
                    const float a0 = m0 == -INFINITY ? 0.0f : fast_exp2(m0 - M);
                    const float a1 = m1 == -INFINITY ? 0.0f : fast_exp2(m1 - M);
#pragma unroll
                    for (int j = 0; j < 8; ++j) oacc[rt][j][c] = a0 * oacc[rt][j][c] + a1 * src[(j * 4 + c) * 64];
                    mm[rt][c] = M;
                    ll[rt][c] = a0 * l0 + a1 * l1;
                }
            }
            __syncthreads();
        }
        if (grp == 1) return;
    }
    if (rows_w <= 0) return;

    if constexpr (!SPLIT) {
        // (m, l) of every row to LDS; lane l then writes rows 4r + c of each tile
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float l = l_run[rt];
            l += shfl_xor(l, 16);
            l += shfl_xor(l, 32);
            if (r == 0) {
                ml_lds[w][rt][n][0] = m_run[rt];
                ml_lds[w][rt][n][1] = l;
            }
        }
        wave_lds_sync();
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int head = head0 + rt;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int t = 4 * r + c;  // row of the tile
            if (t >= rows_w) continue;
            const int tok = tok0 + t;
            const float m = SPLIT ? mm[rt][c] : ml_lds[w][rt][t][0], l = SPLIT ? ll[rt][c] : ml_lds[w][rt][t][1];
            if (direct) {
                const size_t qrow = static_cast<size_t>(min(row0 + tok, a.num_q_rows - 1));
                const float inv = a.v_scale / l;  // V's scale
                _Float16 *orow = reinterpret_cast<_Float16 *>(a.out + (qrow * a.num_q_heads + head) * kHeadDim);
#pragma unroll
                for (int j = 0; j < 8; ++j) orow[16 * j + n] = static_cast<_Float16>(oacc[rt][j][c] * inv);  // dim 16j + n
            } else {
                const int64_t slot64 = static_cast<int64_t>(base_slot) + static_cast<int64_t>(tok) * np + piece;
                const size_t slot = static_cast<size_t>(min<int64_t>(slot64, a.num_slots - 1));
                const size_t rec = slot * a.num_q_heads + head;
                // records hold values (V's scale applied), as the decode pieces' do
#pragma unroll
                for (int j = 0; j < 8; ++j) a.o_part[rec * kHeadDim + 16 * j + n] = oacc[rt][j][c] * a.v_scale;
                if (n == 0) *reinterpret_cast<float2 *>(a.ml_part + rec * 2) = make_float2(m, l);
            }
        }
    }
}

// LDS-DMA prefill helpers: the compiler cannot see which LDS buffer an
// intrinsic transpose read touches and would wait for every DMA in flight;
// these reads and the barrier are plain instructions whose waits are explicit.
__device__ __forceinline__ uint32_t lds_addr(const _Float16 *p) {
    return (uint32_t)(size_t)((const __attribute__((address_space(3))) _Float16 *)p);
}
// eight transpose reads, complete when the statement ends
__device__ __forceinline__ void lds_read_tr16_x8(u2 (&d)[8], const uint32_t (&a)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %10\n\t"
        "ds_read_b64_tr_b16 %3, %11\n\t"
        "ds_read_b64_tr_b16 %4, %12\n\t"
        "ds_read_b64_tr_b16 %5, %13\n\t"
        "ds_read_b64_tr_b16 %6, %14\n\t"
        "ds_read_b64_tr_b16 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]), "=&v"(d[6]), "=&v"(d[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
}
// sixteen transpose reads in the order of two lds_read_tr16_x8 calls, two
// per address (the second 4 KiB further on: the stage's next key block),
// complete when the statement ends
__device__ __forceinline__ void lds_read_tr16_x16(u2 (&d)[2][8], const uint32_t (&a)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\t"
        "ds_read_b64_tr_b16 %1, %16 offset:4096\n\t"
        "ds_read_b64_tr_b16 %2, %17\n\t"
        "ds_read_b64_tr_b16 %3, %17 offset:4096\n\t"
        "ds_read_b64_tr_b16 %4, %18\n\t"
        "ds_read_b64_tr_b16 %5, %18 offset:4096\n\t"
        "ds_read_b64_tr_b16 %6, %19\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:4096\n\t"
        "ds_read_b64_tr_b16 %8, %20\n\t"
        "ds_read_b64_tr_b16 %9, %20 offset:4096\n\t"
        "ds_read_b64_tr_b16 %10, %21\n\t"
        "ds_read_b64_tr_b16 %11, %21 offset:4096\n\t"
        "ds_read_b64_tr_b16 %12, %22\n\t"
        "ds_read_b64_tr_b16 %13, %22 offset:4096\n\t"
        "ds_read_b64_tr_b16 %14, %23\n\t"
        "ds_read_b64_tr_b16 %15, %23 offset:4096\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(d[0][0]), "=&v"(d[0][1]), "=&v"(d[0][2]), "=&v"(d[0][3]), "=&v"(d[0][4]), "=&v"(d[0][5]),
          "=&v"(d[0][6]), "=&v"(d[0][7]), "=&v"(d[1][0]), "=&v"(d[1][1]), "=&v"(d[1][2]), "=&v"(d[1][3]),
          "=&v"(d[1][4]), "=&v"(d[1][5]), "=&v"(d[1][6]), "=&v"(d[1][7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
        : "memory");
}
__device__ __forceinline__ void raw_barrier() { asm volatile("s_barrier" ::: "memory"); }

// The prompt-chunk body for F16 pools, with the copy straight into LDS
// (buffer_load ... lds, 16 bytes per lane): no staging registers, so three
// work-groups fit a CU without spilling, or three LDS buffers keep the copy
// two stages ahead at two per CU.  The tiles sit in unpadded swizzled rows
// (k_swz, v_swz); the copy lane that fills a position loads the global chunk
// the swizzle puts there, and out-of-range lanes of a zero-size resource
// write zeros.  The arithmetic from the scores on and the epilogue are
// prefill_body_fp8's.
// SPLIT: 512 threads, two groups of four waves over the same 32 query rows,
// group 0 walking the first half of the piece's stages and group 1 the rest,
// each with its own LDS buffers; the groups pass the stage barriers together
// and merge their (max, sum, output) through LDS at the end.  A launch of
// few work-groups then keeps eight waves on each CU to the end of its
// longest tile instead of leaving one four-wave work-group alone on it.
template <int NB, bool SPLIT = false>
__device__ __forceinline__ void prefill_body_dma(const DecodeArgs &a, uint32_t bx) {
    static_assert(NB == 2 || NB == 3, "two or three LDS buffers");
    constexpr int kGroups = SPLIT ? 2 : 1;
    constexpr int kThreads = 256 * kGroups;
    const int g = static_cast<int>(bx % a.num_kv_heads);
    const int32_t *it = a.prefill_items + kPrefillItemInts * static_cast<size_t>(bx / a.num_kv_heads);
    const int tid = threadIdx.x;
    const int w8 = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave of the work-group
    const int grp = SPLIT ? w8 >> 2 : 0;                      // its group
    const int w = SPLIT ? w8 & 3 : w8;                        // its wave within the group
    const int lane = tid & 63;
    const int n = lane & 15, r = lane >> 4;

    __shared__ int tbl_lds[kMaxPrefillPieceBlocks];
    // unpadded rows; 16-byte chunk c of row t sits at chunk c ^ k_swz(t) (K)
    // or c ^ v_swz(t) (V); one set per group
    __shared__ __attribute__((aligned(16))) _Float16 k_lds_g[kGroups][NB][kStageBlocks][kBlockSize][kHeadDim];
    __shared__ __attribute__((aligned(16))) _Float16 v_lds_g[kGroups][NB][kStageBlocks][kBlockSize][kHeadDim];
    auto &k_lds = k_lds_g[grp];
    auto &v_lds = v_lds_g[grp];
    __shared__ float alpha_lds[kGroups * kWaves][2][16];
    __shared__ float m_lds[kGroups * kWaves][2][16];

    // Plan entries are clamped so a damaged plan cannot index outside q, out,
    // the tables, the pool or the workspace.
    const int s = min(max(it[0], 0), a.batch - 1);
    const int row0 = max(it[1], 0);
    const int n_q = min(max(it[2], 0), kPrefillTile);
    const int pos0 = max(it[3], 0);
    const int cap = a.max_blocks * kBlockSize;
    const int t_lo = min(max(it[4], 0), cap) & ~(kBlockSize - 1);
    const int t_hi = min(min(it[5], cap), pos0 + n_q);
    const int base_slot = it[6];
    const int np = max(it[7], 1);
    const int piece = min(max(it[8], 0), np - 1);
    const bool direct = base_slot < 0;
    if (!direct && a.num_slots <= 0) return;
    const int b_lo = t_lo / kBlockSize;
    const int b_hi = max(b_lo, min((t_hi + kBlockSize - 1) / kBlockSize, b_lo + kMaxPrefillPieceBlocks));

    const int32_t *table = a.tables + static_cast<size_t>(s) * a.max_blocks;
    for (int i = tid; i < b_hi - b_lo; i += kThreads) tbl_lds[i] = table[b_lo + i];
    __syncthreads();

    // this wave's query tokens and heads, and the keys its rows can see
    const int tok0 = 16 * (w >> 1);
    const int head0 = g * kGroup + 2 * (w & 1);
    const int rows_w = min(16, n_q - tok0);  // may be <= 0: the wave then only helps with the copies
    const int w_end = rows_w > 0 ? min(t_hi, pos0 + tok0 + rows_w) : t_lo;
    const int qp = pos0 + tok0 + n;  // position of row n

    // Q of the two row tiles, as the B operand of S^T: dims 32kk + 8r .. +7
    h8 qv[2][4];
    {
        const bool row_ok = n < rows_w;
        const size_t qr = static_cast<size_t>(min(max(row0 + tok0 + n, 0), a.num_q_rows - 1));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const uint16_t *qrow = a.q + (qr * a.num_q_heads + head0 + rt) * kHeadDim + 8 * r;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const h8 x = *reinterpret_cast<const h8 *>(qrow + 32 * kk);
                qv[rt][kk] = row_ok ? x : h8(0);
            }
        }
    }

    f4 oacc[2][8];
    f4 lacc[2];      // running sums, in oacc's layout: rows 4r + c (every column the same)
    float m_run[2];  // row n of each tile, log2 units
    // the weights' offset (-m_run, 0 while m_run = -inf) and m_run + kTau,
    // kept beside m_run instead of derived from it at each pair (the same
    // values either way); the threshold only where registers allow (three
    // buffers)
    constexpr bool kKeepThreshold = NB == 3;
    float thr[2], negm[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        m_run[rt] = -INFINITY;
        thr[rt] = -INFINITY;
        negm[rt] = 0.0f;
        lacc[rt] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) oacc[rt][j] = f4{0.f, 0.f, 0.f, 0.f};
    }
    const float c_scale = a.scale_log2e;
    const _Float16 one = static_cast<_Float16>(1.0f);
    h8 ones8 = {one, one, one, one, one, one, one, one};
    if constexpr (NB == 3) asm volatile("" : "+v"(ones8));  // held in registers, not rebuilt per pair

    // copies: wave w moves tensor w/2 (K, V) of block w%2 of the pair straight
    // into LDS, 1 KiB per load instruction: lane l fills chunk l%16 of row
    // 4i + l/16 with the global chunk that the swizzle puts there
    const uint32_t last_block = static_cast<uint32_t>(a.num_blocks - 1);
    const size_t tile_bytes = tile_elems() * sizeof(uint16_t);
    constexpr int kCopyBlocks = kStageBlocks / 2;
    constexpr int kLoads = 4;
    const int cp_tensor = w >> 1, cp_blk0 = (w & 1) * kCopyBlocks;
    const char *cp_layer = cp_tensor ? a.v_layer : a.k_layer;
    uint32_t cp_off[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int row = 4 * i + (lane >> 4), pos = lane & 15;
        const int c = pos ^ (cp_tensor ? v_swz(row) : k_swz(row));
        cp_off[i] = static_cast<uint32_t>(row * (kHeadDim * 2) + 16 * c);
    }
    auto fetch = [&](int b, int buf) {  // stage starting at block b, into LDS buffer buf
#pragma unroll
        for (int x = 0; x < kCopyBlocks; ++x) {
            const int bb = b + cp_blk0 + x;
            const bool live = bb < b_hi;
            uint32_t phys = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(tbl_lds[live ? bb - b_lo : 0]));
            phys = phys > last_block ? last_block : phys;
            const size_t base = (static_cast<size_t>(phys) * a.num_kv_heads + g) * tile_bytes;
            // a live block holds at least one key (bb < b_hi), so only the
            // upper clamp is needed for its value rows
            const int rows = cp_tensor ? min(t_hi - bb * kBlockSize, kBlockSize) : kBlockSize;
            const int bytes = live ? rows * kHeadDim * 2 : 0;
            const __amdgpu_buffer_rsrc_t rs = tile_rsrc(cp_layer + base, bytes);
            _Float16 *tile = cp_tensor ? &v_lds[buf][cp_blk0 + x][0][0] : &k_lds[buf][cp_blk0 + x][0][0];
#pragma unroll
            for (int i = 0; i < kLoads; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void *)(tile + 4 * i * kHeadDim), 16, cp_off[i], 0, 0, 0);
        }
    };

    // transpose reads: lane l addresses token 4(l/16) + (l/4)%4, dims 4(l%4) .. +3
    // of a 16-dim slice, so that lane (r, n) receives tokens 4r .. 4r+3 at dim n
    const int tr_row = 4 * r + ((lane >> 2) & 3), tr_col = 4 * (lane & 3);
    const int tr_swz = v_swz(tr_row);
    auto compute = [&](int buf, int sb, int b) {  // blocks sb, sb+1 of the stage = key blocks b, b+1
        // the pair's K operands, read once for both row tiles
        h8 kx[2][4];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                kx[blk][kk] = *reinterpret_cast<const h8 *>(&k_lds[buf][sb + blk][n][8 * ((4 * kk + r) ^ k_swz(n))]);
        // the value operands of P V over dims 16j .. 16j+15: lane (r, n) gets
        // tokens 4r .. 4r+3 of each block at dim 16j + n straight from the
        // transpose reads.  With three buffers (registers to spare) they are
        // read here, behind the key reads, so that one wait covers both (a
        // 2016-token chunk at position 2016 about 1.5 % faster); else just
        // before P V.
        u2 t[2][8];  // [half][4 j's x 2 blocks]
        if constexpr (NB == 3) {
            uint32_t ad[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                ad[j] = lds_addr(&v_lds[buf][sb][tr_row][8 * ((2 * j + (tr_col >> 3)) ^ tr_swz) + (tr_col & 7)]);
            lds_read_tr16_x16(t, ad);
        }
        f4 st[2][2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) st[rt][blk] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
                    st[rt][blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kx[blk][kk], qv[rt][kk], st[rt][blk], 0, 0, 0);
        // masks, only where the pair reaches past the first row's position or
        // the last key this wave sees
        const int k_last = b * kBlockSize + 2 * kBlockSize - 1;
        const bool tail = k_last >= w_end;
        if (k_last > pos0 + tok0 || tail) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int kp = (b + blk) * kBlockSize + 4 * r + c;
                    const bool vis = kp < w_end && kp <= qp;
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) st[rt][blk][c] = vis ? st[rt][blk][c] : -INFINITY;
                }
        }
        h8 pw[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const float m1 = max3_raw(st[rt][0][0], st[rt][0][1], st[rt][0][2]);
            const float m2 = max3_raw(st[rt][0][3], st[rt][1][0], st[rt][1][1]);
            const float m3 = max3_raw(st[rt][1][2], st[rt][1][3], m1);
            const float bmax = max3_raw(m2, m3, m3);
            const float mb = bmax * c_scale;
            if (__builtin_amdgcn_ballot_w64(mb > (kKeepThreshold ? thr[rt] : m_run[rt] + kTau)) != 0) {
                float bm = mb;
                bm = fmaxf(bm, shfl_xor(bm, 16));
                bm = fmaxf(bm, shfl_xor(bm, 32));
                const float m_new = fmaxf(m_run[rt], bm);
                // a row that has seen no key yet keeps m = -inf (and alpha 1)
                const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m_run[rt] - m_new);
                m_run[rt] = m_new;
                thr[rt] = m_new + kTau;
                negm[rt] = m_new == -INFINITY ? 0.0f : -m_new;
                if (r == 0) alpha_lds[w8][rt][n] = alpha;
                wave_lds_sync();
                const float4 al = *reinterpret_cast<const float4 *>(&alpha_lds[w8][rt][4 * r]);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    oacc[rt][j][0] *= al.x;
                    oacc[rt][j][1] *= al.y;
                    oacc[rt][j][2] *= al.z;
                    oacc[rt][j][3] *= al.w;
                }
                lacc[rt][0] *= al.x;
                lacc[rt][1] *= al.y;
                lacc[rt][2] *= al.z;
                lacc[rt][3] *= al.w;
            }
            // weights exp2(s * scale - m) enter P V as F16, and the running
            // sums (one more MFMA, below) add the same rounded values (masked
            // scores give exp2(-inf) = 0)
            const float neg_m = negm[rt];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int c = 0; c < 4; c += 2) {
                    const float p0 = fast_exp2(fmaf(st[rt][blk][c], c_scale, neg_m));
                    const float p1 = fast_exp2(fmaf(st[rt][blk][c + 1], c_scale, neg_m));
                    const h2 pp = {static_cast<_Float16>(p0), static_cast<_Float16>(p1)};
                    pw[rt][4 * blk + c] = pp.x;
                    pw[rt][4 * blk + c + 1] = pp.y;
                }
        }
        if constexpr (NB != 3) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                uint32_t ad[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int j = 4 * hf + (q >> 1), blk = q & 1;
                    ad[q] = lds_addr(
                        &v_lds[buf][sb + blk][tr_row][8 * ((2 * j + (tr_col >> 3)) ^ tr_swz) + (tr_col & 7)]);
                }
                lds_read_tr16_x8(t[hf], ad);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const h4 t0 = __builtin_bit_cast(h4, t[j >> 2][2 * (j & 3)]);
            const h4 t1 = __builtin_bit_cast(h4, t[j >> 2][2 * (j & 3) + 1]);
            const h8 bv = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                oacc[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pw[rt], bv, oacc[rt][j], 0, 0, 0);
        }
        // the row sums of the same F16 weights, on the matrix cores
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) lacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pw[rt], ones8, lacc[rt], 0, 0, 0);
    };

    // the work-group walks every pair of the piece (SPLIT: this group its half
    // of the stages); a wave computes the pairs below its last query's position
    const int n_stages = (b_hi - b_lo + kStageBlocks - 1) / kStageBlocks;
    const int w_blocks = w_end > t_lo ? (w_end + kBlockSize - 1) / kBlockSize - b_lo : 0;  // blocks this wave needs
    const int half = (n_stages + 1) / 2;
    const int my_first = SPLIT && grp ? half : 0;                            // first stage of this group
    const int my_count = SPLIT ? (grp ? n_stages - half : half) : n_stages;  // its stages
    const int rounds = SPLIT ? half : n_stages;  // barrier rounds, the same for both groups
    // this group's stage st reads its LDS buffer st % NB; its loads were
    // issued NB - 1 stages earlier.  Each stage issues kLoads * kCopyBlocks
    // loads per wave.
    constexpr int kAhead = NB - 1;
    constexpr int kStageLoads = kLoads * kCopyBlocks;
#pragma unroll
    for (int s0 = 0; s0 < kAhead; ++s0)
        if (s0 < my_count) fetch(b_lo + (my_first + s0) * kStageBlocks, s0);
    if (rounds > 0) {
        if (kAhead > 1 && my_count > 1) __builtin_amdgcn_s_waitcnt(0x0F70 | (kStageLoads * (kAhead - 1)));
        else __builtin_amdgcn_s_waitcnt(0x0F70);
        raw_barrier();
    }
    auto stage = [&](int st, auto bufc) {
        constexpr int B = decltype(bufc)::value;  // == st % NB
        const int gst = my_first + st;            // the stage within the piece
        const int b0 = b_lo + kStageBlocks * gst;
        const bool more = st + kAhead < my_count;
        if (more) fetch(b0 + kAhead * kStageBlocks, (B + kAhead) % NB);
        if (!SPLIT || st < my_count) {
#pragma unroll
            for (int sb = 0; sb < kStageBlocks; sb += 2)
                if (kStageBlocks * gst + sb < w_blocks) compute(B, sb, b0 + sb);
        }
        // stage st+1's loads must have landed: all but those of later stages
        if (kAhead > 1 && more) __builtin_amdgcn_s_waitcnt(0x0F70 | (kStageLoads * (kAhead - 1)));
        else __builtin_amdgcn_s_waitcnt(0x0F70);
        raw_barrier();
    };
    for (int st = 0; st < rounds; st += NB) {
        stage(st, std::integral_constant<int, 0>{});
        if (st + 1 < rounds) stage(st + 1, std::integral_constant<int, 1>{});
        if constexpr (NB == 3)
            if (st + 2 < rounds) stage(st + 2, std::integral_constant<int, 2 % NB>{});
    }
    if constexpr (SPLIT) {
        // group 1 hands its max, sums and outputs to group 0 through LDS (the
        // key stage buffers are free after the last barrier), one row tile at
        // a time: per lane (r, n) 32 output values, then 4 sums
        float *mrg = reinterpret_cast<float *>(&k_lds_g[0][0][0][0][0]);  // [wave][36][64]
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
            if (r == 0) m_lds[w8][rt][n] = m_run[rt];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            if (grp == 1) {
                float *dst = mrg + w * 36 * 64 + lane;
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) dst[(j * 4 + c) * 64] = oacc[rt][j][c];
#pragma unroll
                for (int c = 0; c < 4; ++c) dst[(32 + c) * 64] = lacc[rt][c];
            }
            __syncthreads();
            if (grp == 0 && rows_w > 0) {
                const float *src = mrg + w * 36 * 64 + lane;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int t = 4 * r + c;
                    const float m0 = m_lds[w][rt][t], m1 = m_lds[4 + w][rt][t];
                    const float M = fmaxf(m0, m1);
                    const float a0 = m0 == -INFINITY ? 0.0f : fast_exp2(m0 - M);
                    const float a1 = m1 == -INFINITY ? 0.0f : fast_exp2(m1 - M);
#pragma unroll
                    for (int j = 0; j < 8; ++j) oacc[rt][j][c] = a0 * oacc[rt][j][c] + a1 * src[(j * 4 + c) * 64];
                    lacc[rt][c] = a0 * lacc[rt][c] + a1 * src[(32 + c) * 64];
                }
            }
            __syncthreads();
        }
        if (grp == 1) return;
        // the merged max of row n, which the records below carry
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) m_run[rt] = fmaxf(m_run[rt], m_lds[4 + w][rt][n]);
    }
    if (rows_w <= 0) return;

    // m of every row to LDS; lane l then writes rows 4r + c of each tile
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
        if (r == 0) m_lds[w][rt][n] = m_run[rt];
    wave_lds_sync();
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int head = head0 + rt;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int t = 4 * r + c;  // row of the tile
            if (t >= rows_w) continue;
            const int tok = tok0 + t;
            const float m = m_lds[w][rt][t], l = lacc[rt][c];
            if (direct) {
                const size_t qrow = static_cast<size_t>(min(row0 + tok, a.num_q_rows - 1));
                const float inv = 1.0f / l;
                _Float16 *orow = reinterpret_cast<_Float16 *>(a.out + (qrow * a.num_q_heads + head) * kHeadDim);
#pragma unroll
                for (int j = 0; j < 8; ++j) orow[16 * j + n] = static_cast<_Float16>(oacc[rt][j][c] * inv);  // dim 16j + n
            } else {
                const int64_t slot64 = static_cast<int64_t>(base_slot) + static_cast<int64_t>(tok) * np + piece;
                const size_t slot = static_cast<size_t>(min<int64_t>(slot64, a.num_slots - 1));
                const size_t rec = slot * a.num_q_heads + head;
#pragma unroll
                for (int j = 0; j < 8; ++j) a.o_part[rec * kHeadDim + 16 * j + n] = oacc[rt][j][c];
                if (n == 0) *reinterpret_cast<float2 *>(a.ml_part + rec * 2) = make_float2(m, l);
            }
        }
    }
}


// FP8 pools: codes are widened on their way into LDS, so the copy goes
// through registers, one stage ahead, three work-groups per CU (160 VGPRs).
template <bool FP8, int WGS>
__global__ __launch_bounds__(256, WGS) void prefill_kernel(DecodeArgs a) {
    static_assert(FP8 && WGS == 3, "F16 pools take prefill_dma_kernel");
    prefill_body_fp8(a, blockIdx.x);
}

// FP8 prompt-chunk launches of at most one four-wave work-group per CU: the
// split body, eight waves, one work-group per CU.
__global__ __launch_bounds__(512, 1) void prefill_fp8_split_kernel(DecodeArgs a) {
    prefill_body_fp8<true>(a, blockIdx.x);
}

// F16 pools: the copy goes straight to LDS, NB - 1 stages ahead; WGS
// work-groups per CU.  launch_prefill chooses.
template <int NB, int WGS>
__global__ __launch_bounds__(256, WGS) void prefill_dma_kernel(DecodeArgs a) {
    prefill_body_dma<NB>(a, blockIdx.x);
}

// F16 prompt-chunk launches of at most one four-wave work-group per CU:
// eight waves, the keys of each piece split between two groups of four, one
// work-group per CU.
__global__ __launch_bounds__(512, 1) void prefill_dma_split_kernel(DecodeArgs a) {
    prefill_body_dma<3, true>(a, blockIdx.x);
}

// A mixed step's decode and prefill pieces in one launch, three work-groups
// per CU: the decode pieces keep two blocks in flight instead of three (158
// VGPRs on their own) and are walked by a.mixed_decode_waves of the four
// waves, the F16 prefill pieces copy straight to LDS one stage ahead, the FP8
// ones through registers.
template <bool FP8>
__global__ __launch_bounds__(256, 3) void mixed_kernel(DecodeArgs a) {
    const uint32_t nd = static_cast<uint32_t>(a.num_items) * static_cast<uint32_t>(a.num_kv_heads);
    if (blockIdx.x < nd) {
        decode_partial_body<2, FP8, true>(a, blockIdx.x, 0, 0);
    } else {
        // the prompt tiles' waves issue ahead of the decode streams that
        // share their SIMDs (wave priority 1 against 0)
        __builtin_amdgcn_s_setprio(1);
        if constexpr (FP8)
            prefill_body_fp8(a, blockIdx.x - nd);
        else
            prefill_body_dma<2>(a, blockIdx.x - nd);
    }
}

}  // namespace

namespace {
// One round: every prefill work-group of the launch fits two per CU.
// Measured on MI355X (256 CUs), F16 pools, per layer:
//  - a 2016-token chunk at position 2016 (504 work-groups, one round): three
//    LDS buffers at two work-groups per CU 117.3-118.2 us, one-stage-ahead
//    copies at three per CU 122.3-122.5 us, register staging two stages
//    ahead at two per CU 121.6-122.5 us;
//  - a 16,384-token chunk at position 16,352 (4,088 work-groups): two LDS
//    buffers at three per CU 6.85 ms, three buffers 6.90 ms, register staging
//    at three per CU 7.07 ms.  Past one round the third slot keeps a CU busy
//    while its tiles finish unevenly.
constexpr int64_t kPrefillRoundGroups = 2 * 256;
// Prompt-chunk launches of at most one four-wave work-group per CU run the
// split kernel instead: the 32 tiles of a 1,024-token chunk at position 3,008
// (256 work-groups) took 96.2 us against 116-122 us.  At two per CU the
// four-wave work-groups are faster: two such chunks (512) 141-148 us against
// 164 us, a 2,016-token chunk at position 2,016 (504) 137.8-142.1 against
// 145.5-146.5.
constexpr int64_t kPrefillSplitGroups = 256;
bool prefill_one_round(const DecodeArgs &a) {
    return static_cast<int64_t>(a.num_prefill_items) * a.num_kv_heads <= kPrefillRoundGroups;
}
}  // namespace

// Mixed steps: F16 16,384-token step 55.7 against 57.0 ms with register
// staging; the 2016-token step 6.35-6.36 against 6.39-6.40 ms.
hipError_t launch_mixed(const DecodeArgs &a, hipStream_t stream) {
    const uint32_t groups =
        static_cast<uint32_t>((static_cast<int64_t>(a.num_items) + a.num_prefill_items) * a.num_kv_heads);
    if (a.elem_bytes == 1)
        hipLaunchKernelGGL(mixed_kernel<true>, dim3(groups), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(mixed_kernel<false>, dim3(groups), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_write_kv(const WriteKvArgs &a, hipStream_t stream) {
    const int64_t total = static_cast<int64_t>(a.n_tokens) * a.num_kv_heads * (kHeadDim / 8);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(write_kv_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_partial(const DecodeArgs &a, hipStream_t stream) {
    if (a.items && a.decode_wave_heads) {  // four KV heads per work-group, one per wave
        const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(a.num_items) * (a.num_kv_heads / kWaves)), 1, 1);
        if (a.elem_bytes == 1)
            hipLaunchKernelGGL((decode_wave_heads_kernel<true>), grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((decode_wave_heads_kernel<false>), grid, dim3(256), 0, stream, a);
        return hipGetLastError();
    }
    const dim3 grid = a.items ? dim3(static_cast<uint32_t>(static_cast<int64_t>(a.num_items) * a.num_kv_heads), 1, 1)
                              : dim3(a.max_splits, a.num_kv_heads, a.batch);
    if (a.elem_bytes == 1)
        hipLaunchKernelGGL((decode_partial_kernel<PA_DECODE_NBUF_FP8, true>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_partial_kernel<PA_DECODE_NBUF, false>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs &a, hipStream_t stream) {
    const int64_t rows = static_cast<int64_t>(a.batch) * a.num_q_heads;
    hipLaunchKernelGGL(decode_merge_kernel, dim3(static_cast<uint32_t>((rows + 1) / 2)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_merge_planned(const DecodeArgs &a, hipStream_t stream) {
    // about 2,048 or more work-groups either way: a 32-head step's 8 merges
    // take 128 of two heads; a prompt chunk's 8,000 take 16,000 of 16
    if (a.num_merges >= 2048)
        hipLaunchKernelGGL(decode_merge_planned_kernel<16>, dim3(a.num_merges, (a.num_q_heads + 15) / 16), dim3(256), 0,
                           stream, a);
    else if (a.num_merges >= 512)
        hipLaunchKernelGGL(decode_merge_planned_kernel<8>, dim3(a.num_merges, (a.num_q_heads + 7) / 8), dim3(256), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(decode_merge_planned_kernel<2>, dim3(a.num_merges, (a.num_q_heads + 1) / 2), dim3(256), 0,
                           stream, a);
    return hipGetLastError();
}

hipError_t launch_prefill(const DecodeArgs &a, hipStream_t stream) {
    const uint32_t groups = static_cast<uint32_t>(static_cast<int64_t>(a.num_prefill_items) * a.num_kv_heads);
    if (a.elem_bytes == 1 && groups <= kPrefillSplitGroups)
        hipLaunchKernelGGL(prefill_fp8_split_kernel, dim3(groups), dim3(512), 0, stream, a);
    else if (a.elem_bytes == 1)
        hipLaunchKernelGGL((prefill_kernel<true, 3>), dim3(groups), dim3(256), 0, stream, a);
    else if (groups <= kPrefillSplitGroups)
        hipLaunchKernelGGL(prefill_dma_split_kernel, dim3(groups), dim3(512), 0, stream, a);
    else if (prefill_one_round(a))
        hipLaunchKernelGGL((prefill_dma_kernel<3, 2>), dim3(groups), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((prefill_dma_kernel<2, 3>), dim3(groups), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_cascade(const DecodeArgs &a, hipStream_t stream) {
    const uint32_t groups =
        static_cast<uint32_t>((static_cast<int64_t>(a.num_items) + a.num_prefix_items) * a.num_kv_heads);
    if (a.elem_bytes == 1)
        hipLaunchKernelGGL(cascade_kernel<true>, dim3(groups), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(cascade_kernel<false>, dim3(groups), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// ---- scratch of the allocation-free decode ---------------------------------
// pa_decode_noalloc keeps its split partials here instead of in a caller's
// workspace, for callers that cannot allocate.  Each GPU holds its own copy at
// its own address until the process ends.  In host code `scratch` is only a
// stand-in for the symbol: its device address comes from hipGetSymbolAddress,
// once per device, and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(hipStream_t stream, void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        // the lookup runs with the stream's device current
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_decode_prefix(const DecodeArgs &a, hipStream_t stream) {
    const uint32_t groups = static_cast<uint32_t>(static_cast<int64_t>(a.num_prefix_items) * a.num_kv_heads);
    if (a.elem_bytes == 1)
        hipLaunchKernelGGL(decode_prefix_kernel<true>, dim3(groups), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(decode_prefix_kernel<false>, dim3(groups), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pa
