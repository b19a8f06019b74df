// pa_api.cpp -- the C ABI declared in include/pa.h: argument checks, the
// split plan, workspace sizing and kernel launches.  No entry point throws,
// allocates device memory, or synchronises.

#include "pa.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <functional>
#include <new>
#include <queue>
#include <vector>

#include "pa_internal.h"

#ifndef PA_SOURCE_SHA256
#define PA_SOURCE_SHA256 "unknown"
#endif
// A sha256 of the sources and flags this library was built from (computed by
// the build script); the Python loader reads it from the file to refuse a
// stale build.  Nothing calls it.
extern "C" __attribute__((used, visibility("default"))) const char pa_build_source[] =
    "pa-source-sha256:" PA_SOURCE_SHA256;

struct pa_pool {
    pa_pool_desc desc;
    void *k;
    void *v;
    std::vector<float> k_scale;  // per layer (FP8 pools); 1 until set
    std::vector<float> v_scale;
    int32_t elem_bytes() const { return desc.dtype == PA_FP8_E4M3 ? 1 : 2; }
    size_t layer_offset(int32_t layer) const {
        return static_cast<size_t>(layer) * pa::layer_bytes(desc.num_blocks, desc.num_kv_heads, elem_bytes());
    }
};

namespace {

using pa::kBlockSize;
using pa::kGroup;
using pa::kHeadDim;
using pa::kMaxSplitTokens;
using pa::kSplitQuantum;

// Work-groups the split plan aims for: one per compute unit of MI355X (256).
// Longer splits keep each wave's load pipeline full for longer and avoid the
// merge; measured on the 8B geometry, splits that give about one
// work-group per unit were the fastest at batch 1, 8 and 32.
constexpr int64_t kTargetWorkGroups = 256;
// Shortest planned piece: 4 blocks per wave.  Small batches do not fill the
// chip anyway, and there each work-group's fixed latency (q, table, the
// four-wave merge) and the extra merge launch outweigh spreading the blocks
// thinner: batch 1 over 32 layers took 9.4 / 12.5 / 14.8 us per layer at
// contexts 256 / 1024 / 2048 with this minimum, against 13.0 / 17.6 / 25.5 us
// with one block per wave.
constexpr int64_t kMinPieceBlocks = 4 * pa::kWaves;

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool desc_ok(const pa_pool_desc *d) {
    return d && d->num_layers > 0 && d->num_blocks > 0 && d->block_size > 0 && d->num_kv_heads > 0 &&
           d->head_dim > 0;
}

bool desc_supported(const pa_pool_desc *d) {
    return d->block_size == kBlockSize && d->head_dim == kHeadDim && (d->dtype == PA_F16 || d->dtype == PA_FP8_E4M3);
}

float inv_scale(float s) { return static_cast<float>(1.0 / static_cast<double>(s)); }

void set_scales(const pa_pool *pool, int32_t layer, pa::DecodeArgs *a) {
    const float ks = pool->k_scale[layer], vs = pool->v_scale[layer];
    a->elem_bytes = pool->elem_bytes();
    a->v_scale = vs;
    a->inv_k_scale = inv_scale(ks);
    a->inv_v_scale = inv_scale(vs);
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Split length in tokens for a launch shape (see pa_decode_split_tokens).
int32_t plan_split(int32_t batch, int32_t num_kv_heads, int32_t max_ctx) {
    if (const char *env = std::getenv("PA_SPLIT_TOKENS")) {
        char *end = nullptr;
        const long v = std::strtol(env, &end, 10);
        if (end != env && v > 0 && v % kSplitQuantum == 0 && v <= kMaxSplitTokens) return static_cast<int32_t>(v);
    }
    if (max_ctx <= 0) return kSplitQuantum;
    const int64_t pairs = static_cast<int64_t>(batch) * num_kv_heads;
    const int64_t splits = std::max<int64_t>(1, (kTargetWorkGroups + pairs - 1) / pairs);
    const int64_t per = (max_ctx + splits - 1) / splits;
    // at least 4 blocks per wave, as for planned pieces (kMinPieceBlocks)
    const int64_t tokens = std::max<int64_t>(kMinPieceBlocks * kBlockSize, round_up(per, kSplitQuantum));
    return static_cast<int32_t>(std::min<int64_t>(tokens, kMaxSplitTokens));
}

struct Plan {
    int32_t split_tokens;
    int32_t max_splits;
    size_t workspace;  // bytes; 0 for single-split launches
    size_t o_bytes;    // offset of the (m, l) array inside the workspace
};

Plan make_plan(const pa_pool *pool, int32_t batch, int32_t num_q_heads, int32_t max_ctx) {
    Plan p{};
    p.split_tokens = plan_split(batch, pool->desc.num_kv_heads, max_ctx);
    p.max_splits = max_ctx <= 0 ? 1 : static_cast<int32_t>((max_ctx + p.split_tokens - 1) / p.split_tokens);
    if (p.max_splits > 1) {
        const size_t rows = static_cast<size_t>(batch) * num_q_heads * p.max_splits;
        p.o_bytes = round_up(static_cast<int64_t>(rows * kHeadDim * sizeof(float)), 256);
        p.workspace = p.o_bytes + rows * 2 * sizeof(float);
    }
    return p;
}

// Checks shared by every decode entry point.
pa_status check_decode_shape(const pa_pool *pool, int32_t batch, int32_t num_q_heads, int32_t max_blocks,
                             int32_t max_ctx) {
    if (!pool) return PA_ERR_INVALID_ARG;
    if (batch < 0 || num_q_heads <= 0 || max_blocks < 0 || max_ctx < 0) return PA_ERR_INVALID_ARG;
    if (num_q_heads % pool->desc.num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    if (static_cast<int64_t>(max_ctx) > static_cast<int64_t>(max_blocks) * pool->desc.block_size)
        return PA_ERR_INVALID_ARG;
    if (num_q_heads != kGroup * pool->desc.num_kv_heads) return PA_ERR_UNSUPPORTED;
    if (max_ctx > pa::kMaxContextTokens || max_blocks > pa::kMaxContextTokens / kBlockSize) return PA_ERR_UNSUPPORTED;
    if (batch > 65535 || pool->desc.num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

pa_status fill_decode_args(pa_pool *pool, int32_t layer, const void *q, const void *k_new, const void *v_new,
                           void *out, const int32_t *tables,
                           int32_t max_blocks, const int32_t *ctx_lens, int32_t batch, int32_t num_q_heads,
                           int32_t max_ctx, float scale, void *ws, size_t ws_bytes, pa::DecodeArgs *a,
                           Plan *plan_out) {
    pa_status st = check_decode_shape(pool, batch, num_q_heads, max_blocks, max_ctx);
    if (st != PA_OK) return st;
    if (layer < 0 || layer >= pool->desc.num_layers) return PA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
    if (batch == 0) {
        *plan_out = Plan{};
        return PA_OK;
    }
    if (!q || !out || !ctx_lens || (max_ctx > 0 && !tables)) return PA_ERR_INVALID_ARG;
    if ((k_new == nullptr) != (v_new == nullptr)) return PA_ERR_INVALID_ARG;
    if (k_new && (!aligned(k_new, 16) || !aligned(v_new, 16))) return PA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(tables, 4) || !aligned(ctx_lens, 4))
        return PA_ERR_INVALID_ARG;
    const Plan plan = make_plan(pool, batch, num_q_heads, max_ctx);
    if (plan.workspace > 0) {
        if (!ws || ws_bytes < plan.workspace) return PA_ERR_WORKSPACE;
        if (!aligned(ws, 256)) return PA_ERR_INVALID_ARG;
    }
    a->k_layer = static_cast<const char *>(pool->k) + pool->layer_offset(layer);
    a->v_layer = static_cast<const char *>(pool->v) + pool->layer_offset(layer);
    set_scales(pool, layer, a);
    a->q = static_cast<const uint16_t *>(q);
    a->k_new = static_cast<const uint16_t *>(k_new);
    a->v_new = static_cast<const uint16_t *>(v_new);
    a->tables = tables;
    a->ctx_lens = ctx_lens;
    a->out = static_cast<uint16_t *>(out);
    a->o_part = plan.workspace ? static_cast<float *>(ws) : nullptr;
    a->ml_part = plan.workspace ? reinterpret_cast<float *>(static_cast<char *>(ws) + plan.o_bytes) : nullptr;
    a->batch = batch;
    a->num_q_rows = batch;
    a->num_q_heads = num_q_heads;
    a->num_kv_heads = pool->desc.num_kv_heads;
    a->num_blocks = pool->desc.num_blocks;
    a->max_blocks = max_blocks;
    a->max_ctx = max_ctx;
    a->split_tokens = plan.split_tokens;
    a->max_splits = plan.max_splits;
    a->scale_log2e = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634 *
                                        (pool->elem_bytes() == 1 ? pool->k_scale[layer] : 1.0f));
    *plan_out = plan;
    return PA_OK;
}

// ---- host-side schedule for pa_decode_plan / pa_decode_run --------------
// Pieces are cut so that about kTargetWorkGroups work-groups do near-equal
// work: M = ceil(total_blocks / (kTargetWorkGroups / Hkv)) blocks per piece,
// clamped to [kWaves, kMaxSplitTokens / kBlockSize]; a sequence of n blocks
// becomes ceil(n / M) pieces of near-equal length, and the pieces are
// dispatched longest first.
struct PlanItem {
    int32_t s, t_begin, t_end, ctx, slot;
};

// ---- piece size by a model of the dispatch ----------------------------------
// Measured on MI355X: a compute unit pulls K/V at about 26 GB/s however few
// others are busy, so a decode launch lasts as long as its most loaded unit.
// The dispatcher hands work-group j of a launch to unit j mod 256 while each
// unit has room for two (j < 512), and each later one to the unit that frees
// a slot first.  The model charges a unit the blocks of every work-group it
// gets, plus kWgOverheadBlocks each for the work-group's fixed work (query,
// table, the four-wave merge), and a plan that cuts a sequence one launch of
// the merge kernel (kMergeBlocks of F16 blocks: about 5 us at that rate).
// Measured against it, per layer: batch 8 / 16 / 24 / 32 at 4096 tokens took
// 29 / 50 / 86 / 82 us, modelled 26 / 46 / 88 / 82 us; the ragged 64-sequence
// step 185 us, modelled 186 us.
constexpr int kDispatchUnits = 256;
constexpr int kSlotsPerUnit = 2;
constexpr int64_t kWgOverheadBlocks = 3;
constexpr int64_t kMergeBlocks = 16;
// Per-wave KV heads (decode_wave_heads): each wave walks a whole piece for
// its own KV head, so a work-group's fixed work (query, table, pipeline
// start, epilogue) is spread over four times the blocks and no partial sums
// cross waves, at three work-groups per unit.  Pieces are then at most one
// table register of blocks.  A work-group moves four times the blocks, so a
// launch of few of them balances worse; the dispatch model above decides,
// and the mode is taken when it models more than 1/64 faster.  Measured
// (one-layer cold decodes, the newest token appended, F16 us, four-wave
// split -> wave heads), every case as the model chose: 4096 x 32 tokens
// 272 -> 126, 2048 x 64 178 -> 114, 128 x 1024 88.4 -> 83.3; kept split:
// 160 x 1024 111 (wave heads 139), 150 x 512 57.6 (72.0), 40 x 4096 cut in
// four 112 (142), 200 x 1024 146.4 (147.0), 300 x 512 115.6 (115.5).
constexpr int kWaveHeadsMaxBlocks = 64;
constexpr int kWaveHeadsSlots = 3;

// Blocks of each piece when every context is cut into near-equal pieces of
// at most max_piece blocks (an empty context gives an empty piece), longest
// first (a counting sort: pieces are at most kMaxSplitTokens / kBlockSize
// blocks).
void piece_blocks(const int32_t *lens, const std::vector<int32_t> &plen, int32_t batch, int64_t max_piece,
                  std::vector<int64_t> *out, bool *cuts) {
    constexpr int64_t kMaxPiece = kMaxSplitTokens / kBlockSize;
    std::vector<int64_t> count(kMaxPiece + 1, 0);
    *cuts = false;
    for (int32_t s = 0; s < batch; ++s) {
        const int64_t nb = (static_cast<int64_t>(lens[s]) - plen[s] + kBlockSize - 1) / kBlockSize;
        if (nb == 0) {
            if (plen[s] == 0) ++count[0];
            continue;
        }
        const int64_t np = (nb + max_piece - 1) / max_piece;
        *cuts = *cuts || np > 1;
        // near-equal: nb % np pieces one block longer (never past max_piece)
        if (nb % np != 0) count[nb / np + 1] += nb % np;
        count[nb / np] += np - nb % np;
    }
    out->clear();
    for (int64_t b = kMaxPiece; b >= 0; --b) out->insert(out->end(), static_cast<size_t>(count[b]), b);
}

// The modelled time of a launch of these pieces, longest first, each run by
// `heads` consecutive work-groups, in blocks of the most loaded unit.  When
// `heads` divides the unit count, a piece's work-groups land on `heads`
// units whose loads stay equal, so the model tracks groups of units.
// `slots` work-groups fit a unit at once, and a work-group moves `scale` times
// its piece's blocks (scale 4 when each of its waves takes its own KV head).
int64_t modelled_makespan(const std::vector<int64_t> &pieces, int32_t heads, int slots = kSlotsPerUnit,
                          int64_t scale = 1) {
    const bool grouped = heads > 0 && kDispatchUnits % heads == 0;
    const int units = grouped ? kDispatchUnits / heads : kDispatchUnits;  // tracked units (or groups)
    const int per = grouped ? 1 : heads;                                  // work-groups per piece and unit
    const int64_t first_round = static_cast<int64_t>(units) * slots;
    std::vector<int64_t> load(units, 0);
    std::priority_queue<std::pair<int64_t, int>, std::vector<std::pair<int64_t, int>>, std::greater<>> later;
    int64_t j = 0;
    for (const int64_t p : pieces) {
        for (int h = 0; h < per; ++h, ++j) {
            const int64_t w = p * scale + kWgOverheadBlocks;
            if (j < first_round) {
                load[j % units] += w;
                if (j + 1 == first_round)
                    for (int u = 0; u < units; ++u) later.push({load[u], u});
            } else {
                const int u = later.top().second;
                later.pop();
                load[u] += w;
                later.push({load[u], u});
            }
        }
    }
    return *std::max_element(load.begin(), load.end());
}

// Piece size (in blocks) from a ladder of candidates, largest first, from
// kMaxSplitTokens / kBlockSize down to kMinPieceBlocks: a smaller piece is
// taken only when its modelled launch time beats the best so far by more
// than 1/32 (3 %).  The model knows nothing of tiles that several sequences
// share and the caches serve (the 256-sequence shared-prefix step took 808 us
// with 256-block pieces and 834 us with the 128-block pieces the model rated
// 2 % faster), so small modelled gains do not change the plan.
// merge_blocks: the charge for a plan that cuts a sequence.  A candidate
// whose lower bound (its work spread evenly, or its longest piece) cannot
// beat the best so far is not simulated.
int64_t balanced_piece(const int32_t *lens, const std::vector<int32_t> &plen, int32_t batch, int32_t heads,
                       int64_t merge_blocks) {
    static const int64_t kLadder[] = {256, 224, 192, 160, 128, 112, 96, 80, 64, 56, 48, 40, 32, 28, 24, 20, 16};
    const bool grouped = heads > 0 && kDispatchUnits % heads == 0;
    const int64_t units = grouped ? kDispatchUnits / heads : kDispatchUnits;
    const int64_t per = grouped ? 1 : heads;
    int64_t best = kMaxSplitTokens / kBlockSize, best_cost = -1;
    std::vector<int64_t> pieces;
    for (const int64_t p : kLadder) {
        if (p < kMinPieceBlocks || p > kMaxSplitTokens / kBlockSize) continue;
        bool cuts = false;
        piece_blocks(lens, plen, batch, p, &pieces, &cuts);
        int64_t work = 0;
        for (const int64_t b : pieces) work += (b + kWgOverheadBlocks) * per;
        const int64_t bound = std::max<int64_t>((work + units - 1) / units,
                                                pieces.empty() ? 0 : pieces[0] + kWgOverheadBlocks) +
                              (cuts ? merge_blocks : 0);
        if (best_cost >= 0 && bound >= best_cost - best_cost / 32) continue;
        const int64_t cost = modelled_makespan(pieces, heads) + (cuts ? merge_blocks : 0);
        if (best_cost < 0 || cost < best_cost - best_cost / 32) {
            best_cost = cost;
            best = p;
        }
    }
    return best;
}

size_t planned_workspace(int64_t slots, int32_t num_q_heads, size_t *o_bytes) {
    const size_t recs = static_cast<size_t>(slots) * num_q_heads;
    *o_bytes = round_up(static_cast<int64_t>(recs * kHeadDim * sizeof(float)), 256);
    return recs ? *o_bytes + recs * 2 * sizeof(float) : 0;
}


// Builds the serialised schedule.  Without groups every sequence is cut into
// near-equal pieces (see above).  With groups, sequence s of group G attends
// to the shared prefix [0, prefix_len[G]) through prefix pieces of up to
// kMaxPrefixPieceBlocks blocks, each serving up to kMaxMembers members at once,
// and to its own suffix [prefix_len[G], ctx) through ordinary pieces; all its
// records are merged.
pa_status build_plan(const pa_pool *pool, const int32_t *lens, int32_t batch, int32_t num_q_heads,
                     const int32_t *group_of, const int32_t *prefix_len, int32_t num_groups, void *plan_host,
                     size_t plan_host_bytes, pa_plan_info *info) {
    try {
        if (!pool || !info || batch < 0 || num_q_heads <= 0) return PA_ERR_INVALID_ARG;
        if (batch > 0 && !lens) return PA_ERR_INVALID_ARG;
        if (num_q_heads % pool->desc.num_kv_heads != 0) return PA_ERR_INVALID_ARG;
        if (num_q_heads != kGroup * pool->desc.num_kv_heads) return PA_ERR_UNSUPPORTED;
        if (batch > (1 << 24) || num_groups > (1 << 24)) return PA_ERR_UNSUPPORTED;
        for (int32_t gi = 0; gi < num_groups; ++gi)
            if (prefix_len[gi] < 0 || prefix_len[gi] % kBlockSize != 0) return PA_ERR_INVALID_ARG;
        std::vector<int32_t> plen(batch, 0);
        std::vector<std::vector<int32_t>> members(num_groups);
        int64_t total_blocks = 0;
        int32_t max_ctx = 0;
        for (int32_t s = 0; s < batch; ++s) {
            if (lens[s] < 0) return PA_ERR_INVALID_ARG;
            if (lens[s] > pa::kMaxContextTokens) return PA_ERR_UNSUPPORTED;
            max_ctx = std::max(max_ctx, lens[s]);
            if (group_of) {
                const int32_t gi = group_of[s];
                if (gi < -1 || gi >= num_groups) return PA_ERR_INVALID_ARG;
                if (gi >= 0 && prefix_len[gi] > 0) {
                    if (prefix_len[gi] > lens[s]) return PA_ERR_INVALID_ARG;
                    plen[s] = prefix_len[gi];
                    members[gi].push_back(s);
                }
            }
            total_blocks += (static_cast<int64_t>(lens[s]) - plen[s] + kBlockSize - 1) / kBlockSize;
        }
        for (int32_t gi = 0; gi < num_groups; ++gi)
            if (!members[gi].empty())
                total_blocks += static_cast<int64_t>(prefix_len[gi] / kBlockSize) *
                                ((members[gi].size() + pa::kMaxMembers - 1) / pa::kMaxMembers);
        const int64_t items_target = std::max<int64_t>(1, kTargetWorkGroups / pool->desc.num_kv_heads);
        // Without shared prefixes the piece size comes from the dispatch model
        // (F16 blocks cost twice an FP8 block's time, so the merge charge
        // doubles in FP8 blocks); with them, from the work-group target.
        const int64_t piece =
            group_of == nullptr
                ? balanced_piece(lens, plen, batch, pool->desc.num_kv_heads, kMergeBlocks * 2 / pool->elem_bytes())
                : std::min<int64_t>(kMaxSplitTokens / kBlockSize,
                                    std::max<int64_t>(kMinPieceBlocks, (total_blocks + items_target - 1) / items_target));
        auto cut = [](int64_t nb, int64_t maxp) { return nb == 0 ? int64_t{0} : (nb + maxp - 1) / maxp; };

        // records: each member owns a contiguous run (prefix pieces, then its
        // suffix pieces); a sequence without prefix owns one only when cut
        std::vector<int32_t> first(batch, -1), n_prefix(batch, 0);
        int64_t slots = 0;  // records per query head; kept below 2^31
        int32_t shared_newest = 0;
        std::vector<int32_t> merges;
        for (int32_t s = 0; s < batch; ++s) {
            const int64_t suffix_blocks = (static_cast<int64_t>(lens[s]) - plen[s] + kBlockSize - 1) / kBlockSize;
            const int64_t np_suffix = cut(suffix_blocks, piece);
            int64_t n = 0;
            if (plen[s] > 0) {
                n_prefix[s] = static_cast<int32_t>(cut(plen[s] / kBlockSize, pa::kMaxPrefixPieceBlocks));
                n = n_prefix[s] + np_suffix;
                if (lens[s] == plen[s]) ++shared_newest;
            } else if (np_suffix > 1) {
                n = np_suffix;
            }
            if (n == 0) continue;
            if (slots + n > 0x7fffffff) return PA_ERR_UNSUPPORTED;
            first[s] = static_cast<int32_t>(slots);
            slots += n;
            merges.insert(merges.end(), {s, first[s], static_cast<int32_t>(n), s});
        }
        // ordinary pieces (whole contexts, or the suffixes of members)
        std::vector<PlanItem> items;
        for (int32_t s = 0; s < batch; ++s) {
            const int32_t ctx = lens[s];
            const int64_t nb = (static_cast<int64_t>(ctx) - plen[s] + kBlockSize - 1) / kBlockSize;
            const int64_t np = cut(nb, piece);
            if (np == 0) {
                if (plen[s] == 0) items.push_back({s, 0, 0, 0, -1});  // empty context: zero output
                continue;
            }
            if (np == 1 && plen[s] == 0) {
                items.push_back({s, 0, ctx, ctx, -1});
                continue;
            }
            const int64_t base = nb / np, extra = nb % np;
            int64_t b0 = 0;
            const int32_t slot0 = first[s] + n_prefix[s];
            for (int64_t i = 0; i < np; ++i) {
                const int64_t b1 = b0 + base + (i < extra ? 1 : 0);
                items.push_back({s, static_cast<int32_t>(plen[s] + b0 * kBlockSize),
                                 static_cast<int32_t>(std::min<int64_t>(ctx, plen[s] + b1 * kBlockSize)), ctx,
                                 static_cast<int32_t>(slot0 + i)});
                b0 = b1;
            }
        }
        std::stable_sort(items.begin(), items.end(), [](const PlanItem &x, const PlanItem &y) {
            return (x.t_end - x.t_begin) > (y.t_end - y.t_begin);
        });
        // prefix pieces: per group, per subgroup of <= kMaxMembers members, per piece
        std::vector<int32_t> pitems, mlist;
        for (int32_t gi = 0; gi < num_groups; ++gi) {
            const std::vector<int32_t> &mem = members[gi];
            if (mem.empty()) continue;
            const int64_t nb = prefix_len[gi] / kBlockSize;
            const int64_t np = cut(nb, pa::kMaxPrefixPieceBlocks);
            const int64_t base = nb / np, extra = nb % np;
            for (size_t m0 = 0; m0 < mem.size(); m0 += pa::kMaxMembers) {
                const size_t cnt = std::min<size_t>(pa::kMaxMembers, mem.size() - m0);
                int64_t b0 = 0;
                for (int64_t p = 0; p < np; ++p) {
                    const int64_t b1 = b0 + base + (p < extra ? 1 : 0);
                    pitems.insert(pitems.end(), {mem[m0], static_cast<int32_t>(b0 * kBlockSize),
                                                 static_cast<int32_t>(b1 * kBlockSize), static_cast<int32_t>(cnt),
                                                 static_cast<int32_t>(mlist.size() / pa::kMemberInts), 0, 0, 0});
                    for (size_t j = 0; j < cnt; ++j) {
                        const int32_t s = mem[m0 + j];
                        mlist.insert(mlist.end(), {s, first[s] + static_cast<int32_t>(p)});
                    }
                    b0 = b1;
                }
            }
        }
        int32_t longest = 0;
        for (const PlanItem &it : items) longest = std::max(longest, it.t_end - it.t_begin);
        const size_t n_items = items.size(), n_merges = merges.size() / pa::kMergeInts;
        const size_t n_pitems = pitems.size() / pa::kPrefixItemInts, n_members = mlist.size() / pa::kMemberInts;
        if (static_cast<int64_t>(std::max(n_items, n_pitems)) * pool->desc.num_kv_heads > 0x7fffffff ||
            n_merges > 0x7fffffff || n_members > 0x7fffffff)
            return PA_ERR_UNSUPPORTED;
        pa_plan_info inf{};
        inf.batch = batch;
        inf.num_q_heads = num_q_heads;
        inf.max_context_len = max_ctx;
        inf.num_items = static_cast<int32_t>(n_items);
        inf.num_merges = static_cast<int32_t>(n_merges);
        inf.num_slots = static_cast<int32_t>(slots);
        inf.max_piece_tokens = longest;
        inf.num_prefix_items = static_cast<int32_t>(n_pitems);
        inf.num_members = static_cast<int32_t>(n_members);
        inf.shared_newest = shared_newest;
        inf.num_prefill_items = 0;
        inf.num_q_rows = batch;
        inf.mixed_decode_waves = pa::kWaves;
        inf.decode_wave_heads = 0;
        if (pool->desc.num_kv_heads % pa::kWaves == 0 && n_items > 0 && longest <= kWaveHeadsMaxBlocks * kBlockSize) {
            std::vector<int64_t> blocks(n_items);  // in dispatch order, longest first
            for (size_t i = 0; i < n_items; ++i)
                blocks[i] = (static_cast<int64_t>(items[i].t_end) - items[i].t_begin + kBlockSize - 1) / kBlockSize;
            const int64_t split = modelled_makespan(blocks, pool->desc.num_kv_heads);
            const int64_t wave_heads =
                modelled_makespan(blocks, pool->desc.num_kv_heads / pa::kWaves, kWaveHeadsSlots, pa::kWaves);
            inf.decode_wave_heads = wave_heads < split - split / 64 ? 1 : 0;
        }
        inf.plan_bytes = sizeof(int32_t) * (pa::kPlanHeader + pa::kItemInts * n_items + merges.size() +
                                            pitems.size() + mlist.size());
        size_t o_bytes = 0;
        inf.workspace_bytes = planned_workspace(slots, num_q_heads, &o_bytes);
        *info = inf;
        if (!plan_host) return PA_OK;  // size query
        if (plan_host_bytes < inf.plan_bytes) return PA_ERR_WORKSPACE;
        int32_t *p = static_cast<int32_t *>(plan_host);
        const int32_t header[pa::kPlanHeader] = {pa::kPlanMagic, batch, num_q_heads, inf.num_items,
                                                 inf.num_merges, inf.num_slots, max_ctx, inf.num_prefix_items};
        p = std::copy(header, header + pa::kPlanHeader, p);
        for (const PlanItem &it : items) {
            const int32_t rec[pa::kItemInts] = {it.s, it.t_begin, it.t_end, it.ctx, it.slot, it.s, 0, 0};
            p = std::copy(rec, rec + pa::kItemInts, p);
        }
        p = std::copy(merges.begin(), merges.end(), p);
        p = std::copy(pitems.begin(), pitems.end(), p);
        std::copy(mlist.begin(), mlist.end(), p);
        return PA_OK;
    } catch (...) {
        return PA_ERR_INVALID_ARG;
    }
}

// Schedule of a chunked-prefill / mixed step.  One-token rows are decode
// pieces cut exactly as build_plan cuts contexts (item field 5 carries the
// packed q/out row).  A longer chunk is cut into tiles of kPrefillTile query
// tokens; tile i of sequence s has its first query at position
// pos0 = seq_len - q_len + kPrefillTile * i and sees keys [0, pos0 + n_q)
// causally.  Key ranges are cut into near-equal pieces of at most P blocks,
// P = ceil(total tile blocks / (kTargetWorkGroups / Hkv)) clamped to
// [8, kMaxPrefillPieceBlocks]; a tile cut into np pieces owns n_q * np
// records (token k's come at base + k * np) and one merge per query token.
// Both kinds of pieces are dispatched longest first.
pa_status build_mixed_plan(const pa_pool *pool, const int32_t *query_start, const int32_t *lens, int32_t batch,
                           int32_t num_q_heads, void *plan_host, size_t plan_host_bytes, pa_plan_info *info) {
    try {
        if (!pool || !info || batch < 0 || num_q_heads <= 0 || !query_start) return PA_ERR_INVALID_ARG;
        if (batch > 0 && !lens) return PA_ERR_INVALID_ARG;
        if (num_q_heads % pool->desc.num_kv_heads != 0) return PA_ERR_INVALID_ARG;
        if (num_q_heads != kGroup * pool->desc.num_kv_heads) return PA_ERR_UNSUPPORTED;
        if (batch > (1 << 24)) return PA_ERR_UNSUPPORTED;
        if (query_start[0] != 0) return PA_ERR_INVALID_ARG;
        int32_t max_ctx = 0;
        int64_t dec_blocks = 0, tile_blocks = 0, n_tiles = 0, max_tile = 0;
        for (int32_t s = 0; s < batch; ++s) {
            const int64_t q_len = static_cast<int64_t>(query_start[s + 1]) - query_start[s];
            if (q_len < 0 || lens[s] < q_len) return PA_ERR_INVALID_ARG;
            if (lens[s] > pa::kMaxContextTokens) return PA_ERR_UNSUPPORTED;
            max_ctx = std::max(max_ctx, lens[s]);
            if (q_len == 1) dec_blocks += (static_cast<int64_t>(lens[s]) + kBlockSize - 1) / kBlockSize;
            for (int64_t j0 = 0; j0 < q_len; j0 += pa::kPrefillTile) {
                if (q_len == 1) break;
                const int64_t kend = lens[s] - q_len + std::min<int64_t>(q_len, j0 + pa::kPrefillTile);
                tile_blocks += (kend + kBlockSize - 1) / kBlockSize;
                ++n_tiles;
                max_tile = std::max<int64_t>(max_tile, (kend + kBlockSize - 1) / kBlockSize);
            }
        }
        const int32_t num_q_rows = query_start[batch];
        if (num_q_rows > (1 << 24)) return PA_ERR_UNSUPPORTED;
        // A launch with both kinds of pieces: when the prompt tiles take longer
        // than the decode pieces, the decode pieces are walked by 2 of their
        // work-group's 4 waves.  Decode streams with all 4 waves fill each CU's
        // memory path, and the prompt tiles sharing the CU barely progress until
        // they end (the launch then costs the sum of its parts); with 2, both
        // kinds run side by side and the decode pieces, at about half their
        // rate, end about when the tiles do.  32 decodes at 4096 tokens beside
        // a 2016-token chunk at position 2016, per layer: decode alone
        // 89 us, chunk alone 142-150 us, fused 228-234 us with 4 waves and
        // 190-198 us with 2 (1 wave: 188 us; 3: 220 us).  The estimate: decode
        // bytes at 6.5 TB/s against the tiles' flops at 0.85 PFLOP/s (their
        // rates measured alone).  With the tiles' waves at the higher issue
        // priority (mixed_kernel) 2 waves still win: that step over 32 layers
        // 5.13 ms against 5.28-5.30 ms with 4.
        double tile_flops = 0.0;
        for (int32_t s = 0; s < batch; ++s) {
            const int64_t q_len = static_cast<int64_t>(query_start[s + 1]) - query_start[s];
            if (q_len < 2) continue;
            const double hist = static_cast<double>(lens[s]) - static_cast<double>(q_len);
            tile_flops += 4.0 * kHeadDim * num_q_heads *
                          (static_cast<double>(q_len) * hist + static_cast<double>(q_len) * (q_len + 1) / 2.0);
        }
        const double dec_bytes = static_cast<double>(dec_blocks) * kBlockSize * pool->desc.num_kv_heads * kHeadDim *
                                 2.0 * pool->elem_bytes();
        const int32_t mixed_waves = tile_flops / 0.85e15 > dec_bytes / 6.5e12 ? 2 : pa::kWaves;
        const int64_t items_target = std::max<int64_t>(1, kTargetWorkGroups / pool->desc.num_kv_heads);
        auto cut = [](int64_t nb, int64_t maxp) { return nb == 0 ? int64_t{0} : (nb + maxp - 1) / maxp; };

        int64_t slots = 0;  // records per query head
        std::vector<int32_t> merges;
        // decode rows
        std::vector<PlanItem> items;
        std::vector<int32_t> item_row;
        const int64_t piece = std::min<int64_t>(kMaxSplitTokens / kBlockSize,
                                                std::max<int64_t>(kMinPieceBlocks, cut(dec_blocks, items_target)));
        for (int32_t s = 0; s < batch; ++s) {
            if (query_start[s + 1] - query_start[s] != 1) continue;
            const int32_t ctx = lens[s], row = query_start[s];
            const int64_t nb = (static_cast<int64_t>(ctx) + kBlockSize - 1) / kBlockSize;
            const int64_t np = cut(nb, piece);
            if (np <= 1) {
                items.push_back({s, 0, ctx, ctx, -1});
                item_row.push_back(row);
                continue;
            }
            if (slots + np > 0x7fffffff) return PA_ERR_UNSUPPORTED;
            merges.insert(merges.end(), {s, static_cast<int32_t>(slots), static_cast<int32_t>(np), row});
            const int64_t base = nb / np, extra = nb % np;
            int64_t b0 = 0;
            for (int64_t i = 0; i < np; ++i) {
                const int64_t b1 = b0 + base + (i < extra ? 1 : 0);
                items.push_back({s, static_cast<int32_t>(b0 * kBlockSize),
                                 static_cast<int32_t>(std::min<int64_t>(ctx, b1 * kBlockSize)), ctx,
                                 static_cast<int32_t>(slots + i)});
                item_row.push_back(row);
                b0 = b1;
            }
            slots += np;
        }
        std::vector<size_t> order(items.size());
        for (size_t i = 0; i < order.size(); ++i) order[i] = i;
        std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) {
            return (items[x].t_end - items[x].t_begin) > (items[y].t_end - items[y].t_begin);
        });
        // prefill tiles
        struct PrefillItem {
            int32_t f[pa::kPrefillItemInts];
        };
        std::vector<PrefillItem> pitems;
        int64_t ppiece = std::min<int64_t>(pa::kMaxPrefillPieceBlocks,
                                           std::max<int64_t>(8, cut(tile_blocks, items_target)));
        // A launch of prompt tiles alone with at most one work-group per CU
        // runs the split kernels (each tile's keys over two wave groups of one
        // work-group), so its tiles are cut only as far as that count allows:
        // into at most items_target / n_tiles pieces each.  The 32 tiles of a
        // 1,024-token chunk at position 3,008 (F16): whole, 94.0-94.6 us,
        // against 121 us cut into 48 pieces for four-wave work-groups.
        if (items.empty() && n_tiles > 0 && n_tiles <= items_target)
            ppiece = std::min<int64_t>(pa::kMaxPrefillPieceBlocks,
                                       std::max<int64_t>(8, cut(max_tile, items_target / n_tiles)));
        for (int32_t s = 0; s < batch; ++s) {
            const int64_t q_len = static_cast<int64_t>(query_start[s + 1]) - query_start[s];
            if (q_len < 2) continue;
            for (int64_t j0 = 0; j0 < q_len; j0 += pa::kPrefillTile) {
                const int32_t n_q = static_cast<int32_t>(std::min<int64_t>(pa::kPrefillTile, q_len - j0));
                const int32_t pos0 = static_cast<int32_t>(lens[s] - q_len + j0);
                const int32_t kend = pos0 + n_q;
                const int32_t row0 = static_cast<int32_t>(query_start[s] + j0);
                const int64_t nb = (kend + kBlockSize - 1) / kBlockSize;
                const int64_t np = cut(nb, ppiece);
                if (slots + static_cast<int64_t>(n_q) * np > 0x7fffffff) return PA_ERR_UNSUPPORTED;
                const int32_t base_slot = np > 1 ? static_cast<int32_t>(slots) : -1;
                if (np > 1) {
                    for (int32_t k = 0; k < n_q; ++k)
                        merges.insert(merges.end(), {s, static_cast<int32_t>(slots + k * np), static_cast<int32_t>(np),
                                                     row0 + k});
                    slots += static_cast<int64_t>(n_q) * np;
                }
                const int64_t base = nb / np, extra = nb % np;
                int64_t b0 = 0;
                for (int64_t p = 0; p < np; ++p) {
                    const int64_t b1 = b0 + base + (p < extra ? 1 : 0);
                    PrefillItem it{};
                    const int32_t f[pa::kPrefillItemInts] = {
                        s, row0, n_q, pos0, static_cast<int32_t>(b0 * kBlockSize),
                        static_cast<int32_t>(std::min<int64_t>(kend, b1 * kBlockSize)), base_slot,
                        static_cast<int32_t>(np), static_cast<int32_t>(p), 0, 0, 0};
                    std::copy(f, f + pa::kPrefillItemInts, it.f);
                    pitems.push_back(it);
                    b0 = b1;
                }
            }
        }
        std::stable_sort(pitems.begin(), pitems.end(), [](const PrefillItem &x, const PrefillItem &y) {
            return (x.f[5] - x.f[4]) > (y.f[5] - y.f[4]);
        });
        // A prefill-only launch that fits in one round of two work-groups per
        // CU starts all its work-groups at once, so order decides only which
        // two share a CU: the dispatcher's second round lands on the CUs in
        // the first round's order.  The longest kTargetWorkGroups/Hkv tiles go
        // first, longest first, and the rest follow shortest first, so the
        // longest tile shares its CU with the shortest.  (A 2016-token chunk at
        // position 2016, 63 tiles: 124.9 us per layer against 127.7-129.2 us
        // longest-first; with decode pieces in the launch, or more tiles than
        // one round holds, the plain longest-first order measured as fast or
        // faster.)
        {
            const int64_t first = kTargetWorkGroups / pool->desc.num_kv_heads;
            const int64_t wgs = static_cast<int64_t>(pitems.size()) * pool->desc.num_kv_heads;
            if (items.empty() && first > 0 && wgs > kTargetWorkGroups && wgs <= 2 * kTargetWorkGroups)
                std::reverse(pitems.begin() + first, pitems.end());
        }
        int32_t longest = 0;
        for (const PlanItem &it : items) longest = std::max(longest, it.t_end - it.t_begin);
        const size_t n_items = items.size(), n_merges = merges.size() / pa::kMergeInts, n_pf = pitems.size();
        if (static_cast<int64_t>(std::max(n_items, n_pf)) * pool->desc.num_kv_heads > 0x7fffffff ||
            n_merges > 0x7fffffff)
            return PA_ERR_UNSUPPORTED;
        pa_plan_info inf{};
        inf.batch = batch;
        inf.num_q_heads = num_q_heads;
        inf.max_context_len = max_ctx;
        inf.num_items = static_cast<int32_t>(n_items);
        inf.num_merges = static_cast<int32_t>(n_merges);
        inf.num_slots = static_cast<int32_t>(slots);
        inf.max_piece_tokens = longest;
        inf.num_prefill_items = static_cast<int32_t>(n_pf);
        inf.num_q_rows = num_q_rows;
        inf.mixed_decode_waves = mixed_waves;
        inf.plan_bytes = sizeof(int32_t) * (pa::kPlanHeader + pa::kItemInts * n_items + merges.size() +
                                            pa::kPrefillItemInts * n_pf);
        size_t o_bytes = 0;
        inf.workspace_bytes = planned_workspace(slots, num_q_heads, &o_bytes);
        *info = inf;
        if (!plan_host) return PA_OK;
        if (plan_host_bytes < inf.plan_bytes) return PA_ERR_WORKSPACE;
        int32_t *p = static_cast<int32_t *>(plan_host);
        const int32_t header[pa::kPlanHeader] = {pa::kPlanMagic, batch, num_q_heads, inf.num_items,
                                                 inf.num_merges, inf.num_slots, max_ctx, 0};
        p = std::copy(header, header + pa::kPlanHeader, p);
        for (size_t i : order) {
            const PlanItem &it = items[i];
            const int32_t rec[pa::kItemInts] = {it.s, it.t_begin, it.t_end, it.ctx, it.slot, item_row[i], 0, 0};
            p = std::copy(rec, rec + pa::kItemInts, p);
        }
        p = std::copy(merges.begin(), merges.end(), p);
        for (const PrefillItem &it : pitems) p = std::copy(it.f, it.f + pa::kPrefillItemInts, p);
        return PA_OK;
    } catch (...) {
        return PA_ERR_INVALID_ARG;
    }
}

// One layer on a serialised schedule (pa_decode_plan, pa_cascade_plan or
// pa_prefill_plan): decode pieces, shared-prefix pieces, prefill pieces, then
// the merges.
pa_status run_plan(pa_pool *pool, int32_t layer, const pa_plan_info *info, const void *plan_dev,
                   size_t plan_dev_bytes, const void *q_dev, const void *k_new_dev, const void *v_new_dev, void *out_dev, const int32_t *block_tables_dev,
                   int32_t max_blocks_per_seq, float scale, void *workspace_dev, size_t workspace_bytes,
                   hipStream_t stream) {
    if (!pool || !info || layer < 0 || layer >= pool->desc.num_layers) return PA_ERR_INVALID_ARG;
    if (info->batch < 0 || info->num_q_heads != kGroup * pool->desc.num_kv_heads) return PA_ERR_INVALID_ARG;
    if (info->num_items < 0 || info->num_prefix_items < 0 || info->num_prefill_items < 0 || info->num_merges < 0 ||
        info->num_slots < 0 || info->num_members < 0 || info->num_q_rows < 0)
        return PA_ERR_INVALID_ARG;
    // The kernels index the plan's sections by these counts, so the plan must
    // be exactly the serialised size they imply and fit the device buffer.
    const uint64_t plan_ints = static_cast<uint64_t>(pa::kPlanHeader) +
                               static_cast<uint64_t>(pa::kItemInts) * info->num_items +
                               static_cast<uint64_t>(pa::kMergeInts) * info->num_merges +
                               static_cast<uint64_t>(pa::kPrefixItemInts) * info->num_prefix_items +
                               static_cast<uint64_t>(pa::kMemberInts) * info->num_members +
                               static_cast<uint64_t>(pa::kPrefillItemInts) * info->num_prefill_items;
    if (info->plan_bytes != plan_ints * sizeof(int32_t)) return PA_ERR_INVALID_ARG;
    if (info->batch == 0 || (info->num_items == 0 && info->num_prefix_items == 0 && info->num_prefill_items == 0))
        return PA_OK;
    if (plan_dev_bytes < info->plan_bytes) return PA_ERR_WORKSPACE;
    if (info->num_q_rows == 0) return PA_ERR_INVALID_ARG;
    if (k_new_dev && info->num_q_rows != info->batch) return PA_ERR_INVALID_ARG;
    if (!plan_dev || !q_dev || !out_dev || !aligned(plan_dev, 16) || !aligned(q_dev, 16) || !aligned(out_dev, 16))
        return PA_ERR_INVALID_ARG;
    if ((k_new_dev == nullptr) != (v_new_dev == nullptr)) return PA_ERR_INVALID_ARG;
    if (k_new_dev && (!aligned(k_new_dev, 16) || !aligned(v_new_dev, 16))) return PA_ERR_INVALID_ARG;
    if (k_new_dev && info->shared_newest > 0) return PA_ERR_INVALID_ARG;  // newest token in a shared block
    if (info->max_context_len > 0 && (!block_tables_dev || !aligned(block_tables_dev, 4))) return PA_ERR_INVALID_ARG;
    if (max_blocks_per_seq < 0 ||
        static_cast<int64_t>(info->max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * kBlockSize)
        return PA_ERR_INVALID_ARG;
    if (info->max_context_len > pa::kMaxContextTokens || max_blocks_per_seq > pa::kMaxContextTokens / kBlockSize)
        return PA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
    size_t o_bytes = 0;
    const size_t need = planned_workspace(info->num_slots, info->num_q_heads, &o_bytes);
    if (need > 0 && (!workspace_dev || workspace_bytes < need)) return PA_ERR_WORKSPACE;
    if (need > 0 && !aligned(workspace_dev, 256)) return PA_ERR_INVALID_ARG;
    pa::DecodeArgs a{};
    a.k_layer = static_cast<const char *>(pool->k) + pool->layer_offset(layer);
    a.v_layer = static_cast<const char *>(pool->v) + pool->layer_offset(layer);
    set_scales(pool, layer, &a);
    a.q = static_cast<const uint16_t *>(q_dev);
    a.k_new = static_cast<const uint16_t *>(k_new_dev);
    a.v_new = static_cast<const uint16_t *>(v_new_dev);
    a.tables = block_tables_dev;
    a.out = static_cast<uint16_t *>(out_dev);
    a.o_part = need ? static_cast<float *>(workspace_dev) : nullptr;
    a.ml_part = need ? reinterpret_cast<float *>(static_cast<char *>(workspace_dev) + o_bytes) : nullptr;
    a.batch = info->batch;
    a.num_q_rows = info->num_q_rows;
    a.num_q_heads = info->num_q_heads;
    a.num_kv_heads = pool->desc.num_kv_heads;
    a.num_blocks = pool->desc.num_blocks;
    a.max_blocks = max_blocks_per_seq;
    a.max_ctx = info->max_context_len;
    a.split_tokens = kMaxSplitTokens;
    a.max_splits = 1;
    a.scale_log2e = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634 *
                                       (pool->elem_bytes() == 1 ? pool->k_scale[layer] : 1.0f));
    a.items = static_cast<const int32_t *>(plan_dev) + pa::kPlanHeader;
    a.merges = a.items + static_cast<size_t>(pa::kItemInts) * info->num_items;
    a.num_items = info->num_items;
    a.num_merges = info->num_merges;
    a.num_slots = info->num_slots;
    a.prefix_items = a.merges + static_cast<size_t>(pa::kMergeInts) * info->num_merges;
    a.members = a.prefix_items + static_cast<size_t>(pa::kPrefixItemInts) * info->num_prefix_items;
    a.num_prefix_items = info->num_prefix_items;
    a.num_members = info->num_members;
    a.prefill_items = a.members + static_cast<size_t>(pa::kMemberInts) * info->num_members;
    a.num_prefill_items = info->num_prefill_items;
    a.mixed_decode_waves = info->mixed_decode_waves == 2 ? 2 : pa::kWaves;
    a.decode_wave_heads = info->decode_wave_heads == 1 && a.num_kv_heads % pa::kWaves == 0 &&
                                  info->max_piece_tokens <= kWaveHeadsMaxBlocks * kBlockSize
                              ? 1
                              : 0;
    if (info->num_items > 0 && info->num_prefill_items > 0 &&
        static_cast<int64_t>(info->num_items + info->num_prefill_items) * pool->desc.num_kv_heads <= 0x7fffffff) {
        // decode and prefill pieces share one launch
        if (pa::launch_mixed(a, stream) != hipSuccess) return PA_ERR_HIP;
    } else if (info->num_items > 0 && info->num_prefix_items > 0 &&
               static_cast<int64_t>(info->num_items + info->num_prefix_items) * pool->desc.num_kv_heads <=
                   0x7fffffff) {
        // ordinary and shared-prefix pieces share one launch
        if (pa::launch_cascade(a, stream) != hipSuccess) return PA_ERR_HIP;
    } else {
        if (info->num_items > 0 && pa::launch_decode_partial(a, stream) != hipSuccess) return PA_ERR_HIP;
        if (info->num_prefill_items > 0 && pa::launch_prefill(a, stream) != hipSuccess) return PA_ERR_HIP;
        if (info->num_prefix_items > 0 && pa::launch_decode_prefix(a, stream) != hipSuccess) return PA_ERR_HIP;
    }
    if (info->num_merges > 0 && pa::launch_decode_merge_planned(a, stream) != hipSuccess) return PA_ERR_HIP;
    return PA_OK;
}

}  // namespace

extern "C" {

pa_status pa_decode_plan(const pa_pool *pool, const int32_t *context_lens_host, int32_t batch, int32_t num_q_heads,
                         void *plan_host, size_t plan_host_bytes, pa_plan_info *info) {
    return build_plan(pool, context_lens_host, batch, num_q_heads, nullptr, nullptr, 0, plan_host, plan_host_bytes,
                      info);
}

pa_status pa_cascade_plan(const pa_pool *pool, const int32_t *context_lens_host, int32_t batch,
                          const int32_t *prefix_group_host, const int32_t *prefix_len_host, int32_t num_groups,
                          int32_t num_q_heads, void *plan_host, size_t plan_host_bytes, pa_plan_info *info) {
    if (num_groups < 0 || (num_groups > 0 && (!prefix_group_host || !prefix_len_host))) return PA_ERR_INVALID_ARG;
    return build_plan(pool, context_lens_host, batch, num_q_heads, prefix_group_host, prefix_len_host, num_groups,
                      plan_host, plan_host_bytes, info);
}

pa_status pa_decode_run(pa_pool *pool, int32_t layer, const pa_plan_info *info, const void *plan_dev,
                        size_t plan_dev_bytes, const void *q_dev, const void *k_new_dev, const void *v_new_dev,
                        void *out_dev, const int32_t *block_tables_dev, int32_t max_blocks_per_seq, float scale,
                        void *workspace_dev, size_t workspace_bytes, hipStream_t stream) {
    if (info && info->num_prefill_items != 0) return PA_ERR_INVALID_ARG;  // a pa_prefill_plan schedule
    return run_plan(pool, layer, info, plan_dev, plan_dev_bytes, q_dev, k_new_dev, v_new_dev, out_dev,
                    block_tables_dev, max_blocks_per_seq, scale, workspace_dev, workspace_bytes, stream);
}

pa_status pa_prefill_plan(const pa_pool *pool, const int32_t *query_start_host, const int32_t *seq_lens_host,
                          int32_t batch, int32_t num_q_heads, void *plan_host, size_t plan_host_bytes,
                          pa_plan_info *info) {
    return build_mixed_plan(pool, query_start_host, seq_lens_host, batch, num_q_heads, plan_host, plan_host_bytes,
                            info);
}

pa_status pa_prefill_run(pa_pool *pool, int32_t layer, const pa_plan_info *info, const void *plan_dev,
                         size_t plan_dev_bytes, const void *q_dev, void *out_dev, const int32_t *block_tables_dev,
                         int32_t max_blocks_per_seq, float scale, void *workspace_dev, size_t workspace_bytes,
                         hipStream_t stream) {
    if (info && (info->num_prefix_items != 0 || info->num_members != 0)) return PA_ERR_INVALID_ARG;
    return run_plan(pool, layer, info, plan_dev, plan_dev_bytes, q_dev, nullptr, nullptr, out_dev,
                    block_tables_dev, max_blocks_per_seq, scale, workspace_dev, workspace_bytes, stream);
}

size_t pa_pool_bytes(const pa_pool_desc *desc) {
    if (!desc_ok(desc)) return 0;
    const size_t elem = desc->dtype == PA_F16 ? 2 : desc->dtype == PA_FP8_E4M3 ? 1 : 0;
    return static_cast<size_t>(desc->num_layers) * desc->num_blocks * desc->block_size * desc->num_kv_heads *
           desc->head_dim * elem;
}

pa_status pa_pool_create(const pa_pool_desc *desc, void *k_pool_dev, void *v_pool_dev, pa_pool **out) {
    if (!out || !desc_ok(desc) || !k_pool_dev || !v_pool_dev) return PA_ERR_INVALID_ARG;
    if (!desc_supported(desc)) return PA_ERR_UNSUPPORTED;
    if (!aligned(k_pool_dev, 256) || !aligned(v_pool_dev, 256)) return PA_ERR_INVALID_ARG;
    pa_pool *p = new (std::nothrow) pa_pool;
    if (!p) return PA_ERR_INVALID_ARG;
    try {
        p->desc = *desc;
        p->k = k_pool_dev;
        p->v = v_pool_dev;
        p->k_scale.assign(desc->num_layers, 1.0f);
        p->v_scale.assign(desc->num_layers, 1.0f);
    } catch (...) {
        delete p;
        return PA_ERR_INVALID_ARG;
    }
    *out = p;
    return PA_OK;
}

pa_status pa_pool_set_scales(pa_pool *pool, int32_t layer, float k_scale, float v_scale) {
    if (!pool || layer < 0 || layer >= pool->desc.num_layers) return PA_ERR_INVALID_ARG;
    if (!(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
        return PA_ERR_INVALID_ARG;
    if (!std::isfinite(1.0f / k_scale) || !std::isfinite(1.0f / v_scale)) return PA_ERR_INVALID_ARG;
    pool->k_scale[layer] = k_scale;
    pool->v_scale[layer] = v_scale;
    return PA_OK;
}

pa_status pa_pool_destroy(pa_pool *pool) {
    delete pool;
    return PA_OK;
}

pa_status pa_write_kv(pa_pool *pool, int32_t layer, const void *k_new_dev, const void *v_new_dev,
                      const int32_t *slot_mapping_dev, int32_t n_tokens, hipStream_t stream) {
    if (!pool || n_tokens < 0 || layer < 0 || layer >= pool->desc.num_layers) return PA_ERR_INVALID_ARG;
    if (n_tokens == 0) return PA_OK;
    if (!k_new_dev || !v_new_dev || !slot_mapping_dev) return PA_ERR_INVALID_ARG;
    if (!aligned(k_new_dev, 16) || !aligned(v_new_dev, 16) || !aligned(slot_mapping_dev, 4))
        return PA_ERR_INVALID_ARG;
    pa::WriteKvArgs a{};
    a.k_layer = static_cast<char *>(pool->k) + pool->layer_offset(layer);
    a.v_layer = static_cast<char *>(pool->v) + pool->layer_offset(layer);
    a.elem_bytes = pool->elem_bytes();
    a.inv_k_scale = inv_scale(pool->k_scale[layer]);
    a.inv_v_scale = inv_scale(pool->v_scale[layer]);
    a.k_new = static_cast<const uint16_t *>(k_new_dev);
    a.v_new = static_cast<const uint16_t *>(v_new_dev);
    a.slot_mapping = slot_mapping_dev;
    a.n_tokens = n_tokens;
    a.num_kv_heads = pool->desc.num_kv_heads;
    a.num_slots = static_cast<int64_t>(pool->desc.num_blocks) * pool->desc.block_size;
    return pa::launch_write_kv(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int32_t pa_decode_split_tokens(const pa_pool *pool, int32_t batch, int32_t num_q_heads, int32_t max_context_len) {
    if (!pool || batch < 0 || num_q_heads <= 0 || max_context_len < 0) return 0;
    return plan_split(batch, pool->desc.num_kv_heads, max_context_len);
}

size_t pa_decode_workspace_bytes(const pa_pool *pool, int32_t batch, int32_t num_q_heads,
                                 int32_t max_context_len) {
    if (!pool || batch <= 0 || num_q_heads <= 0 || max_context_len < 0) return 0;
    return make_plan(pool, batch, num_q_heads, max_context_len).workspace;
}

pa_status pa_decode_partial(pa_pool *pool, int32_t layer, const void *q_dev, const void *k_new_dev,
                            const void *v_new_dev, void *out_dev, const int32_t *block_tables_dev,
                            int32_t max_blocks_per_seq, const int32_t *context_lens_dev, int32_t batch,
                            int32_t num_q_heads, int32_t max_context_len, float scale, void *workspace_dev,
                            size_t workspace_bytes, hipStream_t stream) {
    pa::DecodeArgs a{};
    Plan plan{};
    pa_status st = fill_decode_args(pool, layer, q_dev, k_new_dev, v_new_dev, out_dev, block_tables_dev,
                                    max_blocks_per_seq,
                                    context_lens_dev, batch, num_q_heads, max_context_len, scale, workspace_dev,
                                    workspace_bytes, &a, &plan);
    if (st != PA_OK || batch == 0) return st;
    return pa::launch_decode_partial(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_decode_merge(pa_pool *pool, void *out_dev, const int32_t *context_lens_dev, int32_t batch,
                          int32_t num_q_heads, int32_t max_context_len, const void *workspace_dev,
                          size_t workspace_bytes, hipStream_t stream) {
    pa_status st = check_decode_shape(pool, batch, num_q_heads, (max_context_len + kBlockSize - 1) / kBlockSize,
                                      max_context_len);
    if (st != PA_OK || batch == 0) return st;
    if (!out_dev || !context_lens_dev || !aligned(out_dev, 16) || !aligned(context_lens_dev, 4))
        return PA_ERR_INVALID_ARG;
    const Plan plan = make_plan(pool, batch, num_q_heads, max_context_len);
    if (plan.workspace == 0) return PA_OK;  // the partial phase wrote the output
    if (!workspace_dev || workspace_bytes < plan.workspace) return PA_ERR_WORKSPACE;
    if (!aligned(workspace_dev, 256)) return PA_ERR_INVALID_ARG;
    pa::DecodeArgs a{};
    a.ctx_lens = context_lens_dev;
    a.out = static_cast<uint16_t *>(out_dev);
    a.o_part = static_cast<float *>(const_cast<void *>(workspace_dev));
    a.ml_part = reinterpret_cast<float *>(static_cast<char *>(const_cast<void *>(workspace_dev)) + plan.o_bytes);
    a.batch = batch;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = pool->desc.num_kv_heads;
    a.max_blocks = (max_context_len + kBlockSize - 1) / kBlockSize;
    a.max_ctx = max_context_len;
    a.split_tokens = plan.split_tokens;
    a.max_splits = plan.max_splits;
    return pa::launch_decode_merge(a, stream) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status pa_append_decode(pa_pool *pool, int32_t layer, const void *q_dev, const void *k_new_dev,
                           const void *v_new_dev, void *out_dev, const int32_t *block_tables_dev,
                           int32_t max_blocks_per_seq, const int32_t *context_lens_dev, int32_t batch,
                           int32_t num_q_heads, int32_t max_context_len, float scale, void *workspace_dev,
                           size_t workspace_bytes, hipStream_t stream) {
    if (!k_new_dev || !v_new_dev) return PA_ERR_INVALID_ARG;
    pa_status st = pa_decode_partial(pool, layer, q_dev, k_new_dev, v_new_dev, out_dev, block_tables_dev,
                                     max_blocks_per_seq, context_lens_dev, batch, num_q_heads, max_context_len,
                                     scale, workspace_dev, workspace_bytes, stream);
    if (st != PA_OK || batch == 0) return st;
    return pa_decode_merge(pool, out_dev, context_lens_dev, batch, num_q_heads, max_context_len, workspace_dev,
                           workspace_bytes, stream);
}

pa_status pa_decode(pa_pool *pool, int32_t layer, const void *q_dev, void *out_dev,
                    const int32_t *block_tables_dev, int32_t max_blocks_per_seq, const int32_t *context_lens_dev,
                    int32_t batch, int32_t num_q_heads, int32_t max_context_len, float scale,
                    void *workspace_dev, size_t workspace_bytes, hipStream_t stream) {
    pa_status st = pa_decode_partial(pool, layer, q_dev, nullptr, nullptr, out_dev, block_tables_dev,
                                     max_blocks_per_seq, context_lens_dev, batch, num_q_heads, max_context_len,
                                     scale, workspace_dev, workspace_bytes, stream);
    if (st != PA_OK || batch == 0) return st;
    return pa_decode_merge(pool, out_dev, context_lens_dev, batch, num_q_heads, max_context_len, workspace_dev,
                           workspace_bytes, stream);
}

pa_status pa_decode_noalloc(pa_pool *pool, int32_t layer, const void *q_dev, void *out_dev,
                            const int32_t *block_tables_dev, int32_t max_blocks_per_seq,
                            const int32_t *context_lens_dev, int32_t batch, int32_t num_q_heads,
                            int32_t max_context_len, float scale, hipStream_t stream) {
    const pa_status st = check_decode_shape(pool, batch, num_q_heads, max_blocks_per_seq, max_context_len);
    if (st != PA_OK) return st;
    if (batch == 0)
        return pa_decode(pool, layer, q_dev, out_dev, block_tables_dev, max_blocks_per_seq, context_lens_dev,
                         batch, num_q_heads, max_context_len, scale, nullptr, 0, stream);
    const Plan plan = make_plan(pool, batch, num_q_heads, max_context_len);
    if (plan.workspace > pa::kNoAllocScratchBytes) return PA_ERR_WORKSPACE;
    void *ws = nullptr;
    if (plan.workspace > 0 && pa::noalloc_scratch(stream, &ws) != hipSuccess) return PA_ERR_HIP;
    return pa_decode(pool, layer, q_dev, out_dev, block_tables_dev, max_blocks_per_seq, context_lens_dev, batch,
                     num_q_heads, max_context_len, scale, ws, plan.workspace, stream);
}

const char *pa_status_string(pa_status status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_INVALID_ARG: return "invalid argument";
        case PA_ERR_UNSUPPORTED: return "unsupported geometry";
        case PA_ERR_WORKSPACE: return "workspace too small";
        case PA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

}  // extern "C"
