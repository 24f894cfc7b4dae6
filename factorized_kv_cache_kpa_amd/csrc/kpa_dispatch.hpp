// Kernel-path selection and split-KV planning (host only).
#pragma once

#include <algorithm>

#include "kpa_common.hpp"

namespace kpa {

enum class Path { kUnsupported, kValu, kMfmaSq, kMfmaRebuild };

struct Plan {
    Path path;
    int32_t n_split;
    int32_t chunk_tiles;
    int32_t n_group;        // merge groups (level-2 partials) per (row, head); 1 = single level
    size_t part_floats;     // level-1 partials
    size_t part2_floats;    // level-2 partials
    size_t workspace_bytes;
};

// Split-KV merge levels.  Up to kMergeGroup chunks per (row, head) are merged
// by a 256-thread block; up to kMaxSingleLevel by one 1024-thread block when
// a single pass of loads covers them (at most 16 vectors per thread);
// otherwise blocks merge kMergeGroup chunks each and a second level merges
// their results.
constexpr int kMergeGroup = 64;
constexpr int kMaxSingleLevel = 1024;

inline bool merge_single_level(int64_t s, int64_t dh) {
    if (s <= kMergeGroup) return true;
    if (s > kMaxSingleLevel) return false;
    const int64_t vec = dh % 4 == 0 ? 4 : 2;
    const int64_t per_pass = 1024 / (dh / vec);  // chunks one pass of 1024 threads covers
    return (s + per_pass - 1) / per_pass <= 16;
}

inline const char* path_name(Path p) {
    switch (p) {
        case Path::kValu: return "valu";
        case Path::kMfmaSq: return "mfma_bf16";
        case Path::kMfmaRebuild: return "mfma_rebuild";
        default: return "";
    }
}

inline Path select_path(const kpa_dims& d, int32_t n_q) {
    if (decode_rebuild_supported(d, n_q)) return Path::kMfmaRebuild;
    if (decode_mfma_supported(d, n_q)) return Path::kMfmaSq;
    return Path::kValu;
}

// Chunks per (sequence, query): enough workgroups to cover the chip several
// times over, never an empty chunk.
inline Plan plan_decode(const kpa_dims& d, int32_t batch, int32_t max_ctx, int32_t n_q,
                        int32_t num_splits, int cus) {
    Plan p{};
    p.path = select_path(d, n_q);
    const int64_t tiles = (max_ctx + kTileSlots - 1) / kTileSlots;
    const int64_t rows = (int64_t)batch * n_q;
    int64_t s;
    if (num_splits > 0) {
        s = num_splits;
    } else {
        // one full round of workgroups: as many as the CUs hold at once (the
        // kernel's occupancy from its registers and LDS, as the runtime
        // reports it; a partial second round would leave most CUs idle)
        const bool mfma = p.path == Path::kMfmaSq, rebuild = p.path == Path::kMfmaRebuild;
        const int64_t per_cu = rebuild ? decode_rebuild_blocks_per_cu(d)
                               : mfma  ? decode_mfma_blocks_per_cu(d, n_q)
                                       : decode_valu_blocks_per_cu(d);
        // (a tuned matrix-core kernel may ask for a fraction of them)
        const int64_t fill = mfma ? decode_mfma_fill_pct(d, n_q) : 100;
        const int64_t target = std::max<int64_t>(1, per_cu * cus * fill / 100);
        // workgroups per chunk: one per query group (matrix cores; the
        // rebuild kernel also one per A head), one per query (VALU)
        const int64_t wg_rows = rebuild ? (int64_t)batch * decode_rebuild_head_groups(d) * decode_rebuild_query_groups(n_q)
                                : mfma  ? (int64_t)batch * decode_mfma_query_groups(d, n_q)
                                        : rows;
        s = wg_rows > 0 ? (target + wg_rows - 1) / wg_rows : 1;
        const int64_t min_tiles_per_chunk = 2;
        const int64_t cap = (tiles + min_tiles_per_chunk - 1) / min_tiles_per_chunk;
        if (s > cap) s = cap;
        // a second merge level costs a same-address atomic per block (slow
        // on this part): stay within one level; fewer, longer chunks still
        // fill the chip
        const int64_t dh = (int64_t)d.q1 * d.q2;
        const int64_t vec = dh % 4 == 0 ? 4 : 2;
        const int64_t one_level = std::min<int64_t>(kMaxSingleLevel, 16 * (1024 / (dh / vec)));
        if (s > one_level) s = std::max<int64_t>(one_level, kMergeGroup);
    }
    if (s > tiles) s = tiles;
    if (s < 1) s = 1;
    int64_t chunk = tiles > 0 ? (tiles + s - 1) / s : 1;
    s = tiles > 0 ? (tiles + chunk - 1) / chunk : 1;
    const int64_t s_max = (int64_t)kMergeGroup * kMergeGroup;  // two merge levels
    if (s > s_max) {  // widen the chunks
        chunk = (tiles + s_max - 1) / s_max;
        s = (tiles + chunk - 1) / chunk;
    }
    p.n_split = (int32_t)s;
    p.chunk_tiles = (int32_t)chunk;
    const int64_t h = (int64_t)d.p1 * d.p2, dh = (int64_t)d.q1 * d.q2;
    p.n_group = merge_single_level(s, dh) ? 1 : (int32_t)((s + kMergeGroup - 1) / kMergeGroup);
    // each region starts 16-byte aligned (the merge reads partials as float4)
    auto round4 = [](size_t x) { return (x + 3) / 4 * 4; };
    p.part_floats = s > 1 ? round4((size_t)(rows * s * h * (dh + 2))) : 0;
    p.part2_floats = p.n_group > 1 ? round4((size_t)(rows * p.n_group * h * (dh + 2))) : 0;
    const size_t counters = p.n_group > 1 ? (size_t)(rows * h) : 0;
    p.workspace_bytes = (p.part_floats + p.part2_floats + counters) * sizeof(float);
    return p;
}

inline hipError_t launch_plan(const Plan& plan, const DecodeParams& P, hipStream_t s, const KernelEvents& ev) {
    switch (plan.path) {
        case Path::kValu: return launch_decode_valu(P, s, ev);
        case Path::kMfmaSq: return launch_decode_mfma(P, s, ev);
        case Path::kMfmaRebuild: return launch_decode_rebuild(P, s, ev);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kpa
