// Kernel-path selection and split-KV planning (host only).
#pragma once

#include "kpa_common.hpp"

namespace kpa {

enum class Path { kUnsupported, kValu, kMfmaSq };

struct Plan {
    Path path;
    int32_t n_split;
    int32_t chunk_tiles;
    size_t workspace_bytes;
};

inline const char* path_name(Path p) {
    switch (p) {
        case Path::kValu: return "valu";
        case Path::kMfmaSq: return "mfma_bf16";
        default: return "";
    }
}

inline Path select_path(const kpa_dims& d, int32_t n_q) {
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
        // workgroups in flight: the VALU kernel is one 256-thread group per
        // chunk; the matrix-core kernel one wave per (chunk, iF)
        const int64_t target = (p.path == Path::kMfmaSq ? 2LL : 4LL) * cus;
        s = rows > 0 ? (target + rows - 1) / rows : 1;
        const int64_t min_tiles_per_chunk = 2;
        const int64_t cap = (tiles + min_tiles_per_chunk - 1) / min_tiles_per_chunk;
        if (s > cap) s = cap;
    }
    if (s > tiles) s = tiles;
    if (s < 1) s = 1;
    int64_t chunk = tiles > 0 ? (tiles + s - 1) / s : 1;
    s = tiles > 0 ? (tiles + chunk - 1) / chunk : 1;
    if (s > 65535) {  // grid.x limit; widen the chunks
        chunk = (tiles + 65535 - 1) / 65535;
        s = (tiles + chunk - 1) / chunk;
    }
    p.n_split = (int32_t)s;
    p.chunk_tiles = (int32_t)chunk;
    const int64_t h = (int64_t)d.p1 * d.p2, dh = (int64_t)d.q1 * d.q2;
    p.workspace_bytes = s > 1 ? (size_t)(rows * s * h * (dh + 2) * sizeof(float)) : 0;
    return p;
}

inline hipError_t launch_plan(const Plan& plan, const DecodeParams& P, hipStream_t s) {
    switch (plan.path) {
        case Path::kValu: return launch_decode_valu(P, s);
        case Path::kMfmaSq: return launch_decode_mfma(P, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kpa
