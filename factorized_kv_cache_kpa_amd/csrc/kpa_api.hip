// libkpa C ABI: argument checks, split-KV planning and kernel dispatch.
// Declarations and the contract of every entry point are in include/kpa.h.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "kpa_common.hpp"
#include "kpa_dispatch.hpp"

using namespace kpa;

namespace {

bool dims_ok(const kpa_dims* d) {
    if (d->p1 <= 0 || d->p2 <= 0 || d->q1 <= 0 || d->q2 <= 0 || d->r_k <= 0 || d->r_v <= 0) return false;
    if (d->q2 % 2) return false;
    const int64_t h = (int64_t)d->p1 * d->p2, dh = (int64_t)d->q1 * d->q2;
    if (h > KPA_MAX_HEADS || dh > KPA_MAX_HEAD_DIM || h * dh > KPA_MAX_HD) return false;
    if (d->r_k > KPA_MAX_RANK || d->r_v > KPA_MAX_RANK) return false;
    if (!(d->rope_base > 0.f) || !isfinite(d->rope_base)) return false;
    return true;
}

int check_dims(const kpa_dims* d) {
    if (!d) return KPA_ERR_NULL_PTR;
    if (d->dtype != KPA_F32 && d->dtype != KPA_BF16) return KPA_ERR_DTYPE;
    if (!dims_ok(d)) return KPA_ERR_INVALID_DIMS;
    return KPA_OK;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Compute units of the current device, looked up once per device.
int num_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

int check_decode_args(const kpa_dims* d, int32_t batch, int32_t capacity, int32_t max_ctx, int32_t n_q) {
    int st = check_dims(d);
    if (st != KPA_OK) return st;
    if (batch < 0 || capacity < 0 || capacity > KPA_MAX_CAPACITY || max_ctx < 0 || max_ctx > capacity)
        return KPA_ERR_INVALID_ARG;
    if (n_q < 1 || n_q > KPA_MAX_NQ) return KPA_ERR_INVALID_ARG;
    if ((int64_t)batch * n_q > 65535) return KPA_ERR_INVALID_ARG;
    return KPA_OK;
}

}  // namespace

extern "C" {

int kpa_cache_layout(const kpa_dims* dims, int32_t batch, int32_t capacity, kpa_layout_info* out) {
    int st = check_dims(dims);
    if (st != KPA_OK) return st;
    if (!out) return KPA_ERR_NULL_PTR;
    if (batch < 0 || capacity < 0 || capacity > KPA_MAX_CAPACITY) return KPA_ERR_INVALID_ARG;
    Layout L = make_layout(*dims, batch, capacity);
    out->version = KPA_LAYOUT_VERSION;
    out->tile_slots = kTileSlots;
    out->elem_bytes = L.elem_bytes;
    out->n_tiles = L.n_tiles;
    out->tile_bytes = L.tile_bytes;
    for (int c = 0; c < 4; ++c) {
        out->comp_offset[c] = L.off[c];
        out->comp_elems[c] = L.elems[c];
    }
    out->positions_offset = L.positions_off;
    out->total_bytes = L.total_bytes;
    return KPA_OK;
}

size_t kpa_cache_bytes(const kpa_dims* dims, int32_t batch, int32_t capacity) {
    kpa_layout_info info;
    if (kpa_cache_layout(dims, batch, capacity, &info) != KPA_OK) return 0;
    return (size_t)info.total_bytes;
}

int kpa_cache_append(const kpa_dims* dims, void* cache, int32_t batch, int32_t capacity,
                     const void* a_k, const void* b_k, const void* a_v, const void* b_v,
                     const int32_t* positions, const int32_t* slot0, int32_t n_new,
                     uint32_t* dev_status, void* stream) {
    int st = check_dims(dims);
    if (st != KPA_OK) return st;
    if (batch < 0 || capacity < 0 || capacity > KPA_MAX_CAPACITY || n_new < 0 || batch > 65535)
        return KPA_ERR_INVALID_ARG;
    if (batch == 0 || n_new == 0) return KPA_OK;
    if (!cache || !a_k || !b_k || !a_v || !b_v || !positions || !slot0) return KPA_ERR_NULL_PTR;
    if (!aligned(cache, 16)) return KPA_ERR_INVALID_ARG;
    AppendParams P{};
    P.d = *dims;
    P.L = make_layout(*dims, batch, capacity);
    P.cache = static_cast<uint8_t*>(cache);
    P.batch = batch;
    P.capacity = capacity;
    P.in = AppendInputs{a_k, b_k, a_v, b_v, positions, slot0, n_new};
    P.dev_status = dev_status;
    return launch_append(P, static_cast<hipStream_t>(stream)) == hipSuccess ? KPA_OK : KPA_ERR_HIP;
}

// Events the next decode, projection or streaming-read call on this thread
// has stamped with its main kernel's start and end
// (kpa_time_next_decode_kernel).
static thread_local KernelEvents t_kernel_events;

int kpa_project_append(const kpa_dims* dims, void* cache, int32_t batch, int32_t capacity, const void* x,
                       int32_t d_model, const void* w, const int32_t* positions, const int32_t* slot0,
                       int32_t n_new, uint32_t* dev_status, void* stream) {
    // a pending measurement request applies to this call only
    const KernelEvents ev = t_kernel_events;
    t_kernel_events = KernelEvents{};
    int st = check_dims(dims);
    if (st != KPA_OK) return st;
    if (batch < 0 || capacity < 0 || capacity > KPA_MAX_CAPACITY || n_new < 0 || batch > 65535)
        return KPA_ERR_INVALID_ARG;
    if (d_model <= 0 || d_model % 64 != 0 || d_model > (1 << 20)) return KPA_ERR_INVALID_ARG;
    if (batch == 0 || n_new == 0) return KPA_OK;
    const int64_t n_tok = (int64_t)batch * n_new;
    if (n_tok > 65535LL * 32) return KPA_ERR_INVALID_ARG;
    if (!cache || !x || !w || !positions || !slot0) return KPA_ERR_NULL_PTR;
    if (!aligned(cache, 16) || !aligned(x, 16) || !aligned(w, 16)) return KPA_ERR_INVALID_ARG;
    ProjectParams P{};
    P.d = *dims;
    P.L = make_layout(*dims, batch, capacity);
    P.cache = static_cast<uint8_t*>(cache);
    P.capacity = capacity;
    P.n_new = n_new;
    P.n_tok = (int32_t)n_tok;
    P.n_feat = P.L.elems[0] + P.L.elems[1] + P.L.elems[2] + P.L.elems[3];
    P.d_model = d_model;
    P.x = static_cast<const uint16_t*>(x);
    P.w = static_cast<const uint16_t*>(w);
    P.positions = positions;
    P.slot0 = slot0;
    P.dev_status = dev_status;
    return launch_project_append(P, static_cast<hipStream_t>(stream), ev) == hipSuccess ? KPA_OK : KPA_ERR_HIP;
}

int kpa_stream_xor(const void* buf, size_t bytes, uint32_t* partial, int32_t n_blocks, void* stream) {
    // a pending measurement request applies to this call only
    const KernelEvents ev = t_kernel_events;
    t_kernel_events = KernelEvents{};
    if (!buf || !partial) return KPA_ERR_NULL_PTR;
    if (bytes == 0 || bytes % 16 != 0 || bytes > ((size_t)1 << 40) || !aligned(buf, 16)) return KPA_ERR_INVALID_ARG;
    if (n_blocks < 1 || n_blocks > 65535) return KPA_ERR_INVALID_ARG;
    return launch_stream_xor(buf, (int64_t)bytes, partial, n_blocks, static_cast<hipStream_t>(stream), ev) == hipSuccess
               ? KPA_OK
               : KPA_ERR_HIP;
}

size_t kpa_decode_workspace_bytes(const kpa_dims* dims, int32_t batch, int32_t max_ctx, int32_t n_q,
                                  int32_t num_splits) {
    if (check_decode_args(dims, batch, max_ctx, max_ctx, n_q) != KPA_OK) return 0;
    Plan plan = plan_decode(*dims, batch, max_ctx, n_q, num_splits, num_cus());
    return plan.workspace_bytes;
}


// factored: the query is (a_q, b_q, r_q); otherwise the dense q.  app: new
// tokens to append to the (writable) cache first, or NULL.
static int decode_common(const kpa_dims* dims, const void* cache, int32_t batch, int32_t capacity,
                         const int32_t* ctx_len, int32_t max_ctx, int32_t n_q, int32_t causal, bool factored,
                         const float* q, const float* a_q, const float* b_q, int32_t r_q,
                         const int32_t* q_pos, float* out, float* lse,
                         void* workspace, size_t workspace_bytes, int32_t num_splits,
                         uint32_t* dev_status, void* stream, const AppendInputs* app = nullptr) {
    // a pending measurement request applies to this call only
    const KernelEvents ev = t_kernel_events;
    t_kernel_events = KernelEvents{};
    int st = check_decode_args(dims, batch, capacity, max_ctx, n_q);
    if (st != KPA_OK) return st;
    if (factored && (r_q < 1 || r_q > KPA_MAX_RANK)) return KPA_ERR_INVALID_DIMS;
    if (app && app->n_new < 0) return KPA_ERR_INVALID_ARG;
    if (batch == 0) return KPA_OK;
    if (app && app->n_new > 0 &&
        (!app->a_k || !app->b_k || !app->a_v || !app->b_v || !app->positions || !app->slot0))
        return KPA_ERR_NULL_PTR;
    if (!cache || !ctx_len || !q_pos || !out || (factored ? (!a_q || !b_q) : !q)) return KPA_ERR_NULL_PTR;
    if (!aligned(cache, 16) || !aligned(out, 16) || (!factored && !aligned(q, 16)) ||
        (factored && (!aligned(a_q, 16) || !aligned(b_q, 16))))
        return KPA_ERR_INVALID_ARG;
    Plan plan = plan_decode(*dims, batch, max_ctx, n_q, num_splits, num_cus());
    if (plan.path == Path::kUnsupported) return KPA_ERR_UNSUPPORTED;
    if (plan.workspace_bytes > 0) {
        if (!workspace || workspace_bytes < plan.workspace_bytes) return KPA_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return KPA_ERR_INVALID_ARG;
    }
    DecodeParams P{};
    P.d = *dims;
    P.L = make_layout(*dims, batch, capacity);
    P.cache = static_cast<const uint8_t*>(cache);
    P.batch = batch;
    P.capacity = capacity;
    P.max_ctx = max_ctx;
    P.n_q = n_q;
    P.causal = causal ? 1 : 0;
    P.ctx_len = ctx_len;
    P.q = q;
    P.a_q = a_q;
    P.b_q = b_q;
    P.r_q = factored ? r_q : 0;
    P.q_pos = q_pos;
    P.out = out;
    P.lse = lse;
    P.dev_status = dev_status;
    P.n_split = plan.n_split;
    P.chunk_tiles = plan.chunk_tiles;
    const int h = dims->p1 * dims->p2, dh = dims->q1 * dims->q2;
    P.n_group = plan.n_group;
    if (plan.n_split > 1) {
        float* ws = static_cast<float*>(workspace);
        P.part_o = ws;
        P.part_ml = P.part_o + (size_t)batch * n_q * plan.n_split * h * dh;
        if (plan.n_group > 1) {
            P.part2_o = ws + plan.part_floats;
            P.part2_ml = P.part2_o + (size_t)batch * n_q * plan.n_group * h * dh;
            P.merge_count = reinterpret_cast<uint32_t*>(ws + plan.part_floats + plan.part2_floats);
        }
    }
    P.q_scale = (float)(1.4426950408889634 / (dims->r_k * sqrt((double)dh)));
    P.v_scale = (float)(1.0 / dims->r_v);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (app && app->n_new > 0) {
        if (plan.path == Path::kMfmaSq && n_q == 1) {
            // the single-query matrix-core kernels write the new tokens themselves
            P.app = *app;
            P.cache_w = const_cast<uint8_t*>(P.cache);
        } else {
            AppendParams A{};
            A.d = *dims;
            A.L = P.L;
            A.cache = const_cast<uint8_t*>(P.cache);
            A.batch = batch;
            A.capacity = capacity;
            A.in = *app;
            A.dev_status = dev_status;
            if (launch_append(A, s) != hipSuccess) return KPA_ERR_HIP;
        }
    }
    hipError_t e = launch_plan(plan, P, s, ev);
    if (e != hipSuccess) return KPA_ERR_HIP;
    if (plan.n_split > 1 && launch_merge(P, s) != hipSuccess) return KPA_ERR_HIP;
    return KPA_OK;
}

int kpa_time_next_decode_kernel(void* start_event, void* stop_event) {
    if ((start_event == nullptr) != (stop_event == nullptr)) return KPA_ERR_NULL_PTR;
    t_kernel_events = KernelEvents{static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
    return KPA_OK;
}

int kpa_decode(const kpa_dims* dims, const void* cache, int32_t batch, int32_t capacity,
               const int32_t* ctx_len, int32_t max_ctx, const float* q, const int32_t* q_pos,
               float* out, float* lse, void* workspace, size_t workspace_bytes,
               int32_t num_splits, uint32_t* dev_status, void* stream) {
    return decode_common(dims, cache, batch, capacity, ctx_len, max_ctx, 1, 0, false, q, nullptr, nullptr, 0, q_pos,
                         out, lse, workspace, workspace_bytes, num_splits, dev_status, stream);
}

int kpa_decode_multiq(const kpa_dims* dims, const void* cache, int32_t batch, int32_t capacity,
                      const int32_t* ctx_len, int32_t max_ctx, int32_t n_q, int32_t causal,
                      const float* q, const int32_t* q_pos, float* out, float* lse,
                      void* workspace, size_t workspace_bytes, int32_t num_splits,
                      uint32_t* dev_status, void* stream) {
    return decode_common(dims, cache, batch, capacity, ctx_len, max_ctx, n_q, causal, false, q, nullptr, nullptr, 0,
                         q_pos, out, lse, workspace, workspace_bytes, num_splits, dev_status, stream);
}

int kpa_decode_factored(const kpa_dims* dims, int32_t r_q, const void* cache, int32_t batch, int32_t capacity,
                        const int32_t* ctx_len, int32_t max_ctx, int32_t n_q, int32_t causal,
                        const float* a_q, const float* b_q, const int32_t* q_pos, float* out, float* lse,
                        void* workspace, size_t workspace_bytes, int32_t num_splits,
                        uint32_t* dev_status, void* stream) {
    return decode_common(dims, cache, batch, capacity, ctx_len, max_ctx, n_q, causal, true, nullptr, a_q, b_q, r_q,
                         q_pos, out, lse, workspace, workspace_bytes, num_splits, dev_status, stream);
}

int kpa_append_decode(const kpa_dims* dims, void* cache, int32_t batch, int32_t capacity,
                      const void* a_k, const void* b_k, const void* a_v, const void* b_v,
                      const int32_t* positions, const int32_t* slot0, int32_t n_new,
                      const int32_t* ctx_len, int32_t max_ctx, int32_t n_q, int32_t causal,
                      const float* q, const int32_t* q_pos, float* out, float* lse,
                      void* workspace, size_t workspace_bytes, int32_t num_splits,
                      uint32_t* dev_status, void* stream) {
    const AppendInputs app{a_k, b_k, a_v, b_v, positions, slot0, n_new};
    return decode_common(dims, cache, batch, capacity, ctx_len, max_ctx, n_q, causal, false, q, nullptr, nullptr, 0,
                         q_pos, out, lse, workspace, workspace_bytes, num_splits, dev_status, stream, &app);
}

}  // extern "C"

// Scratch of kpa_append_decode_noalloc (the split-KV partials): one array of
// KPA_NOALLOC_SCRATCH_BYTES per device, for the life of the process.  In host
// code `scratch` names a host-side stand-in; the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) uint8_t scratch[KPA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (its address set up on first use).
int scratch_of_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KPA_ERR_HIP;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KPA_ERR_HIP;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return KPA_OK;
}

}  // namespace

extern "C" {

int kpa_append_decode_noalloc(const kpa_dims* dims, void* cache, int32_t batch, int32_t capacity,
                              const void* a_k, const void* b_k, const void* a_v, const void* b_v,
                              const int32_t* positions, const int32_t* slot0, int32_t n_new,
                              const int32_t* ctx_len, int32_t max_ctx, int32_t n_q, int32_t causal,
                              const float* q, const int32_t* q_pos, float* out, float* lse,
                              int32_t num_splits, uint32_t* dev_status, void* stream) {
    int st = check_decode_args(dims, batch, capacity, max_ctx, n_q);
    if (st != KPA_OK) {
        t_kernel_events = KernelEvents{};  // a pending measurement request applies to this call only
        return st;
    }
    const Plan plan = plan_decode(*dims, batch, max_ctx, n_q, num_splits, num_cus());
    void* ws = nullptr;
    if (plan.workspace_bytes > 0) {
        if (plan.workspace_bytes > KPA_NOALLOC_SCRATCH_BYTES) {
            t_kernel_events = KernelEvents{};
            return KPA_ERR_WORKSPACE;
        }
        st = scratch_of_current_device(&ws);
        if (st != KPA_OK) {
            t_kernel_events = KernelEvents{};
            return st;
        }
    }
    const AppendInputs app{a_k, b_k, a_v, b_v, positions, slot0, n_new};
    return decode_common(dims, cache, batch, capacity, ctx_len, max_ctx, n_q, causal, false, q, nullptr, nullptr, 0,
                         q_pos, out, lse, ws, ws ? (size_t)KPA_NOALLOC_SCRATCH_BYTES : 0, num_splits, dev_status,
                         stream, &app);
}

const char* kpa_status_string(int status) {
    switch (status) {
        case KPA_OK: return "ok";
        case KPA_ERR_INVALID_DIMS: return "invalid dims (non-positive split or rank, odd q2, or above the build limits)";
        case KPA_ERR_NULL_PTR: return "a required pointer is NULL";
        case KPA_ERR_DTYPE: return "unknown cache element type";
        case KPA_ERR_WORKSPACE: return "workspace missing or smaller than kpa_decode_workspace_bytes()";
        case KPA_ERR_UNSUPPORTED: return "shape not supported by any kernel in this build";
        case KPA_ERR_HIP: return "HIP runtime error";
        case KPA_ERR_INVALID_ARG: return "argument out of range or misaligned pointer";
        default: return "unknown status";
    }
}

const char* kpa_decode_path(const kpa_dims* dims, int32_t n_q) {
    if (check_dims(dims) != KPA_OK || n_q < 1 || n_q > KPA_MAX_NQ) return "";
    return path_name(select_path(*dims, n_q));
}

}  // extern "C"
