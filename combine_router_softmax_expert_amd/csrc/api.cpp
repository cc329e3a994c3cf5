// api.cpp -- the C ABI of libmoe_ep.so (declared in include/moe_ep.h): argument
// validation, workspace layout, launch sequencing on the caller's stream, the
// handle's generation check and optional per-kernel event timing.
#include "moe_ep.h"

#include <hip/hip_runtime.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <new>
#include <string>
#include <vector>

#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

constexpr size_t kAlign = 256;
constexpr int kFp8Block = 128;   // channels per FP8 scale, per token
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Opens one library call: clears this thread's error text (so moe_last_error
// always describes the latest call) and pushes a roctx range, so that a
// rocprofv3 --marker-trace shows each call of the path (route, dispatch and its
// halves, stub, combine and its halves) around the kernels it launched.
struct CallScope {
    explicit CallScope(const char* name) {
        g_last_error.clear();
        roctxRangePushA(name);
    }
    ~CallScope() { roctxRangePop(); }
    CallScope(const CallScope&) = delete;
    CallScope& operator=(const CallScope&) = delete;
};

// A failing status with its reason, for moe_last_error.
moe_status fail(moe_status s, const char* why) {
    g_last_error = why;
    return s;
}

moe_status bad_scales() { return fail(MOE_ERR_INVALID_ARG, "scales: required for FP8 dispatch, NULL for bf16"); }

// Row arrays are moved 16 bytes per lane; the 4-byte arrays are read a word at
// a time, wave-uniform ones through the scalar cache, which drops the low two
// address bits.  NULL passes (the null checks come first).
moe_status check_alignment(std::initializer_list<const void*> rows, std::initializer_list<const void*> words) {
    for (const void* p : rows)
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
            return fail(MOE_ERR_INVALID_ARG, "a row buffer is not 16-byte aligned");
    for (const void* p : words)
        if (reinterpret_cast<uintptr_t>(p) % 4 != 0)
            return fail(MOE_ERR_INVALID_ARG, "logits, topk_ids, topk_w or a scale array is not 4-byte aligned");
    return MOE_OK;
}

struct TimingRecord {
    const char* name;
    hipEvent_t start, stop;
};

}  // namespace

struct moe_ctx {
    moe_shape shape;
    moe::Dims d;
    // byte offsets of the workspace arrays
    size_t o_n, o_N, o_expert_off, o_rank_recv_off, o_send_off, o_recv_off, o_C, o_bucket_rank, o_send_pos,
        o_recv_pos, o_send_to_recv, o_recv_to_send, o_send_meta, o_recv_meta, o_bad_ids, ws_bytes;
    uint64_t generation = 0;
    uint64_t received = 0;       // generation whose receive side is complete (exchange or direct pack)
    uint64_t combine_sent = 0;   // generation whose reverse exchange was issued
    uint64_t direct_sent = 0;    // generation dispatched by moe_dispatch_direct
    void* workspace = nullptr;   // workspace of the latest dispatch (the split receive phase reads its maps)
    int static_device = -1;      // moe_dispatch_noalloc: the device whose static workspace the latest dispatch used
    uint64_t static_claim = 0;   // and that dispatch's claim on it (0: the latest dispatch used a caller workspace)
    bool timing = false;
    bool debug = false;    // MOE_EP_DEBUG: validate ids on the device (and synchronise) before dispatching
    std::vector<TimingRecord> records;
    std::vector<hipEvent_t> free_events;
};

namespace {

moe_status hip_fail(hipError_t e, const char* where) {
    g_last_error = std::string(where) + ": " + hipGetErrorString(e);
    return MOE_ERR_HIP;
}

hipEvent_t take_event(moe_ctx* ctx) {
    if (!ctx->free_events.empty()) {
        hipEvent_t e = ctx->free_events.back();
        ctx->free_events.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Launches one kernel through `fn`; when timing is on, the launch carries a
// start and a stop event that bracket the kernel's execution.
template <typename Fn>
moe_status launch(moe_ctx* ctx, const char* name, hipStream_t st, Fn&& fn, bool timed = true) {
    (void)st;
    hipEvent_t a = nullptr, b = nullptr;
    timed = timed && ctx->timing;
    if (timed) {
        a = take_event(ctx);
        b = take_event(ctx);
        if (!a || !b) return hip_fail(hipErrorOutOfMemory, "hipEventCreate");
    }
    moe::launch_timing = {a, b};
    hipError_t e = fn();
    moe::launch_timing = {};
    if (e != hipSuccess) return hip_fail(e, name);
    if (timed) ctx->records.push_back({name, a, b});
    return MOE_OK;
}

moe::Workspace carve(const moe_ctx* ctx, void* base) {
    char* p = static_cast<char*>(base);
    moe::Workspace w;
    w.n = reinterpret_cast<int32_t*>(p + ctx->o_n);
    w.N = reinterpret_cast<int32_t*>(p + ctx->o_N);
    w.expert_off = reinterpret_cast<int32_t*>(p + ctx->o_expert_off);
    w.rank_recv_off = reinterpret_cast<int32_t*>(p + ctx->o_rank_recv_off);
    w.send_off = reinterpret_cast<int32_t*>(p + ctx->o_send_off);
    w.recv_off = reinterpret_cast<int32_t*>(p + ctx->o_recv_off);
    w.C = reinterpret_cast<int32_t*>(p + ctx->o_C);
    w.bucket_rank = reinterpret_cast<int32_t*>(p + ctx->o_bucket_rank);
    w.send_pos = reinterpret_cast<int32_t*>(p + ctx->o_send_pos);
    w.recv_pos = reinterpret_cast<int32_t*>(p + ctx->o_recv_pos);
    w.send_to_recv = reinterpret_cast<int32_t*>(p + ctx->o_send_to_recv);
    w.recv_to_send = reinterpret_cast<int32_t*>(p + ctx->o_recv_to_send);
    w.send_meta = p + ctx->o_send_meta;
    w.recv_meta = p + ctx->o_recv_meta;
    w.bad_ids = reinterpret_cast<int32_t*>(p + ctx->o_bad_ids);
    return w;
}

// The arrays the expert stage and the combine read, taken from the handle.
moe::Workspace from_handle(const moe_handle* h) {
    moe::Workspace w{};
    w.rank_recv_off = const_cast<int32_t*>(h->rank_recv_offsets);
    w.recv_pos = const_cast<int32_t*>(h->recv_pos);
    w.recv_meta = const_cast<moe_meta*>(h->recv_meta);
    return w;
}

// Whether the kernels that work on a handle's rows take the token-affine layout
// (moe::token_affine): after a direct dispatch, whose pack wrote the receive
// rows in that layout, or everywhere when MOE_EP_LAYOUT=tokens asks for it.
bool affine_layout(const moe_ctx* ctx, const moe_handle* h) {
    if (!moe::token_affine(ctx->d)) return false;
    return h->generation == ctx->direct_sent || ctx->d.layout == moe::Layout::kTokens;
}

// Publishes a dispatch: bumps the ctx generation and points the handle at the
// workspace arrays (no send-side record when the rows went straight to their
// receive rows).
void fill_handle(moe_ctx* ctx, const moe::Workspace& ws, moe_handle* handle, bool with_send) {
    ctx->generation += 1;
    ctx->static_claim = 0;   // moe_dispatch_noalloc sets its claim after this
    handle->expert_counts = ws.N;
    handle->expert_offsets = ws.expert_off;
    handle->rank_recv_offsets = ws.rank_recv_off;
    handle->count_matrix = ws.C;
    handle->rank_expert_counts = ws.n;
    handle->send_offsets = ws.send_off;
    handle->recv_offsets = ws.recv_off;
    handle->send_pos = ws.send_pos;
    handle->recv_pos = ws.recv_pos;
    handle->send_meta = with_send ? static_cast<const moe_meta*>(ws.send_meta) : nullptr;
    handle->recv_meta = static_cast<const moe_meta*>(ws.recv_meta);
    handle->ctx = ctx;
    handle->generation = ctx->generation;
}

// Debug mode: count invalid ids on the device, wait for the answer and refuse
// the dispatch if there are any (before any payload kernel is launched).
moe_status validate_ids(moe_ctx* ctx, const moe::Dims& d, const int32_t* topk_ids, const moe::Workspace& ws,
                        hipStream_t st) {
    if (!ctx->debug) return MOE_OK;
    hipError_t e = moe::launch_validate_ids(d, topk_ids, ws.bad_ids, st);
    if (e != hipSuccess) return hip_fail(e, "validate_ids");
    int32_t bad = 0;
    e = hipMemcpyAsync(&bad, ws.bad_ids, sizeof(bad), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, "validate_ids");
    if (bad != 0) {
        g_last_error = "topk_ids: " + std::to_string(bad) + " assignment(s) out of range or repeated within a token";
        return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

// The count kernel (and the scan kernel unless one workgroup does both).
moe_status count_and_scan(moe_ctx* ctx, const moe::Dims& d, const int32_t* topk_ids, const moe::Workspace& ws,
                          hipStream_t st, bool timed = true) {
    moe_status s = launch(ctx, "count", st, [&] { return moe::launch_count(d, topk_ids, ws, st); }, timed);
    if (s == MOE_OK && !moe::count_is_single(d))
        s = launch(ctx, "scan", st, [&] { return moe::launch_scan(d, ws, st); }, timed);
    return s;
}

moe_status check_handle(const moe_ctx* ctx, const moe_handle* h) {
    if (!h) return fail(MOE_ERR_INVALID_ARG, "handle is NULL");
    if (h->ctx != ctx || h->generation != ctx->generation || ctx->generation == 0)
        return fail(MOE_ERR_STALE_HANDLE, "the handle is not from this ctx's latest dispatch");
    if (ctx->static_claim != 0 && moe::static_workspace_latest_claim(ctx->static_device) != ctx->static_claim)
        return fail(MOE_ERR_STALE_HANDLE,
                    "a later moe_dispatch_noalloc on this device has reused the static workspace the handle points into");
    return MOE_OK;
}

// The stages after the exchange need the receive side of the handle's dispatch.
moe_status check_received(const moe_ctx* ctx, const moe_handle* h, const char* who) {
    moe_status s = check_handle(ctx, h);
    if (s != MOE_OK) return s;
    if (ctx->received != h->generation) {
        g_last_error = std::string(who) + ": moe_dispatch_recv has not been issued for this handle";
        return MOE_ERR_INVALID_ARG;
    }
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_STALE_HANDLE: return "stale or foreign dispatch handle";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_NO_MEMORY: return "host allocation failed";
    }
    return "unknown status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status moe_ctx_create(const moe_shape* shape, moe_ctx** out) {
    g_last_error.clear();
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!shape) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
    const moe_shape s = *shape;
    if (s.num_ranks < 1 || s.tokens_per_rank < 0 || s.num_experts < 1 || s.top_k < 1 || s.hidden < 8 ||
        s.num_experts % s.num_ranks != 0 || s.top_k > s.num_experts || s.hidden % 8 != 0 ||
        (s.dispatch_dtype != MOE_DTYPE_BF16 && s.dispatch_dtype != MOE_DTYPE_FP8_E4M3))
        return fail(MOE_ERR_INVALID_ARG,
                    "shape: needs num_ranks >= 1, tokens_per_rank >= 0, 1 <= top_k <= num_experts, num_experts a "
                    "multiple of num_ranks, hidden a positive multiple of 8 and a known dispatch_dtype");
    const bool fp8 = s.dispatch_dtype == MOE_DTYPE_FP8_E4M3;
    const long long T = (long long)s.num_ranks * s.tokens_per_rank;
    const long long Na = T * s.top_k;
    if (s.num_experts > 1024 || s.num_experts / s.num_ranks > 32767 || s.top_k > 32 || s.hidden > 65536 ||
        (fp8 && s.hidden % kFp8Block != 0) || Na >= (1LL << 31) ||
        Na * (s.hidden / 1024 + 1) >= (1LL << 31) ||
        // a row kernel's grid is at most N_a + P rows of H/8 units rounded up to a
        // workgroup (< 512 more), in one dimension of fewer than 2^32 work-items
        (Na + s.num_ranks) * (s.hidden / 8 + 512) >= (1LL << 32))
        return fail(MOE_ERR_UNSUPPORTED, "shape outside the supported limits of moe_ctx_create");

    moe_ctx* ctx = new (std::nothrow) moe_ctx();
    if (!ctx) return fail(MOE_ERR_NO_MEMORY, "host allocation of the ctx failed");
    ctx->shape = s;
    moe::Dims& d = ctx->d;
    d.P = s.num_ranks;
    d.Tp = s.tokens_per_rank;
    d.T = (int)T;
    d.E = s.num_experts;
    d.Ep = s.num_experts / s.num_ranks;
    d.k = s.top_k;
    d.H = s.hidden;
    d.fp8 = fp8;
    d.Na = Na;
    d.row_units = fp8 ? s.hidden / 16 : s.hidden / 8;
    d.out_units = s.hidden / 8;
    d.scales = fp8 ? s.hidden / kFp8Block : 0;
    // MOE_EP_CACHE_POLICY=temporal|streaming overrides the size-based choice (for A/B measurements)
    d.policy = moe::CachePolicy::kAuto;
    if (const char* pol = std::getenv("MOE_EP_CACHE_POLICY")) {
        if (std::strcmp(pol, "temporal") == 0) d.policy = moe::CachePolicy::kTemporal;
        if (std::strcmp(pol, "streaming") == 0) d.policy = moe::CachePolicy::kStreaming;
    }
    // MOE_EP_DEBUG=1: dispatch checks the ids on the device first (see validate_ids)
    if (const char* dbg = std::getenv("MOE_EP_DEBUG")) ctx->debug = std::strcmp(dbg, "0") != 0 && dbg[0] != 0;
    // MOE_EP_COUNT_PATH=separate|fused overrides the size-based choice (for A/B tests)
    d.count_path = moe::CountPath::kAuto;
    if (const char* cp = std::getenv("MOE_EP_COUNT_PATH")) {
        if (std::strcmp(cp, "separate") == 0) d.count_path = moe::CountPath::kSeparate;
        if (std::strcmp(cp, "fused") == 0) d.count_path = moe::CountPath::kFused;
    }
    // MOE_EP_LAYOUT=rows|tokens overrides the size-based workgroup layout (for A/B tests)
    d.layout = moe::Layout::kAuto;
    if (const char* lay = std::getenv("MOE_EP_LAYOUT")) {
        if (std::strcmp(lay, "rows") == 0) d.layout = moe::Layout::kRows;
        if (std::strcmp(lay, "tokens") == 0) d.layout = moe::Layout::kTokens;
    }

    const size_t P = d.P, E = d.E, tk = (size_t)Na;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
    const moe::CountLayout cl = moe::count_layout(P, E);   // the count arrays first, as the counting pack expects
    ctx->o_n = cl.n;
    ctx->o_N = cl.N;
    ctx->o_expert_off = cl.expert_off;
    ctx->o_rank_recv_off = cl.rank_recv_off;
    ctx->o_send_off = cl.send_off;
    ctx->o_recv_off = cl.recv_off;
    ctx->o_C = cl.C;
    off = cl.end;
    ctx->o_bucket_rank = take(4 * tk);
    ctx->o_send_pos = take(4 * tk);
    ctx->o_recv_pos = take(4 * tk);
    ctx->o_send_to_recv = take(4 * tk);
    ctx->o_recv_to_send = take(4 * tk);
    ctx->o_send_meta = take(sizeof(moe_meta) * tk);
    ctx->o_recv_meta = take(sizeof(moe_meta) * tk);
    ctx->o_bad_ids = take(4);
    ctx->ws_bytes = off;
    *out = ctx;
    return MOE_OK;
}

void moe_ctx_destroy(moe_ctx* ctx) {
    if (!ctx) return;
    for (auto& r : ctx->records) {
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    for (auto e : ctx->free_events) (void)hipEventDestroy(e);
    delete ctx;
}

size_t moe_workspace_bytes(const moe_ctx* ctx) { return ctx ? ctx->ws_bytes : 0; }
size_t moe_dispatch_row_bytes(const moe_ctx* ctx) { return ctx ? (size_t)ctx->d.row_units * 16 : 0; }
int32_t moe_scales_per_row(const moe_ctx* ctx) { return ctx ? ctx->d.scales : 0; }
int64_t moe_num_assignments(const moe_ctx* ctx) { return ctx ? ctx->d.Na : 0; }

moe_status moe_route_topk(moe_ctx* ctx, const float* logits, int32_t* topk_ids, float* topk_w, void* stream) {
    const CallScope scope("moe_route_topk");
    if (!ctx) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
    if (ctx->d.T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_w) return fail(MOE_ERR_INVALID_ARG, "logits, topk_ids or topk_w is NULL");
    if (moe_status a = check_alignment({}, {logits, topk_ids, topk_w}); a != MOE_OK) return a;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const moe::Dims d = ctx->d;
    return launch(ctx, "route_topk", st, [&] { return moe::launch_route_topk(d, logits, topk_ids, topk_w, st); });
}

}  // extern "C"

namespace {

// The send half of the base dispatch into `workspace` (already checked): count,
// scan and pack.  `extras` enables per-kernel timing events and the debug-mode
// id check, which create events or read back to the host.
moe_status dispatch_send_impl(moe_ctx* ctx, const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                              void* workspace, void* send_buf, float* send_scales, moe_handle* handle,
                              hipStream_t st, bool extras) {
    const moe::Dims d = ctx->d;
    const moe::Workspace ws = carve(ctx, workspace);
    if (d.T > 0) {
        moe_status s = extras ? validate_ids(ctx, d, topk_ids, ws, st) : MOE_OK;
        if (s != MOE_OK) return s;
        const bool fused = moe::pack_counts(d);
        if (!fused) s = count_and_scan(ctx, d, topk_ids, ws, st, extras);
        if (s == MOE_OK)
            s = launch(ctx, fused ? "count_pack" : "pack", st, [&] {
                return moe::launch_pack(d, x, topk_ids, topk_w, ws, send_buf, send_scales, false, st);
            }, extras);
        if (s != MOE_OK) return s;
    }
    ctx->workspace = workspace;
    fill_handle(ctx, ws, handle, true);
    return MOE_OK;
}

// The receive half (the exchange) of the latest base dispatch (handle already checked).
moe_status dispatch_recv_impl(moe_ctx* ctx, const moe_handle* handle, const void* send_buf, const float* send_scales,
                              void* recv_buf, float* recv_scales, hipStream_t st, bool extras) {
    const moe::Dims d = ctx->d;
    if (d.T > 0) {
        const moe::Workspace ws = carve(ctx, ctx->workspace);
        moe_status s = launch(ctx, "exchange", st, [&] {
            return moe::launch_exchange(d, ws, send_buf, send_scales, recv_buf, recv_scales, affine_layout(ctx, handle),
                                        st);
        }, extras);
        if (s != MOE_OK) return s;
    }
    ctx->received = ctx->generation;
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_dispatch_send(moe_ctx* ctx, const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                             void* workspace, size_t workspace_bytes, void* send_buf, float* send_scales,
                             moe_handle* handle, void* stream) {
    const CallScope scope("moe_dispatch_send");
    if (!ctx || !handle) return fail(MOE_ERR_INVALID_ARG, "ctx or handle is NULL");
    const moe::Dims d = ctx->d;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
        return fail(MOE_ERR_INVALID_ARG, "workspace is NULL or not 256-byte aligned");
    if (workspace_bytes < ctx->ws_bytes) return fail(MOE_ERR_WORKSPACE, "workspace_bytes < moe_workspace_bytes(ctx)");
    if (d.T > 0 && (!x || !topk_ids || !topk_w || !send_buf))
        return fail(MOE_ERR_INVALID_ARG, "x, topk_ids, topk_w or send_buf is NULL");
    if (d.fp8 ? (d.T > 0 && !send_scales) : send_scales != nullptr) return bad_scales();
    if (moe_status a = check_alignment({x, send_buf}, {topk_ids, topk_w, send_scales}); a != MOE_OK) return a;
    return dispatch_send_impl(ctx, x, topk_ids, topk_w, workspace, send_buf, send_scales, handle,
                              static_cast<hipStream_t>(stream), true);
}

moe_status moe_dispatch_recv(moe_ctx* ctx, const moe_handle* handle, const void* send_buf, const float* send_scales,
                             void* recv_buf, float* recv_scales, void* stream) {
    const CallScope scope("moe_dispatch_recv");
    if (!ctx) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
    moe_status s = check_handle(ctx, handle);
    if (s != MOE_OK) return s;
    if (!handle->send_meta || ctx->received == ctx->generation) {
        g_last_error = "moe_dispatch_recv: the handle's receive side is already complete";
        return MOE_ERR_INVALID_ARG;
    }
    const moe::Dims d = ctx->d;
    if (d.T > 0 && (!send_buf || !recv_buf)) return fail(MOE_ERR_INVALID_ARG, "send_buf or recv_buf is NULL");
    if (d.fp8 ? (d.T > 0 && (!send_scales || !recv_scales)) : (send_scales || recv_scales))
        return bad_scales();
    if (moe_status a = check_alignment({send_buf, recv_buf}, {send_scales, recv_scales}); a != MOE_OK) return a;
    return dispatch_recv_impl(ctx, handle, send_buf, send_scales, recv_buf, recv_scales,
                              static_cast<hipStream_t>(stream), true);
}

moe_status moe_dispatch(moe_ctx* ctx, const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                        void* workspace, size_t workspace_bytes, void* send_buf, float* send_scales,
                        void* recv_buf, float* recv_scales, moe_handle* handle, void* stream) {
    const CallScope scope("moe_dispatch");
    if (!ctx || !handle) return fail(MOE_ERR_INVALID_ARG, "ctx or handle is NULL");
    const moe::Dims d = ctx->d;
    // every argument is checked before anything is enqueued
    if (d.T > 0 && !recv_buf) return fail(MOE_ERR_INVALID_ARG, "recv_buf is NULL");
    if (d.fp8 ? (d.T > 0 && !recv_scales) : recv_scales != nullptr) return bad_scales();
    if (moe_status a = check_alignment({recv_buf}, {recv_scales}); a != MOE_OK) return a;
    moe_status s = moe_dispatch_send(ctx, x, topk_ids, topk_w, workspace, workspace_bytes, send_buf, send_scales,
                                     handle, stream);
    if (s != MOE_OK) return s;
    return moe_dispatch_recv(ctx, handle, send_buf, send_scales, recv_buf, recv_scales, stream);
}

moe_status moe_dispatch_noalloc(moe_ctx* ctx, const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                                void* send_buf, float* send_scales, void* recv_buf, float* recv_scales,
                                moe_handle* handle, void* stream) {
    const CallScope scope("moe_dispatch_noalloc");
    if (!ctx || !handle) return fail(MOE_ERR_INVALID_ARG, "ctx or handle is NULL");
    const moe::Dims d = ctx->d;
    if (ctx->ws_bytes > moe::kStaticWorkspaceBytes)
        return fail(MOE_ERR_WORKSPACE,
                    "moe_workspace_bytes(ctx) exceeds the library's static workspace of 8 MiB: use moe_dispatch with "
                    "a caller workspace");
    if (d.T > 0 && (!x || !topk_ids || !topk_w || !send_buf || !recv_buf))
        return fail(MOE_ERR_INVALID_ARG, "x, topk_ids, topk_w, send_buf or recv_buf is NULL");
    if (d.fp8 ? (d.T > 0 && (!send_scales || !recv_scales)) : (send_scales || recv_scales)) return bad_scales();
    if (moe_status a = check_alignment({x, send_buf, recv_buf}, {topk_ids, topk_w, send_scales, recv_scales});
        a != MOE_OK)
        return a;
    int device = -1;
    void* workspace = nullptr;
    if (hipError_t e = moe::static_workspace(&device, &workspace); e != hipSuccess)
        return hip_fail(e, "hipGetSymbolAddress of the static workspace");
    hipStream_t st = static_cast<hipStream_t>(stream);
    // no timing events and no debug read-back here: both would create runtime objects
    moe_status s = dispatch_send_impl(ctx, x, topk_ids, topk_w, workspace, send_buf, send_scales, handle, st, false);
    if (s == MOE_OK) s = dispatch_recv_impl(ctx, handle, send_buf, send_scales, recv_buf, recv_scales, st, false);
    if (s != MOE_OK) return s;
    ctx->static_device = device;
    ctx->static_claim = moe::static_workspace_claim(device);
    return MOE_OK;
}

moe_status moe_dispatch_direct(moe_ctx* ctx, const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                               void* workspace, size_t workspace_bytes, void* recv_buf, float* recv_scales,
                               moe_handle* handle, void* stream) {
    const CallScope scope("moe_dispatch_direct");
    if (!ctx || !handle) return fail(MOE_ERR_INVALID_ARG, "ctx or handle is NULL");
    const moe::Dims d = ctx->d;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
        return fail(MOE_ERR_INVALID_ARG, "workspace is NULL or not 256-byte aligned");
    if (workspace_bytes < ctx->ws_bytes) return fail(MOE_ERR_WORKSPACE, "workspace_bytes < moe_workspace_bytes(ctx)");
    if (d.T > 0 && (!x || !topk_ids || !topk_w || !recv_buf))
        return fail(MOE_ERR_INVALID_ARG, "x, topk_ids, topk_w or recv_buf is NULL");
    if (d.fp8 ? (d.T > 0 && !recv_scales) : recv_scales != nullptr) return bad_scales();
    if (moe_status a = check_alignment({x, recv_buf}, {topk_ids, topk_w, recv_scales}); a != MOE_OK) return a;

    const moe::Workspace ws = carve(ctx, workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (d.T > 0) {
        moe_status s = validate_ids(ctx, d, topk_ids, ws, st);
        if (s != MOE_OK) return s;
        const bool fused = moe::pack_counts(d);
        if (!fused) s = count_and_scan(ctx, d, topk_ids, ws, st);
        if (s == MOE_OK)
            s = launch(ctx, fused ? "count_pack_direct" : "pack_direct", st, [&] {
                return moe::launch_pack(d, x, topk_ids, topk_w, ws, recv_buf, recv_scales, true, st);
            });
        if (s != MOE_OK) return s;
    }
    ctx->workspace = workspace;
    fill_handle(ctx, ws, handle, false);
    ctx->received = ctx->generation;
    ctx->direct_sent = ctx->generation;
    return MOE_OK;
}

moe_status moe_dispatch_allgather(moe_ctx* ctx, const uint16_t* x, const int32_t* topk_ids, const float* topk_w,
                                  void* workspace, size_t workspace_bytes, void* gathered, float* gathered_scales,
                                  void* recv_buf, float* recv_scales, moe_handle* handle, void* stream) {
    const CallScope scope("moe_dispatch_allgather");
    if (!ctx || !handle) return fail(MOE_ERR_INVALID_ARG, "ctx or handle is NULL");
    const moe::Dims d = ctx->d;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
        return fail(MOE_ERR_INVALID_ARG, "workspace is NULL or not 256-byte aligned");
    if (workspace_bytes < ctx->ws_bytes) return fail(MOE_ERR_WORKSPACE, "workspace_bytes < moe_workspace_bytes(ctx)");
    if (d.T > 0 && (!x || !topk_ids || !topk_w || !gathered || !recv_buf))
        return fail(MOE_ERR_INVALID_ARG, "x, topk_ids, topk_w, gathered or recv_buf is NULL");
    if (d.fp8 ? (d.T > 0 && (!gathered_scales || !recv_scales)) : (gathered_scales || recv_scales))
        return bad_scales();
    if (moe_status a = check_alignment({x, gathered, recv_buf}, {topk_ids, topk_w, gathered_scales, recv_scales});
        a != MOE_OK)
        return a;
    // the gathered rows (P * T of them, indexed in 32 bits) in one grid dimension of fewer than 2^32 work-items
    if ((long long)d.P * d.T * (d.H / 8 + 512) >= (1LL << 32))
        return fail(MOE_ERR_UNSUPPORTED, "P * T gathered rows exceed one grid dimension");

    const moe::Workspace ws = carve(ctx, workspace);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (d.T > 0) {
        moe_status s = validate_ids(ctx, d, topk_ids, ws, st);
        if (s != MOE_OK) return s;
        s = launch(ctx, "allgather", st, [&] { return moe::launch_allgather(d, x, gathered, gathered_scales, st); });
        const bool fused = moe::pack_counts(d);
        if (s == MOE_OK && !fused) s = count_and_scan(ctx, d, topk_ids, ws, st);
        if (s == MOE_OK)
            s = launch(ctx, fused ? "count_handles" : "handles", st,
                       [&] { return moe::launch_pack_handles(d, topk_ids, topk_w, ws, st); });
        if (s == MOE_OK)
            s = launch(ctx, "select", st, [&] {
                return moe::launch_select(d, ws, topk_ids, gathered, gathered_scales, recv_buf, recv_scales, st);
            });
        if (s != MOE_OK) return s;
    }
    ctx->workspace = workspace;
    fill_handle(ctx, ws, handle, false);
    ctx->received = ctx->generation;
    return MOE_OK;
}

moe_status moe_expert_stub(moe_ctx* ctx, const moe_handle* handle, const void* recv_buf, const float* recv_scales,
                           uint16_t* expert_out, void* stream) {
    const CallScope scope("moe_expert_stub");
    if (!ctx) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
    moe_status s = check_received(ctx, handle, "moe_expert_stub");
    if (s != MOE_OK) return s;
    const moe::Dims d = ctx->d;
    if (d.T == 0) return MOE_OK;
    if (!recv_buf || !expert_out) return fail(MOE_ERR_INVALID_ARG, "recv_buf or expert_out is NULL");
    if (d.fp8 ? !recv_scales : recv_scales != nullptr) return bad_scales();
    if (moe_status a = check_alignment({recv_buf, expert_out}, {recv_scales}); a != MOE_OK) return a;
    const moe::Workspace ws = from_handle(handle);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool affine = affine_layout(ctx, handle);
    return launch(ctx, "stub", st,
                  [&] { return moe::launch_stub(d, ws, recv_buf, recv_scales, expert_out, affine, st); });
}

moe_status moe_combine_send(moe_ctx* ctx, const moe_handle* handle, const uint16_t* expert_out,
                            uint16_t* comb_buf, void* stream) {
    const CallScope scope("moe_combine_send");
    if (!ctx) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
    moe_status s = check_received(ctx, handle, "moe_combine_send");
    if (s != MOE_OK) return s;
    const moe::Dims d = ctx->d;
    if (d.T > 0) {
        if (!expert_out || !comb_buf) return fail(MOE_ERR_INVALID_ARG, "expert_out or comb_buf is NULL");
        if (moe_status a = check_alignment({expert_out, comb_buf}, {}); a != MOE_OK) return a;
        const moe::Workspace ws = from_handle(handle);
        hipStream_t st = static_cast<hipStream_t>(stream);
        s = launch(ctx, "reverse_exchange", st,
                   [&] {
                       return moe::launch_reverse_exchange(d, ws, expert_out, comb_buf, affine_layout(ctx, handle), st);
                   });
        if (s != MOE_OK) return s;
    }
    ctx->combine_sent = ctx->generation;
    return MOE_OK;
}

moe_status moe_combine_recv(moe_ctx* ctx, const moe_handle* handle, const uint16_t* comb_buf, const float* topk_w,
                            uint16_t* y, void* stream) {
    const CallScope scope("moe_combine_recv");
    if (!ctx) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
    moe_status s = check_received(ctx, handle, "moe_combine_recv");
    if (s != MOE_OK) return s;
    if (ctx->combine_sent != handle->generation) {
        g_last_error = "moe_combine_recv: moe_combine_send has not been issued for this handle";
        return MOE_ERR_INVALID_ARG;
    }
    const moe::Dims d = ctx->d;
    if (d.T == 0) return MOE_OK;
    if (!comb_buf || !topk_w || !y) return fail(MOE_ERR_INVALID_ARG, "comb_buf, topk_w or y is NULL");
    if (moe_status a = check_alignment({comb_buf, y}, {topk_w}); a != MOE_OK) return a;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool affine = affine_layout(ctx, handle);
    return launch(ctx, "reduce", st,
                  [&] { return moe::launch_reduce(d, comb_buf, nullptr, topk_w, y, false, affine, st); });
}

moe_status moe_combine(moe_ctx* ctx, const moe_handle* handle, const uint16_t* expert_out, const float* topk_w,
                       uint16_t* comb_buf, uint16_t* y, void* stream) {
    const CallScope scope("moe_combine");
    if (!ctx) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
    moe_status s = check_received(ctx, handle, "moe_combine");
    if (s != MOE_OK) return s;
    if (ctx->d.T > 0 && (!expert_out || !topk_w || !comb_buf || !y))
        return fail(MOE_ERR_INVALID_ARG, "expert_out, topk_w, comb_buf or y is NULL");
    if (moe_status a = check_alignment({expert_out, comb_buf, y}, {topk_w}); a != MOE_OK) return a;
    s = moe_combine_send(ctx, handle, expert_out, comb_buf, stream);
    if (s != MOE_OK) return s;
    return moe_combine_recv(ctx, handle, comb_buf, topk_w, y, stream);
}

moe_status moe_combine_direct(moe_ctx* ctx, const moe_handle* handle, const uint16_t* expert_out,
                              const float* topk_w, uint16_t* y, void* stream) {
    const CallScope scope("moe_combine_direct");
    if (!ctx) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
    moe_status s = check_received(ctx, handle, "moe_combine_direct");
    if (s != MOE_OK) return s;
    const moe::Dims d = ctx->d;
    if (d.T == 0) return MOE_OK;
    if (!expert_out || !topk_w || !y) return fail(MOE_ERR_INVALID_ARG, "expert_out, topk_w or y is NULL");
    if (moe_status a = check_alignment({expert_out, y}, {topk_w}); a != MOE_OK) return a;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return launch(ctx, "reduce_direct", st, [&] {
        return moe::launch_reduce(d, expert_out, handle->recv_pos, topk_w, y, true, affine_layout(ctx, handle), st);
    });
}

moe_status moe_event_create(void** event) {
    const CallScope scope("moe_event_create");
    if (!event) return fail(MOE_ERR_INVALID_ARG, "event is NULL");
    hipEvent_t ev = nullptr;
    if (hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventDisableSystemFence); e != hipSuccess)
        return hip_fail(e, "hipEventCreateWithFlags");
    *event = ev;
    return MOE_OK;
}

moe_status moe_event_destroy(void* event) {
    const CallScope scope("moe_event_destroy");
    if (!event) return MOE_OK;
    hipError_t e = hipEventDestroy(static_cast<hipEvent_t>(event));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "hipEventDestroy");
}

}  // extern "C"

namespace {

moe_status refuse_capture(hipStream_t st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipError_t e = hipStreamIsCapturing(st, &cs); e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone) return fail(MOE_ERR_UNSUPPORTED, "the stream is capturing a graph");
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_event_record(void* event, void* stream) {
    const CallScope scope("moe_event_record");
    if (!event) return fail(MOE_ERR_INVALID_ARG, "event is NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (moe_status s = refuse_capture(st); s != MOE_OK) return s;
    hipError_t e = hipEventRecord(static_cast<hipEvent_t>(event), st);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "hipEventRecord");
}

moe_status moe_stream_wait_event(void* stream, void* event) {
    const CallScope scope("moe_stream_wait_event");
    if (!event) return fail(MOE_ERR_INVALID_ARG, "event is NULL");
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (moe_status s = refuse_capture(st); s != MOE_OK) return s;
    hipError_t e = hipStreamWaitEvent(st, static_cast<hipEvent_t>(event), 0);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "hipStreamWaitEvent");
}

moe_status moe_probe_copy(const void* src, void* dst, size_t bytes, int32_t policy, void* stream) {
    const CallScope scope("moe_probe_copy");
    if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "src or dst is NULL");
    if (policy < 0 || policy > 2) return fail(MOE_ERR_INVALID_ARG, "policy must be 0, 1 or 2");
    if (bytes % 16 != 0) return fail(MOE_ERR_INVALID_ARG, "bytes is not a multiple of 16");
    if ((bytes / 16) / 256 >= (1ULL << 31)) return fail(MOE_ERR_UNSUPPORTED, "bytes beyond one grid dimension");
    if (moe_status a = check_alignment({src, dst}, {}); a != MOE_OK) return a;
    hipError_t e = moe::launch_probe_copy(src, dst, (long long)(bytes / 16), policy, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "probe_copy");
}

moe_status moe_probe_gather(const void* src, int32_t src_rows, void* dst, const int32_t* perm, int32_t rows,
                            int32_t row_bytes, int32_t policy, void* stream) {
    const CallScope scope("moe_probe_gather");
    if (!src || !dst || !perm) return fail(MOE_ERR_INVALID_ARG, "src, dst or perm is NULL");
    if (policy < 0 || policy > 2) return fail(MOE_ERR_INVALID_ARG, "policy must be 0, 1 or 2");
    if (rows < 0 || src_rows <= 0) return fail(MOE_ERR_INVALID_ARG, "rows is negative or src_rows is not positive");
    if (row_bytes <= 0 || row_bytes % 16 != 0) return fail(MOE_ERR_INVALID_ARG, "row_bytes is not a positive multiple of 16");
    // every row's slices in one grid dimension of fewer than 2^32 work-items (a row takes fewer than 512 more)
    if ((long long)rows * (row_bytes / 16 + 512) >= (1LL << 32))
        return fail(MOE_ERR_UNSUPPORTED, "rows x row_bytes beyond one grid dimension");
    if (moe_status a = check_alignment({src, dst}, {perm}); a != MOE_OK) return a;
    hipError_t e = moe::launch_probe_gather(src, src_rows, dst, perm, rows, row_bytes / 16, policy,
                                            static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "probe_gather");
}

moe_status moe_probe_read(const void* src, size_t bytes, uint32_t* sink, int32_t nontemporal, void* stream) {
    const CallScope scope("moe_probe_read");
    if (!src || !sink) return fail(MOE_ERR_INVALID_ARG, "src or sink is NULL");
    if (bytes % 16 != 0) return fail(MOE_ERR_INVALID_ARG, "bytes is not a multiple of 16");
    if ((bytes / 16) / 256 >= (1ULL << 31)) return fail(MOE_ERR_UNSUPPORTED, "bytes beyond one grid dimension");
    if (moe_status a = check_alignment({src}, {sink}); a != MOE_OK) return a;
    hipError_t e = moe::launch_probe_read(src, sink, (long long)(bytes / 16), nontemporal != 0,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : hip_fail(e, "probe_read");
}

moe_status moe_timing_begin(moe_ctx* ctx) {
    g_last_error.clear();
    if (!ctx) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
    ctx->timing = true;
    return MOE_OK;
}

moe_status moe_timing_end(moe_ctx* ctx, moe_kernel_time* out, int32_t max, int32_t* count) {
    g_last_error.clear();
    if (!ctx || !count || (max > 0 && !out)) return fail(MOE_ERR_INVALID_ARG, "ctx, count or out is NULL");
    ctx->timing = false;
    std::vector<moe_kernel_time> agg;
    moe_status status = MOE_OK;
    for (auto& r : ctx->records) {
        float ms = 0.0f;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess && status == MOE_OK) status = hip_fail(e, "hipEventElapsedTime");
        size_t i = 0;
        while (i < agg.size() && std::strcmp(agg[i].kernel, r.name) != 0) ++i;
        if (i == agg.size()) agg.push_back({r.name, 0, 0.0f});
        agg[i].launches += 1;
        agg[i].total_ms += ms;
        ctx->free_events.push_back(r.start);
        ctx->free_events.push_back(r.stop);
    }
    ctx->records.clear();
    *count = (int32_t)agg.size();
    for (int32_t i = 0; i < (int32_t)agg.size() && i < max; ++i) out[i] = agg[i];
    return status;
}

}  // extern "C"
