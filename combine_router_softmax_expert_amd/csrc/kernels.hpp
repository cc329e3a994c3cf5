// kernels.hpp -- host launchers of the gfx950 kernels (internal to libmoe_ep.so).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

namespace moe {

// Events the next kernel launch of this thread records at its start and end
// (set by the library while it times kernels; null otherwise).  The events
// travel in the dispatch itself, so they bracket the kernel alone, not the
// gaps between launches.
struct LaunchTiming {
    hipEvent_t start = nullptr, stop = nullptr;
};
inline thread_local LaunchTiming launch_timing;

// Launches `kernel` on `st` and returns the launch's own status (not the
// thread's last-error slot, which an earlier failing runtime call may hold).
// The arguments are converted to the kernel's parameter types as
// hipExtLaunchKernelGGL converts them.
template <typename... Args, typename F = void (*)(Args...)>
inline hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, size_t lds_bytes, hipStream_t st, Args... args) {
    auto given = std::tuple<Args...>{args...};
    auto formal = validateArgsCountType(kernel, given);
    void* argv[sizeof...(Args) > 0 ? sizeof...(Args) : 1];
    pArgs<0>(formal, argv);
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds_bytes, st,
                              launch_timing.start, launch_timing.stop, 0);
}

// The 16-byte handle record that travels with every dispatched row (the ABI's moe_meta).
struct HandleRecord {
    int32_t src_rank;
    int32_t src_token;
    int16_t slot;
    int16_t local_expert;
    float weight;
};
static_assert(sizeof(HandleRecord) == 16, "handle record is 16 bytes");

// Cache policy of the payload kernels: kAuto streams (nontemporal accesses, gather
// form of the exchanges) when a kernel moves at least kStreamingBytes.
enum class CachePolicy { kAuto = 0, kTemporal = 1, kStreaming = 2 };
constexpr long long kStreamingBytes = 128LL << 20;

// How dispatch ranks the assignments: kAuto lets the pack kernel count by itself
// when the problem is small enough (pack_counts), kSeparate always launches the
// count (and scan) kernels first, kFused counts in the pack kernel whenever its
// id loads fit (kMaxIdsPerThread per thread).
enum class CountPath { kAuto = 0, kSeparate = 1, kFused = 2 };

// Workgroup layout of the kernels after the pack: kAuto takes the token-affine
// layout for cache-resident problems (token_affine), kRows always walks rows,
// kTokens always takes the token-affine layout.
enum class Layout { kAuto = 0, kRows = 1, kTokens = 2 };

struct Dims {
    int P, Tp, T, E, Ep, k, H;
    CachePolicy policy;
    CountPath count_path;
    Layout layout;
    bool fp8;
    long long Na;          // T * k
    int row_units;         // 16-byte units per dispatched row (2H/16 or H/16)
    int out_units;         // 16-byte units per bf16 output row (2H/16)
    int scales;            // fp32 scales per dispatched row (H/128 or 0)
};

struct Workspace {         // device arrays carved from the caller's workspace
    int32_t* n;            // [P][E]
    int32_t* N;            // [E]
    int32_t* expert_off;   // [E+1]
    int32_t* rank_recv_off;// [P+1]
    int32_t* send_off;     // [P][E]
    int32_t* recv_off;     // [P][E]
    int32_t* C;            // [P][P]
    int32_t* bucket_rank;  // [T*k] rank of the assignment inside its (source, expert) bucket
    int32_t* send_pos;     // [T*k]
    int32_t* recv_pos;     // [T*k]
    int32_t* send_to_recv; // [N_a] receive row of each send row
    int32_t* recv_to_send; // [N_a] send row of each receive row
    void* send_meta;       // [N_a] 16-byte records
    void* recv_meta;       // [N_a]
    int32_t* bad_ids;      // [1] debug mode: number of invalid assignments found
};

// Byte offsets of the count arrays from the start of the workspace, in the
// order the workspace holds them, each on 256 bytes.  The host carves the
// workspace with it, and the counting pack's per-rank workgroups find the seven
// arrays from the workspace's start with it, so the pack takes one pointer for
// them (kernel arguments past the first 14 dwords are not preloaded).
struct CountLayout {
    size_t n, N, expert_off, rank_recv_off, send_off, recv_off, C, end;
};
__host__ __device__ constexpr size_t ws_align(size_t x) { return (x + 255) / 256 * 256; }
__host__ __device__ inline CountLayout count_layout(size_t P, size_t E) {
    CountLayout c{};
    c.n = 0;
    c.N = ws_align(c.n + 4 * P * E);
    c.expert_off = ws_align(c.N + 4 * E);
    c.rank_recv_off = ws_align(c.expert_off + 4 * (E + 1));
    c.send_off = ws_align(c.rank_recv_off + 4 * (P + 1));
    c.recv_off = ws_align(c.send_off + 4 * P * E);
    c.C = ws_align(c.recv_off + 4 * E * P);
    c.end = ws_align(c.C + 4 * P * P);
    return c;
}

// Debug check: the number of ids outside [0, E) or repeated within a token.
hipError_t launch_validate_ids(const Dims& d, const int32_t* ids, int32_t* bad_out, hipStream_t st);
hipError_t launch_route_topk(const Dims& d, const float* logits, int32_t* ids, float* w, hipStream_t st);
hipError_t launch_count(const Dims& d, const int32_t* ids, const Workspace& ws, hipStream_t st);
hipError_t launch_scan(const Dims& d, const Workspace& ws, hipStream_t st);
// direct: rows, scales and records go straight to their receive rows (dst = the receive buffer)
hipError_t launch_pack(const Dims& d, const uint16_t* x, const int32_t* ids, const float* w,
                       const Workspace& ws, void* dst, float* dst_scales, bool direct, hipStream_t st);
// All-gather dispatcher: every rank's copy of every token's dispatched row
// (gathered = [P*T][row], scales [P*T][H/128]); the receive-side positions and
// records without rows; each rank's pick of its receive rows from its copy.
hipError_t launch_allgather(const Dims& d, const uint16_t* x, void* gathered, float* gathered_scales, hipStream_t st);
hipError_t launch_pack_handles(const Dims& d, const int32_t* ids, const float* w, const Workspace& ws,
                               hipStream_t st);
hipError_t launch_select(const Dims& d, const Workspace& ws, const int32_t* ids, const void* gathered,
                         const float* gathered_scales, void* recv, float* recv_scales, hipStream_t st);
// affine: the token-affine layout (token_affine(d) must hold), else row grids.
hipError_t launch_exchange(const Dims& d, const Workspace& ws, const void* send, const float* send_scales,
                           void* recv, float* recv_scales, bool affine, hipStream_t st);
hipError_t launch_stub(const Dims& d, const Workspace& ws, const void* recv, const float* recv_scales,
                       uint16_t* out, bool affine, hipStream_t st);
hipError_t launch_reverse_exchange(const Dims& d, const Workspace& ws, const uint16_t* expert_out,
                                   uint16_t* comb, bool affine, hipStream_t st);
// direct: rows = the expert output, read through recv_pos; else rows = the combine buffer
hipError_t launch_reduce(const Dims& d, const uint16_t* rows, const int32_t* recv_pos, const float* w, uint16_t* y,
                         bool direct, bool affine, hipStream_t st);

// Measurement aids (probe.hip): a plain copy and a streaming read of `units`
// 16-byte units, one unit per lane; the read's sink holds 256 words.
// Copy policy: 0 temporal, 1 nontemporal, 2 temporal loads with write-through stores.
hipError_t launch_probe_copy(const void* src, void* dst, long long units, int policy, hipStream_t st);
hipError_t launch_probe_read(const void* src, uint32_t* sink, long long units, bool nontemporal, hipStream_t st);
// Row gather: dst row r (of `units` units) = src row perm[r] clamped into [0, src_rows), r < rows.
hipError_t launch_probe_gather(const void* src, int src_rows, void* dst, const int32_t* perm, int rows, int units,
                               int policy, hipStream_t st);

// The library's own dispatch workspace (static_workspace.hip), for moe_dispatch_noalloc.
constexpr size_t kStaticWorkspaceBytes = 8u << 20;
// Device address of the current device's copy (taken with hipGetSymbolAddress on
// first use on that device) and that device's ordinal.
hipError_t static_workspace(int* device, void** ptr);
// Marks a dispatch into the device's copy; returns its claim number (1, 2, ...).
uint64_t static_workspace_claim(int device);
// The claim number of the latest dispatch into the device's copy.
uint64_t static_workspace_latest_claim(int device);

inline bool streaming(const Dims& d, long long bytes) {
    return d.policy == CachePolicy::kStreaming || (d.policy == CachePolicy::kAuto && bytes >= kStreamingBytes);
}

// Grid of a row kernel: rows x slices workgroups in one dimension, the slices of
// a row adjacent, so that workgroups issued together cover consecutive bytes
// (measured on gfx950 with 14 KiB rows: a gathering copy 5.6 -> 6.0 TB/s and
// the weighted reduction 5.7 -> 5.9 TB/s against a (rows, slices) grid).  The
// shape limits keep rows x slices x block below 2^32 work-items.
inline dim3 row_grid(long long rows, int slices) { return dim3((unsigned)(rows * slices)); }

// Kernel arguments.  The library is built with kernel-argument preloading: a
// gfx950 wave starts with the first 14 dwords of its kernel arguments already
// in SGPRs (16 user SGPRs less the kernarg segment pointer), and the rest, the
// hidden ones (workgroup size, grid size) included, come from a scalar load.
// So the path's kernels list first the arguments their first loads depend on,
// take their workgroup size as an argument (bs, equal to blockDim.x) where the
// hidden one would fall past the preloaded dwords (kernels with at most 10
// dwords of arguments, such as the router and the reverse exchange, still read
// it), and take no aggregate arguments (an aggregate ends the preloaded ones).
// Measured on gfx950 at 128 tokens x top-8 x 7168: whole step 29.57 -> 28.52
// us, dispatch + combine 20.48 -> 19.89 us.

// Threads per block of the streaming (nontemporal) exchange, reverse exchange
// and expert stub: one wave, so a row takes L / 64 workgroups.  Measured on
// gfx950 at 8192 tokens x top-8 x 7168 (65,536 rows) against the row-dividing
// 448-thread workgroups: exchange of 7 KiB e4m3 rows 159.6 -> 156.1 us, reverse
// exchange of 14 KiB rows 308.0 -> 302.9 us, e4m3 stub 228.8 -> 220.1 us; at
// 32,768 rows of 8 KiB each moved by less than 1.5%.  The pack (k stores per
// lane) ran 8% slower with one wave and the reduction (k loads per lane) no
// faster, so they keep their sizes.
constexpr int kStreamBlock = 64;

// Threads per block for a row of `n` per-thread work items: the whole row when it
// fits in 512 threads, else a divisor of n from 512 down to 256, else 256.
inline int pick_block(long long n) {
    if (n <= 512) return (int)((n + 63) / 64 * 64);
    for (int b = 512; b >= 256; b -= 64)
        if (n % b == 0) return b;
    return 256;
}

// True when one workgroup does count and scan together (launch_scan is then not needed).
bool count_is_single(const Dims& d);

// True when launch_pack counts and ranks the assignments itself and writes the
// counts and offsets too (launch_count and launch_scan are then not needed).
bool pack_counts(const Dims& d);

// Token-affine layout.  Workgroup w runs on XCD w mod 8 (workgroups are handed
// out round-robin over the 8 XCDs), and the lines a kernel writes stay in that
// XCD's L2 for the next kernel: rereading 14.7 MB there took half the time of
// rereading it from another XCD on gfx950.  The pack's workgroup for token group
// g (its tokens_per_block tokens) and slice s runs on XCD (g * slices + s) mod 8;
// in this layout every later kernel serves token group g, slice s on that XCD
// again, so each reads what the previous one wrote through its own L2.  It needs
// bf16 rows (dispatch and output rows then have the same slices) and pays when
// an output buffer fits well inside the L2s; token_affine says whether a ctx
// allows it (not under Layout::kRows).  The library takes it after a direct
// dispatch (measured at 128 tokens x top-8 x 7168: step 24.8 -> 23.9 us); after
// the base dispatch, whose exchange and reverse exchange then have to load
// their positions before their rows, it measured no faster (33.0 against 33.3
// us) and is used only under Layout::kTokens.
constexpr long long kAffineBytes = 24LL << 20;
bool token_affine(const Dims& d);

// The grid of a token-affine kernel: `rounds` rounds of 2^m_log2 workgroups (a
// power of two at least groups * slices and 8); within a round, workgroup
// g * slices + s serves token group g, slice s, the rest exit.  Round r is slot
// r >> tpb_log2 (0 for per-token kernels) of token g * 2^tpb_log2 + (r & mask).
struct TokenGrid {
    int groups, slices, tpb_log2, m_log2, rounds;
    dim3 grid() const { return dim3((unsigned)rounds << m_log2); }
};
TokenGrid token_grid(const Dims& d, int slices, bool per_assignment);

}  // namespace moe
