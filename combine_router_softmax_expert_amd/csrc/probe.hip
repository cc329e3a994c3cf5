// probe.hip -- measurement aids, not part of the path: the rate this GPU reaches
// for the access patterns the path's row kernels use, so that each kernel's
// achieved bandwidth can be read against a ceiling measured on the same
// machine ("[Infra-10] All-to-All Optimization" 11.2: profile against what the
// hardware can actually deliver, not against the data sheet alone).
//
//  - copy: one 16-byte unit per lane, consecutive lanes on consecutive units, a
//    1-D grid of 256-thread workgroups, with temporal, nontemporal or
//    write-through stores: the row kernels' pattern with the permutation taken
//    out;
//  - gather: destination row r takes source row perm[r], one unit per lane with
//    the slices of a row adjacent, as the streaming exchange moves rows: a
//    chain of such copies, each reading what the one before wrote through a
//    permutation, has the hand-over of the path's dependent kernels;
//  - read: the same loads and no stores (each lane folds its unit into a
//    value that is stored only if it equals a constant no input reaches, so the
//    loads stay live), the ceiling for kernels that mostly read.
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;

// POLICY 0: temporal loads and write-back stores; 1: nontemporal loads and
// stores; 2: temporal loads and write-through stores (device scope, as the
// row kernels' st16_row), each workgroup's 4 KiB slice taken as one row.
template <int POLICY>
__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const uint4* __restrict__ src,
                                                                   uint4* __restrict__ dst, long long units) {
    const long long u = (long long)blockIdx.x * kProbeThreads + threadIdx.x;
    if (u >= units) return;
    const uint4 v = ld16<POLICY == 1>(&src[u]);
    if constexpr (POLICY == 2) st16_row<false>(dst, (int)blockIdx.x, kProbeThreads, (int)threadIdx.x, v);
    else st16<POLICY == 1>(&dst[u], v);
}

// POLICY as probe_copy_kernel.  perm[r] is clamped into [0, src_rows), so no
// entry can address outside the source.
template <int POLICY>
__global__ __launch_bounds__(512) void probe_gather_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                           const int32_t* __restrict__ perm, int src_rows, int units,
                                                           int slices) {
    const auto [r, slice] = row_slice(slices);
    const int u = slice * blockDim.x + threadIdx.x;
    const int p = min(max(perm[r], 0), src_rows - 1);
    if (u >= units) return;
    const uint4 v = ld16<POLICY == 1>(&src[(size_t)p * units + u]);
    if constexpr (POLICY == 0) st16<false>(&dst[(size_t)r * units + u], v);
    else st16_row<POLICY == 1>(dst, r, units, u, v);   // nontemporal, or write-through
}

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* __restrict__ src,
                                                                   uint32_t* __restrict__ sink, long long units,
                                                                   uint32_t never) {
    const long long u = (long long)blockIdx.x * kProbeThreads + threadIdx.x;
    if (u >= units) return;
    const uint4 v = ld16<NT>(&src[u]);
    const uint32_t f = v.x ^ (v.y * 3u) ^ (v.z * 5u) ^ (v.w * 7u);
    if (f == never) sink[threadIdx.x] = f;   // per-lane address: a vector store, in bounds of a 256-word sink
}

}  // namespace

hipError_t launch_probe_copy(const void* src, void* dst, long long units, int policy, hipStream_t st) {
    if (units == 0) return hipSuccess;
    const dim3 grid((unsigned)((units + kProbeThreads - 1) / kProbeThreads));
    auto kernel = policy == 1 ? probe_copy_kernel<1> : policy == 2 ? probe_copy_kernel<2> : probe_copy_kernel<0>;
    return launch_kernel(kernel, grid, dim3(kProbeThreads), 0, st, static_cast<const uint4*>(src),
                         static_cast<uint4*>(dst), units);
}

hipError_t launch_probe_gather(const void* src, int src_rows, void* dst, const int32_t* perm, int rows, int units,
                              int policy, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    // nontemporal gathers of streaming size run one-wave workgroups, as the
    // library's streaming row kernels do; the rest the row-dividing size
    const bool stream_shape = policy == 1 && (long long)rows * units * 16 >= kStreamingBytes;
    const int B = stream_shape ? kStreamBlock : pick_block(units);
    const int slices = (units + B - 1) / B;
    auto kernel = policy == 1 ? probe_gather_kernel<1> : policy == 2 ? probe_gather_kernel<2> : probe_gather_kernel<0>;
    return launch_kernel(kernel, row_grid(rows, slices), dim3(B), 0, st, static_cast<const uint4*>(src),
                         static_cast<uint4*>(dst), perm, src_rows, units, slices);
}

hipError_t launch_probe_read(const void* src, uint32_t* sink, long long units, bool nontemporal, hipStream_t st) {
    if (units == 0) return hipSuccess;
    const dim3 grid((unsigned)((units + kProbeThreads - 1) / kProbeThreads));
    auto kernel = nontemporal ? probe_read_kernel<true> : probe_read_kernel<false>;
    // a value the fold never gives for the probe's inputs (the caller fills the source with zeros,
    // whose fold is 0)
    return launch_kernel(kernel, grid, dim3(kProbeThreads), 0, st, static_cast<const uint4*>(src), sink, units,
                         0xA5A5A5A5u);
}

}  // namespace moe
