// exchange.hip -- the all-to-all-v exchange of dispatch and its reverse for the
// combine, for P logical ranks whose send and receive buffers share one HBM.
//
// Forward ("[Infra-10] All-to-All Optimization" 1: all-to-all as a distributed
// transpose, rank j receives piece j of every rank; "Expert Parallel: MoE
// Token ..." worked example: each rank's receive region is grouped by local
// expert): send row p lands on receive row send_to_recv[p] together with its
// FP8 scales and its handle record.  Reverse ("Combine 不是简单把结果发回来":
// outputs go back to their token by the handle, never in arrival order):
// receive row q goes to combine row (s*T/P + i)*k + j of the (s, i, j) its
// record names.
//
// Rows are moved whole with 16-byte loads and stores, one unit per thread (a
// second load in flight before the stores runs 4x slower on gfx950 when the
// buffers sit in the last-level cache); a workgroup slice covers a row or part
// of one, so the permutation costs one index (or record) load per row.
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

struct Rec { int32_t src_rank, src_token; int16_t slot, local_expert; float weight; };

__global__ __launch_bounds__(512) void exchange_kernel(const uint4* __restrict__ send, uint4* __restrict__ recv,
                                                       const int32_t* __restrict__ send_to_recv,
                                                       const float* __restrict__ send_scales,
                                                       float* __restrict__ recv_scales,
                                                       const uint4* __restrict__ send_meta,
                                                       uint4* __restrict__ recv_meta, int L, int nb, int slices) {
    const int p = blockIdx.x / slices;
    const int slice = blockIdx.x - p * slices;
    const int q = send_to_recv[p];
    const int u = slice * blockDim.x + threadIdx.x;
    if (u < L) recv[(size_t)q * L + u] = send[(size_t)p * L + u];
    if (slice == 0) {
        for (int x = threadIdx.x; x < nb; x += blockDim.x) recv_scales[(size_t)q * nb + x] = send_scales[(size_t)p * nb + x];
        if (threadIdx.x == blockDim.x - 1) recv_meta[q] = send_meta[p];
    }
}

__global__ __launch_bounds__(512) void reverse_exchange_kernel(const uint4* __restrict__ expert_out,
                                                               uint4* __restrict__ comb,
                                                               const Rec* __restrict__ recv_meta, int Tp, int k,
                                                               int L, int slices) {
    const int q = blockIdx.x / slices;
    const int slice = blockIdx.x - q * slices;
    const Rec m = recv_meta[q];
    const long long c = ((long long)m.src_rank * Tp + m.src_token) * k + m.slot;
    const int u = slice * blockDim.x + threadIdx.x;
    if (u < L) comb[(size_t)c * L + u] = expert_out[(size_t)q * L + u];
}

}  // namespace

hipError_t launch_exchange(const Dims& d, const Workspace& ws, const void* send, const float* send_scales,
                           void* recv, float* recv_scales, hipStream_t st) {
    if (d.Na == 0) return hipSuccess;
    const int L = d.row_units;
    const int B = pick_block(L);
    const int slices = (L + B - 1) / B;
    hipLaunchKernelGGL(exchange_kernel, dim3((unsigned)(d.Na * slices)), dim3(B), 0, st,
                       reinterpret_cast<const uint4*>(send), reinterpret_cast<uint4*>(recv), ws.send_to_recv,
                       send_scales, recv_scales, reinterpret_cast<const uint4*>(ws.send_meta),
                       reinterpret_cast<uint4*>(ws.recv_meta), L, d.scales, slices);
    return hipGetLastError();
}

hipError_t launch_reverse_exchange(const Dims& d, const Workspace& ws, const uint16_t* expert_out, uint16_t* comb,
                                   hipStream_t st) {
    if (d.Na == 0) return hipSuccess;
    const int L = d.out_units;
    const int B = pick_block(L);
    const int slices = (L + B - 1) / B;
    hipLaunchKernelGGL(reverse_exchange_kernel, dim3((unsigned)(d.Na * slices)), dim3(B), 0, st,
                       reinterpret_cast<const uint4*>(expert_out), reinterpret_cast<uint4*>(comb),
                       reinterpret_cast<const Rec*>(ws.recv_meta), d.Tp, d.k, L, slices);
    return hipGetLastError();
}

}  // namespace moe
