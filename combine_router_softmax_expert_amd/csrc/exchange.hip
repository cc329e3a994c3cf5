// exchange.hip -- the all-to-all-v exchange of dispatch and its reverse for the
// combine, for P logical ranks whose send and receive buffers share one HBM.
//
// Forward ("[Infra-10] All-to-All Optimization" 1: all-to-all as a distributed
// transpose, rank j receives piece j of every rank; "Expert Parallel: MoE
// Token ..." worked example: each rank's receive region is grouped by local
// expert): send row p lands on receive row q = send_to_recv[p] together with
// its FP8 scales and its handle record.  Reverse ("Combine 不是简单把结果发回来":
// outputs go back to their token by the handle, never in arrival order):
// receive row q goes to combine row (s*T/P + i)*k + j of the (s, i, j) its
// record names, which is the row whose recv_pos is q.
//
// Rows move whole with 16-byte loads and stores, one unit per thread (two or
// four units, or two rows, per thread measured no faster on gfx950); a
// workgroup slice covers a row or part of one, so the permutation costs one
// index (or record) load per row.  Two forms:
//  - temporal (buffers that stay in cache): walk the source rows and scatter;
//  - streaming (large buffers): walk the destination rows in order, gather
//    from the source, nontemporal loads and stores (~18% faster there).
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

template <bool GATHER>
__global__ __launch_bounds__(512) void exchange_kernel(const int32_t* __restrict__ map, const uint4* __restrict__ send,
                                                       uint4* __restrict__ recv, int L, int slices, int bs, int nb,
                                                       const uint4* __restrict__ send_meta,
                                                       uint4* __restrict__ recv_meta,
                                                       const float* __restrict__ send_scales,
                                                       float* __restrict__ recv_scales) {
    const auto [b, slice] = row_slice(slices);
    const int u = slice * bs + threadIdx.x;
    const bool copies_scale = slice == 0 && (int)threadIdx.x < nb;
    const bool copies_record = slice == 0 && (int)threadIdx.x == bs - 1;
    // The map entry is uniform, so it loads through the scalar cache (the
    // scatter form's row load does not depend on it).  The row's first scales
    // and its record load together with the row, before any store: vmcnt
    // counts loads and stores in order, so a load issued after the row's store
    // would first wait for that store to complete.
    const int m = map[b];
    const int p = GATHER ? m : b;               // gather: the source row comes from the map
    const int q = GATHER ? b : m;               // scatter: the destination row does
    uint4 v, rec;
    float sc;
    if (u < L) v = ld16<GATHER>(&send[(size_t)p * L + u]);
    if (copies_scale) sc = send_scales[(size_t)p * nb + threadIdx.x];
    if (copies_record) rec = send_meta[p];
    if (u < L) st16_row<GATHER>(recv, q, L, u, v);
    // the scatter form writes the row's scales and record through as well, so that
    // they, like the row, leave no dirty lines for the write-back at the kernel
    // boundary (128 tokens x top-8 x 7168 on gfx950: exchange 4.73 -> 4.48 us,
    // dispatch + combine 19.91 -> 19.68 us; write-through stores of the pack's
    // positions, maps and records instead cost it 0.07-0.17 us)
    if (copies_scale) {
        if (GATHER) recv_scales[(size_t)q * nb + threadIdx.x] = sc;
        else st_through_row(recv_scales, q, nb, (int)threadIdx.x, sc);
        for (int x = threadIdx.x + bs; x < nb; x += bs)   // rows with more scales than threads
            recv_scales[(size_t)q * nb + x] = send_scales[(size_t)p * nb + x];
    }
    if (copies_record) {
        if (GATHER) recv_meta[q] = rec;
        else st_through_row(recv_meta, q, 1, 0, rec);
    }
}

__global__ __launch_bounds__(512) void reverse_exchange_scatter_kernel(const uint4* __restrict__ expert_out,
                                                                       uint4* __restrict__ comb,
                                                                       const HandleRecord* __restrict__ recv_meta, int Tp,
                                                                       int k, int L, int slices) {
    const auto [q, slice] = row_slice(slices);
    const int u = slice * blockDim.x + threadIdx.x;
    uint4 v;
    if (u < L) v = expert_out[(size_t)q * L + u];   // data first: its load overlaps the record's
    __builtin_amdgcn_sched_barrier(0);
    const HandleRecord m = recv_meta[q];
    const long long c = ((long long)m.src_rank * Tp + m.src_token) * k + m.slot;
    if (u < L) st16_row<false>(comb, (int)c, L, u, v);
}

__global__ __launch_bounds__(512) void reverse_exchange_gather_kernel(const uint4* __restrict__ expert_out,
                                                                      uint4* __restrict__ comb,
                                                                      const int32_t* __restrict__ recv_pos, int L,
                                                                      int slices) {
    const auto [c, slice] = row_slice(slices);  // combine row t*k + j
    const int q = recv_pos[c];
    const int u = slice * blockDim.x + threadIdx.x;
    if (u < L) st16_row<true>(comb, c, L, u, ld16<true>(&expert_out[(size_t)q * L + u]));
}

// Token-affine forms (cache-resident bf16 problems, token_affine): workgroup
// (t, j, slice) moves the rows of assignment t*k + j on the XCD whose L2 holds
// what the previous kernel wrote for that token and slice.  The positions come
// from the handle (every slice of the pack wrote them), then the row.  Their
// stores are write-back (plain), not st16_row's write-through: the next kernel
// reads each line on the same XCD, from that L2.
__global__ __launch_bounds__(512) void exchange_affine_kernel(const int32_t* __restrict__ send_pos,
                                                              const int32_t* __restrict__ recv_pos,
                                                              const uint4* __restrict__ send, int L, int k, int T,
                                                              int bs, int tg_groups, int tg_slices, int tg_tpb_log2,
                                                              int tg_m_log2, uint4* __restrict__ recv, int nb,
                                                              const uint4* __restrict__ send_meta,
                                                              uint4* __restrict__ recv_meta,
                                                              const float* __restrict__ send_scales,
                                                              float* __restrict__ recv_scales) {
    int t, j, slice;
    if (!token_item(tg_groups, tg_slices, tg_tpb_log2, tg_m_log2, T, t, j, slice)) return;
    const int a = t * k + j;
    const int p = send_pos[a], q = recv_pos[a];
    const int u = slice * bs + threadIdx.x;
    const bool copies_scale = slice == 0 && (int)threadIdx.x < nb;
    const bool copies_record = slice == 0 && (int)threadIdx.x == bs - 1;
    uint4 v, rec;
    float sc;
    if (u < L) v = send[(size_t)p * L + u];
    if (copies_scale) sc = send_scales[(size_t)p * nb + threadIdx.x];   // loads before stores, as in exchange_kernel
    if (copies_record) rec = send_meta[p];
    if (u < L) recv[(size_t)q * L + u] = v;
    if (copies_scale) {
        recv_scales[(size_t)q * nb + threadIdx.x] = sc;
        for (int x = threadIdx.x + bs; x < nb; x += bs)
            recv_scales[(size_t)q * nb + x] = send_scales[(size_t)p * nb + x];
    }
    if (copies_record) recv_meta[q] = rec;
}

__global__ __launch_bounds__(512) void reverse_exchange_affine_kernel(const int32_t* __restrict__ recv_pos,
                                                                      const uint4* __restrict__ expert_out,
                                                                      uint4* __restrict__ comb, int L, int k, int T,
                                                                      int bs, int tg_groups, int tg_slices,
                                                                      int tg_tpb_log2, int tg_m_log2) {
    int t, j, slice;
    if (!token_item(tg_groups, tg_slices, tg_tpb_log2, tg_m_log2, T, t, j, slice)) return;
    const int a = t * k + j;                    // combine row of the assignment
    const int q = recv_pos[a];
    const int u = slice * bs + threadIdx.x;
    if (u < L) comb[(size_t)a * L + u] = expert_out[(size_t)q * L + u];
}

// The all-gather dispatcher's local pick ("Expert Parallel: MoE Token ...",
// section "为什么不用 AllGather 收集所有 token": each rank picks its own
// assignments out of the gathered tokens): receive row q of rank r takes the
// token (s, i) its record names from rank r's own copy, row r*T + s*T/P + i,
// with its FP8 scales.
template <bool NT>
__global__ __launch_bounds__(512) void select_kernel(const uint4* __restrict__ gathered,
                                                     const float* __restrict__ gathered_scales,
                                                     uint4* __restrict__ recv, float* __restrict__ recv_scales,
                                                     const HandleRecord* __restrict__ recv_meta,
                                                     const int32_t* __restrict__ rank_recv_off, int P, int T, int Tp,
                                                     int L, int nb, int slices) {
    const auto [q, slice] = row_slice(slices);
    const int u = slice * blockDim.x + threadIdx.x;
    const int r = owner_rank(rank_recv_off, P, q);
    const HandleRecord m = recv_meta[q];
    const size_t src = (size_t)r * T + (size_t)m.src_rank * Tp + m.src_token;
    const bool copies_scale = slice == 0 && (int)threadIdx.x < nb;
    uint4 v;
    float sc;
    if (u < L) v = ld16<NT>(&gathered[src * L + u]);
    if (copies_scale) sc = gathered_scales[src * nb + threadIdx.x];   // loads before stores, as in exchange_kernel
    if (u < L) st16_row<NT>(recv, q, L, u, v);
    if (copies_scale) {
        recv_scales[(size_t)q * nb + threadIdx.x] = sc;
        for (int x = threadIdx.x + blockDim.x; x < nb; x += blockDim.x)
            recv_scales[(size_t)q * nb + x] = gathered_scales[src * nb + x];
    }
}

// Source-walking form of the same pick, for when every rank's copy is mostly
// needed (P <= 2k): workgroup (r, t) loads row t of rank r's copy at once, then
// stores it to the receive row of every slot of token t whose expert lives on
// rank r (ids and positions load alongside the row, so no load waits on another).
template <bool NT>
__global__ __launch_bounds__(512) void select_scatter_kernel(const uint4* __restrict__ gathered,
                                                             const float* __restrict__ gathered_scales,
                                                             uint4* __restrict__ recv, float* __restrict__ recv_scales,
                                                             const int32_t* __restrict__ ids,
                                                             const int32_t* __restrict__ recv_pos, int T, int Ep, int k,
                                                             int L, int nb, int slices) {
    const auto [g, slice] = row_slice(slices);   // row r*T + t of the gathered copies
    const int r = g / T, t = g - r * T;
    const int u = slice * blockDim.x + threadIdx.x;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (u < L) v = ld16<NT>(&gathered[(size_t)g * L + u]);
    for (int j = 0; j < k; ++j) {
        const int a = t * k + j;
        if (ids[a] / Ep != r) continue;        // uniform: the same slot in every lane
        const int q = recv_pos[a];
        if (u < L) st16_row<NT>(recv, q, L, u, v);
        if (slice == 0)
            for (int x = threadIdx.x; x < nb; x += blockDim.x)
                recv_scales[(size_t)q * nb + x] = gathered_scales[(size_t)g * nb + x];
    }
}

}  // namespace

hipError_t launch_select(const Dims& d, const Workspace& ws, const int32_t* ids, const void* gathered,
                         const float* gathered_scales, void* recv, float* recv_scales, hipStream_t st) {
    if (d.Na == 0) return hipSuccess;
    const int L = d.row_units;
    const int B = pick_block(L);
    const int slices = (L + B - 1) / B;
    const bool nt = streaming(d, 2LL * d.Na * (16LL * L + 4LL * d.scales));
    if (d.P <= 2 * d.k) {
        auto kernel = nt ? select_scatter_kernel<true> : select_scatter_kernel<false>;
        return launch_kernel(kernel, row_grid((long long)d.P * d.T, slices), dim3(B), 0, st,
                      reinterpret_cast<const uint4*>(gathered), gathered_scales, reinterpret_cast<uint4*>(recv),
                      recv_scales, ids, ws.recv_pos, d.T, d.Ep, d.k, L, d.scales, slices);
    }
    auto kernel = nt ? select_kernel<true> : select_kernel<false>;
    return launch_kernel(kernel, row_grid(d.Na, slices), dim3(B), 0, st,
                  reinterpret_cast<const uint4*>(gathered), gathered_scales, reinterpret_cast<uint4*>(recv), recv_scales,
                  reinterpret_cast<const HandleRecord*>(ws.recv_meta), ws.rank_recv_off, d.P, d.T, d.Tp, L, d.scales,
                  slices);
}

hipError_t launch_exchange(const Dims& d, const Workspace& ws, const void* send, const float* send_scales,
                           void* recv, float* recv_scales, bool affine, hipStream_t st) {
    if (d.Na == 0) return hipSuccess;
    const int L = d.row_units;
    const int B = pick_block(L);
    const int slices = (L + B - 1) / B;
    if (affine) {
        const TokenGrid tg = token_grid(d, slices, true);
        return launch_kernel(exchange_affine_kernel, tg.grid(), dim3(B), 0, st, ws.send_pos, ws.recv_pos,
                             reinterpret_cast<const uint4*>(send), L, d.k, d.T, B, tg.groups, tg.slices, tg.tpb_log2,
                             tg.m_log2, reinterpret_cast<uint4*>(recv), d.scales, reinterpret_cast<const uint4*>(ws.send_meta),
                             reinterpret_cast<uint4*>(ws.recv_meta), send_scales, recv_scales);
    }
    const bool gather = streaming(d, 2LL * d.Na * (16LL * L + 4LL * d.scales));
    auto kernel = gather ? exchange_kernel<true> : exchange_kernel<false>;
    const int Bx = gather ? kStreamBlock : B;
    const int sx = (L + Bx - 1) / Bx;
    return launch_kernel(kernel, row_grid(d.Na, sx), dim3(Bx), 0, st, gather ? ws.recv_to_send : ws.send_to_recv,
                         reinterpret_cast<const uint4*>(send), reinterpret_cast<uint4*>(recv), L, sx, Bx, d.scales,
                         reinterpret_cast<const uint4*>(ws.send_meta), reinterpret_cast<uint4*>(ws.recv_meta),
                         send_scales, recv_scales);
}

hipError_t launch_reverse_exchange(const Dims& d, const Workspace& ws, const uint16_t* expert_out, uint16_t* comb,
                                   bool affine, hipStream_t st) {
    if (d.Na == 0) return hipSuccess;
    const int L = d.out_units;
    const int B = pick_block(L);
    const int slices = (L + B - 1) / B;
    if (affine) {
        const TokenGrid tg = token_grid(d, slices, true);
        return launch_kernel(reverse_exchange_affine_kernel, tg.grid(), dim3(B), 0, st, ws.recv_pos,
                             reinterpret_cast<const uint4*>(expert_out), reinterpret_cast<uint4*>(comb), L, d.k, d.T, B,
                             tg.groups, tg.slices, tg.tpb_log2, tg.m_log2);
    }
    if (streaming(d, 2LL * d.Na * 16LL * L)) {
        const int Br = kStreamBlock;
        const int sr = (L + Br - 1) / Br;
        return launch_kernel(reverse_exchange_gather_kernel, row_grid(d.Na, sr), dim3(Br), 0, st,
                             reinterpret_cast<const uint4*>(expert_out), reinterpret_cast<uint4*>(comb), ws.recv_pos, L,
                             sr);
    }
    return launch_kernel(reverse_exchange_scatter_kernel, row_grid(d.Na, slices), dim3(B), 0, st,
                         reinterpret_cast<const uint4*>(expert_out), reinterpret_cast<uint4*>(comb),
                         reinterpret_cast<const HandleRecord*>(ws.recv_meta), d.Tp, d.k, L, slices);
}

}  // namespace moe
