// reduce.hip -- routing-weighted top-k reduction back into original token
// order ("Expert Parallel: MoE Token ..." section "Combine 不是简单把结果发回来":
// the outputs of a token's k assignments are summed with the router weights;
// "高效且便携的专家混合通信": the combine receiver writes the weighted sum into a
// caller-allocated tensor).
//
// y[t] = bf16(acc), acc = fma(w[t][j], comb[t*k + j], acc) for j = 0..k-1 from
// acc = 0, in fp32: the combine rows of a token are adjacent, so a lane reads
// its 16 bytes of each of the k rows and writes 16 bytes of y.  The direct form
// reads row recv_pos[t*k + j] of the expert output instead, gathering through
// the handle with no combine buffer in between.  Large problems
// stream (nontemporal loads, ~16% faster for k = 8 rows of 14 KiB).
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// Up to kChunk rows are loaded before their fused multiply-adds, which still
// run in slot order.
constexpr int kChunk = 8;

// Token t's slice of y, the lane's 16-byte unit u.
template <bool NTL, bool NTS, bool DIRECT>
__device__ __forceinline__ void reduce_unit(const uint4* __restrict__ rows, const int32_t* __restrict__ recv_pos,
                                            const float* __restrict__ w, uint4* __restrict__ y, int k, int L, int t,
                                            int u) {
    if (u >= L) return;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += kChunk) {
        uint4 v[kChunk];
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            if (j0 + j < k) {
                const int a = t * k + j0 + j;               // combine row of slot j0 + j
                const int row = DIRECT ? recv_pos[a] : a;   // direct: the expert output itself
                v[j] = ld16<NTL>(&rows[(size_t)row * L + u]);
            }
        }
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
            if (j0 + j < k) {
                const float wj = w[(size_t)t * k + j0 + j];
                float f[8];
                unpack8_bf16(v[j], f);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj, f[i], acc[i]);
            }
        }
    }
    st16_row<NTS>(y, t, L, u, pack8_bf16(acc));
}

// Row grid over the tokens (row_grid).
template <bool NTL, bool NTS, bool DIRECT>
__global__ __launch_bounds__(512) void reduce_kernel(const uint4* __restrict__ rows, const int32_t* __restrict__ recv_pos,
                                                     const float* __restrict__ w, uint4* __restrict__ y, int k, int L,
                                                     int bs, int slices) {
    const auto [t, slice] = row_slice(slices);
    reduce_unit<NTL, NTS, DIRECT>(rows, recv_pos, w, y, k, L, t, slice * bs + threadIdx.x);
}

// The token-affine grid (token_affine), which serves token t's slice on the
// XCD whose L2 holds that token's rows.  The grid's fields come as scalars: an
// aggregate argument would end the arguments preloaded into SGPRs.
template <bool DIRECT>
__global__ __launch_bounds__(512) void reduce_affine_kernel(const uint4* __restrict__ rows,
                                                            const int32_t* __restrict__ recv_pos, int k, int L, int bs,
                                                            int tg_groups, int tg_slices, int tg_tpb_log2,
                                                            int tg_m_log2, int T, const float* __restrict__ w,
                                                            uint4* __restrict__ y) {
    int t, j, slice;
    if (!token_item(tg_groups, tg_slices, tg_tpb_log2, tg_m_log2, T, t, j, slice)) return;
    reduce_unit<false, false, DIRECT>(rows, recv_pos, w, y, k, L, t, slice * bs + threadIdx.x);
}

}  // namespace

hipError_t launch_reduce(const Dims& d, const uint16_t* rows, const int32_t* recv_pos, const float* w, uint16_t* y,
                         bool direct, bool affine, hipStream_t st) {
    if (d.T == 0) return hipSuccess;
    const int L = d.out_units;
    if (affine) {
        const int B = pick_block(L);
        const int slices = (L + B - 1) / B;
        const TokenGrid tg = token_grid(d, slices, false);
        auto kernel = direct ? reduce_affine_kernel<true> : reduce_affine_kernel<false>;
        return launch_kernel(kernel, tg.grid(), dim3(B), 0, st, reinterpret_cast<const uint4*>(rows), recv_pos, d.k, L,
                             B, tg.groups, tg.slices, tg.tpb_log2, tg.m_log2, d.T, w, reinterpret_cast<uint4*>(y));
    }
    const bool nt = streaming(d, (d.Na + d.T) * 16LL * L);
    // streaming: two-wave workgroups, seven per 7168-channel row (measured on gfx950 at 8192 tokens x top-8,
    // whole step 993 -> 987 us, direct form 547 -> 541 us; 16384 tokens x top-2 at 4096 channels unchanged;
    // the temporal sizes below it were as fast or faster with the row-dividing workgroup)
    const int B = nt ? std::min(128, pick_block(L)) : pick_block(L);
    const int slices = (L + B - 1) / B;
    auto kernel = direct ? (nt ? reduce_kernel<true, true, true> : reduce_kernel<false, false, true>)
                         : (nt ? reduce_kernel<true, true, false> : reduce_kernel<false, false, false>);
    return launch_kernel(kernel, row_grid(d.T, slices), dim3(B), 0, st, reinterpret_cast<const uint4*>(rows), recv_pos,
                         w, reinterpret_cast<uint4*>(y), d.k, L, B, slices);
}

}  // namespace moe
