// reduce.hip -- routing-weighted top-k reduction back into original token
// order ("Expert Parallel: MoE Token ..." section "Combine 不是简单把结果发回来":
// the outputs of a token's k assignments are summed with the router weights;
// "高效且便携的专家混合通信": the combine receiver writes the weighted sum into a
// caller-allocated tensor).
//
// y[t] = bf16(acc), acc = fma(w[t][j], comb[t*k + j], acc) for j = 0..k-1 from
// acc = 0, in fp32: the combine rows of a token are adjacent, so a lane reads
// its 16 bytes of each of the k rows and writes 16 bytes of y.  Large problems
// stream (nontemporal loads, ~16% faster for k = 8 rows of 14 KiB).
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

template <bool NTL, bool NTS>
__global__ __launch_bounds__(512) void reduce_kernel(const uint4* __restrict__ comb, const float* __restrict__ w,
                                                     uint4* __restrict__ y, int k, int L, int slices) {
    const int t = blockIdx.x / slices;
    const int slice = blockIdx.x - t * slices;
    const int u = slice * blockDim.x + threadIdx.x;
    if (u >= L) return;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    const uint4* rows = comb + (size_t)t * k * L + u;
    for (int j = 0; j < k; ++j) {
        const float wj = w[(size_t)t * k + j];
        float f[8];
        unpack8_bf16(ld16<NTL>(&rows[(size_t)j * L]), f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj, f[i], acc[i]);
    }
    st16<NTS>(&y[(size_t)t * L + u], pack8_bf16(acc));
}

}  // namespace

hipError_t launch_reduce(const Dims& d, const uint16_t* comb, const float* w, uint16_t* y, hipStream_t st) {
    if (d.T == 0) return hipSuccess;
    const int L = d.out_units;
    const int B = pick_block(L);
    const int slices = (L + B - 1) / B;
    auto kernel = streaming(d, (d.Na + d.T) * 16LL * L) ? reduce_kernel<true, true> : reduce_kernel<false, false>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)((long long)d.T * slices)), dim3(B), 0, st,
                       reinterpret_cast<const uint4*>(comb), w, reinterpret_cast<uint4*>(y), d.k, L, slices);
    return hipGetLastError();
}

}  // namespace moe
