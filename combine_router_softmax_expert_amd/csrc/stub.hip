// stub.hip -- per-expert scalar stand-in for the grouped GEMM that consumes the
// expert-contiguous receive rows ("[Infra-10] All-to-All Optimization" 5.2:
// the receive layout is the expert kernel's input; "Expert Parallel: MoE Token
// ..." worked example: each rank runs its local experts on what it received).
//
// expert_out[q] = bf16(deq(recv[q]) * m_e), m_e = (E + e) / E in fp32, with e
// the global expert of receive row q: local expert from the row's handle record
// and owner rank from the receive-region offsets (a wave ballot over
// rank_recv_off).  deq is the bf16 value itself, or code * scale in fp32 for
// e4m3 rows (lane = 16 codes of one 128-channel block, decoded exactly by
// v_cvt_pk_f32_fp8).  Each product rounds
// to fp32 and the result once to bf16.
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// bf16 rows: one lane per 16-byte unit in and out.  e4m3 rows: one lane per 16
// codes (a 16-byte load) and two 16-byte stores; with half-width (8-byte) code
// loads instead, the kernel ran ~25% slower on gfx950, and the split stores must
// stay temporal (nontemporal ones cannot merge the half-lines and ran ~40% slower).
template <bool FP8, bool NTL, bool NTS>
__global__ __launch_bounds__(512) void stub_kernel(const uint4* __restrict__ recv, const float* __restrict__ scales,
                                                   const HandleRecord* __restrict__ meta,
                                                   const int32_t* __restrict__ rank_recv_off,
                                                   uint4* __restrict__ out, int P, int E, int Ep, int L, int slices) {
    const auto [q, slice] = row_slice(slices);
    const int u = slice * blockDim.x + threadIdx.x;   // input unit of 16 bytes
    // every load first, unconditional at clamped addresses, so that all of them
    // are in flight before the first wait: one memory round trip in all
    const int uc = min(u, L - 1);
    const uint4 c = ld16<NTL>(&recv[(size_t)q * L + uc]);
    float sc = 0.0f;
    if constexpr (FP8) sc = scales[(size_t)q * (L / 8) + (uc >> 3)];
    const int local = meta[q].local_expert;
    __builtin_amdgcn_sched_barrier(0);
    const int r = owner_rank(rank_recv_off, P, q);
    const int e = r * Ep + local;
    const float m = (float)(E + e) / (float)E;
    if (u >= L) return;
    if (FP8) {
        float f[16];
        unpack4_e4m3(c.x, f);
        unpack4_e4m3(c.y, f + 4);
        unpack4_e4m3(c.z, f + 8);
        unpack4_e4m3(c.w, f + 12);
        float lo[8], hi[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float a = f[i] * sc, b = f[8 + i] * sc;
            lo[i] = a * m;
            hi[i] = b * m;
        }
        st16<NTS>(&out[(size_t)q * (2 * L) + 2 * u], pack8_bf16(lo));
        st16<NTS>(&out[(size_t)q * (2 * L) + 2 * u + 1], pack8_bf16(hi));
    } else {
        float f[8];
        unpack8_bf16(c, f);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = f[i] * m;
        st16<NTS>(&out[(size_t)q * L + u], pack8_bf16(f));
    }
}

}  // namespace

hipError_t launch_stub(const Dims& d, const Workspace& ws, const void* recv, const float* recv_scales, uint16_t* out,
                       hipStream_t st) {
    if (d.Na == 0) return hipSuccess;
    const int L = d.row_units;
    const int B = pick_block(L);
    const int slices = (L + B - 1) / B;
    const bool nt = streaming(d, d.Na * (16LL * L + 4LL * d.scales + 2LL * d.H));
    // streaming: e4m3 rows load nontemporally, bf16 rows store nontemporally (best of the four choices each)
    auto kernel = d.fp8 ? (nt ? stub_kernel<true, true, false> : stub_kernel<true, false, false>)
                        : (nt ? stub_kernel<false, false, true> : stub_kernel<false, false, false>);
    launch_kernel(kernel, row_grid(d.Na, slices), dim3(B), 0, st, reinterpret_cast<const uint4*>(recv), recv_scales,
                  reinterpret_cast<const HandleRecord*>(ws.recv_meta), ws.rank_recv_off, reinterpret_cast<uint4*>(out),
                  d.P, d.E, d.Ep, L, slices);
    return hipGetLastError();
}

}  // namespace moe
