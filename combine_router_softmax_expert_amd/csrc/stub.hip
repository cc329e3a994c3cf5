// stub.hip -- per-expert scalar stand-in for the grouped GEMM that consumes the
// expert-contiguous receive rows ("[Infra-10] All-to-All Optimization" 5.2:
// the receive layout is the expert kernel's input; "Expert Parallel: MoE Token
// ..." worked example: each rank runs its local experts on what it received).
//
// expert_out[q] = bf16(deq(recv[q]) * m_e), m_e = (E + e) / E in fp32, with e
// the global expert of receive row q: local expert from the row's handle record
// and owner rank from the receive-region offsets (a wave ballot over
// rank_recv_off).  deq is the bf16 value itself, or code * scale in fp32 for
// e4m3 rows (decoded exactly by v_cvt_pk_f32_fp8).  Each product rounds to fp32
// and the result once to bf16.
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// One 16-byte unit of a bf16 row times m_e, rounded once to bf16.
__device__ __forceinline__ uint4 scale_bf16_unit(const uint4& c, float m) {
    float f[8];
    unpack8_bf16(c, f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = f[i] * m;
    return pack8_bf16(f);
}

// bf16 rows: one lane per 16-byte unit in and out.  e4m3 rows: a lane reads 16
// codes as two 8-byte pieces, 64 pieces apart, and writes their two 16-byte
// outputs, so that each wave-wide store covers 1 KiB contiguously (one 16-byte
// load of adjacent codes with two half-line stores ran 12% slower at 4096 rows
// and 4% slower at 65536 rows on gfx950; one 8-byte piece per lane, 25% slower).
// A workgroup slice covers bs (the workgroup size) 16-code units, 2 * bs
// pieces; a wave covers 128 pieces (bs is a multiple of 64).
template <bool FP8, bool NTL, bool NTS>
__global__ __launch_bounds__(512) void stub_kernel(const uint4* __restrict__ recv, const HandleRecord* __restrict__ meta,
                                                   const int32_t* __restrict__ rank_recv_off,
                                                   uint4* __restrict__ out, int P, int E, int Ep, int L, int slices,
                                                   int bs, const float* __restrict__ scales) {
    const auto [q, slice] = row_slice(slices);
    // every load first, unconditional at clamped addresses, so that all of them
    // are in flight before the first wait: one memory round trip in all
    if constexpr (FP8) {
        const int lane = threadIdx.x & (kWave - 1);
        const int p0 = 2 * (slice * bs + ((int)threadIdx.x - lane)) + lane;   // 8-code pieces
        const int p1 = p0 + kWave;
        const int n = 2 * L;                                    // pieces per row
        const uint2* row = reinterpret_cast<const uint2*>(recv) + (size_t)q * n;
        const uint2 a = ld8<NTL>(&row[min(p0, n - 1)]);
        const uint2 b = ld8<NTL>(&row[min(p1, n - 1)]);
        const float sa = scales[(size_t)q * (L / 8) + (min(p0, n - 1) >> 4)];   // 16 pieces per 128-channel block
        const float sb = scales[(size_t)q * (L / 8) + (min(p1, n - 1) >> 4)];
        const int local = meta[q].local_expert;
        __builtin_amdgcn_sched_barrier(0);
        const int r = owner_rank(rank_recv_off, P, q);
        const float m = (float)(E + r * Ep + local) / (float)E;
        float f[8];
        if (p0 < n) {
            unpack4_e4m3(a.x, f);
            unpack4_e4m3(a.y, f + 4);
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = (f[i] * sa) * m;
            st16_row<NTS>(out, q, n, p0, pack8_bf16(f));
        }
        if (p1 < n) {
            unpack4_e4m3(b.x, f);
            unpack4_e4m3(b.y, f + 4);
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = (f[i] * sb) * m;
            st16_row<NTS>(out, q, n, p1, pack8_bf16(f));
        }
    } else {
        const int u = slice * bs + threadIdx.x;                 // 16-byte unit
        const uint4 c = ld16<NTL>(&recv[(size_t)q * L + min(u, L - 1)]);
        const int local = meta[q].local_expert;
        __builtin_amdgcn_sched_barrier(0);
        const int r = owner_rank(rank_recv_off, P, q);
        const float m = (float)(E + r * Ep + local) / (float)E;
        if (u >= L) return;
        st16_row<NTS>(out, q, L, u, scale_bf16_unit(c, m));
    }
}

// Token-affine form for bf16 rows (token_affine): workgroup (t, j, slice) scales
// receive row recv_pos[t*k + j] on the XCD whose L2 holds what the exchange (or
// the direct pack) wrote there.
__global__ __launch_bounds__(512) void stub_affine_kernel(const int32_t* __restrict__ recv_pos,
                                                          const uint4* __restrict__ recv,
                                                          const HandleRecord* __restrict__ meta, int L, int k, int T,
                                                          int bs, int tg_groups, int tg_slices, int tg_tpb_log2,
                                                          int tg_m_log2, uint4* __restrict__ out,
                                                          const int32_t* __restrict__ rank_recv_off,
                                                          int P, int E, int Ep) {
    int t, j, slice;
    if (!token_item(tg_groups, tg_slices, tg_tpb_log2, tg_m_log2, T, t, j, slice)) return;
    const int q = recv_pos[t * k + j];
    const int u = slice * bs + threadIdx.x;
    const uint4 c = recv[(size_t)q * L + min(u, L - 1)];
    const int local = meta[q].local_expert;
    __builtin_amdgcn_sched_barrier(0);
    const int r = owner_rank(rank_recv_off, P, q);
    const float m = (float)(E + r * Ep + local) / (float)E;
    if (u < L) out[(size_t)q * L + u] = scale_bf16_unit(c, m);   // write-back: read next on this XCD
}

}  // namespace

hipError_t launch_stub(const Dims& d, const Workspace& ws, const void* recv, const float* recv_scales, uint16_t* out,
                       bool affine, hipStream_t st) {
    if (d.Na == 0) return hipSuccess;
    const int L = d.row_units;
    const int B = pick_block(L);
    const int slices = (L + B - 1) / B;
    if (affine) {   // bf16 rows
        const TokenGrid tg = token_grid(d, slices, true);
        return launch_kernel(stub_affine_kernel, tg.grid(), dim3(B), 0, st, ws.recv_pos,
                             reinterpret_cast<const uint4*>(recv), reinterpret_cast<const HandleRecord*>(ws.recv_meta),
                             L, d.k, d.T, B, tg.groups, tg.slices, tg.tpb_log2, tg.m_log2,
                             reinterpret_cast<uint4*>(out), ws.rank_recv_off, d.P, d.E, d.Ep);
    }
    const bool nt = streaming(d, d.Na * (16LL * L + 4LL * d.scales + 2LL * d.H));
    // streaming: e4m3 rows load and store nontemporally (stub 224 -> 231 us but the reverse exchange
    // after it 320 -> 307 us at 65536 rows: no dirty lines left behind), bf16 rows store nontemporally
    auto kernel = d.fp8 ? (nt ? stub_kernel<true, true, true> : stub_kernel<true, false, false>)
                        : (nt ? stub_kernel<false, false, true> : stub_kernel<false, false, false>);
    const int Bs = nt ? kStreamBlock : B;
    const int ss = (L + Bs - 1) / Bs;
    return launch_kernel(kernel, row_grid(d.Na, ss), dim3(Bs), 0, st, reinterpret_cast<const uint4*>(recv),
                         reinterpret_cast<const HandleRecord*>(ws.recv_meta), ws.rank_recv_off,
                         reinterpret_cast<uint4*>(out), d.P, d.E, d.Ep, L, ss, Bs, recv_scales);
}

}  // namespace moe
