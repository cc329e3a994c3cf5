// pack.hip -- stable permute-and-pack of the hidden rows into the send buffer,
// with the combine handle, and FP8 E4M3 quantisation on the way.
//
// Follows "Expert Parallel: MoE Token 为什么要两次穿过 GPU 网络", section
// "Dispatch 前为什么必须 count 和 permute" ("按目的地写入连续 buffer": each
// assignment writes the hidden state, its local expert id, its source token
// index and its top-k slot / weight into its destination's range), and
// "[Infra-10] All-to-All Optimization" 4.3 (write the permutation straight into
// the communication buffer, coalesced) and 4.1 (quantise before sending).
//
// One token per workgroup slice: the token's row is read once (16-byte loads)
// and written to its k send rows; the FP8 form is computed once per token and
// copied k times.  FP8: a lane owns 16 channels, 8 lanes a 128-channel block;
// amax by xor shuffles, scale = amax / 448 (fp32 division), code =
// e4m3(x / scale) (fp32 division, then v_cvt_pk_fp8_f32: nearest even).  The positions of the k
// assignments are send_off[s][e] + bucket rank and recv_off[s][e] + bucket
// rank; the first slice also writes the handle record, the position arrays and
// the send <-> receive maps that the exchange uses.  The direct form writes each
// row, scale and record straight to its receive row instead ("[Infra-10]
// All-to-All Optimization" 4.3: permute straight into the destination buffer;
// "高效且便携的专家混合通信", further improvements: over a shared-memory link,
// buffers shared across devices remove copies), which models a peer write
// over the link and leaves no send buffer to exchange.  Large problems load x
// nontemporally; the k row stores stay temporal (nontemporal stores of k = 8
// scattered rows ran at 60% of the temporal bandwidth on gfx950).
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

template <bool FP8, bool NTL = false, bool NTS = false, bool DIRECT = false>
__global__ __launch_bounds__(512) void pack_kernel(const uint4* __restrict__ x, const int32_t* __restrict__ ids,
                                                   const float* __restrict__ w,
                                                   const int32_t* __restrict__ bucket_rank,
                                                   const int32_t* __restrict__ send_off,
                                                   const int32_t* __restrict__ recv_off,
                                                   uint4* __restrict__ dst, float* __restrict__ dst_scales,
                                                   HandleRecord* __restrict__ dst_meta, int32_t* __restrict__ send_to_recv,
                                                   int32_t* __restrict__ recv_to_send,
                                                   int32_t* __restrict__ send_pos, int32_t* __restrict__ recv_pos,
                                                   int Tp, int E, int Ep, int P, int k, int L, int slices) {
    __shared__ int32_t pos[32];
    const int t = blockIdx.x;
    const int slice = blockIdx.y;
    const int s = t / Tp;
    const int tid = threadIdx.x;
    const int u = slice * blockDim.x + tid;   // 16-byte output unit of the row

    // the row's loads go out first so they overlap the position lookups below
    uint4 xa = make_uint4(0u, 0u, 0u, 0u), xb = xa;
    if (u < L) {
        if (FP8) {
            xa = ld16<NTL>(&x[(size_t)t * (2 * L) + 2 * u]);
            xb = ld16<NTL>(&x[(size_t)t * (2 * L) + 2 * u + 1]);
        } else {
            xa = ld16<NTL>(&x[(size_t)t * L + u]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    if (tid < k) {
        const int a = t * k + tid;
        const int e = ids[a];
        const int br = bucket_rank[a];
        const int p = send_off[s * E + e] + br;
        const int q = recv_off[s * E + e] + br;
        pos[tid] = DIRECT ? q : p;
        if (slice == 0) {
            send_pos[a] = p;
            recv_pos[a] = q;
            if (!DIRECT) {
                send_to_recv[p] = q;
                recv_to_send[q] = p;
            }
            HandleRecord m;
            m.src_rank = s;
            m.src_token = t - s * Tp;
            m.slot = (int16_t)tid;
            m.local_expert = (int16_t)(e % Ep);
            m.weight = w[a];
            dst_meta[DIRECT ? q : p] = m;
        }
    }
    __syncthreads();

    if (FP8) {
        // lanes u..u+7 share a 128-channel block; L % 8 == 0 and blocks start at
        // multiples of 64 lanes, so a block's lanes are all valid or all not
        if (u >= L) return;
        float f[16];
        {
            float lo[8], hi[8];
            unpack8_bf16(xa, lo);
            unpack8_bf16(xb, hi);
#pragma unroll
            for (int i = 0; i < 8; ++i) { f[i] = lo[i]; f[8 + i] = hi[i]; }
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
        amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
        amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
        const float scale = amax / 448.0f;
        uint32_t q[4];
        if (amax == 0.0f) {                       // all zeros: scale 0, codes keep each zero's sign
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                q[w4] = 0u;
#pragma unroll
                for (int i = 0; i < 4; ++i) q[w4] |= ((__float_as_uint(f[4 * w4 + i]) >> 24) & 0x80u) << (8 * i);
            }
        } else {
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4)
                q[w4] = pack4_e4m3(f[4 * w4] / scale, f[4 * w4 + 1] / scale, f[4 * w4 + 2] / scale,
                                   f[4 * w4 + 3] / scale);
        }
        const uint4 out = make_uint4(q[0], q[1], q[2], q[3]);
        const int nb = L / 8;
        for (int j = 0; j < k; ++j) {
            const int p = pos[j];
            st16<NTS>(&dst[(size_t)p * L + u], out);
            if ((u & 7) == 0) dst_scales[(size_t)p * nb + (u >> 3)] = scale;
        }
    } else {
        if (u >= L) return;
        for (int j = 0; j < k; ++j) st16<NTS>(&dst[(size_t)pos[j] * L + u], xa);
    }
}

}  // namespace

hipError_t launch_pack(const Dims& d, const uint16_t* x, const int32_t* ids, const float* w, const Workspace& ws,
                       void* dst, float* dst_scales, bool direct, hipStream_t st) {
    if (d.T == 0) return hipSuccess;
    const int L = d.row_units;                 // 16-byte output units per dispatched row
    const int B = pick_block(L);
    const int slices = (L + B - 1) / B;
    const bool nt = streaming(d, 2LL * d.H * d.T + d.Na * (16LL * L + 4LL * d.scales));
    auto kernel = pack_kernel<false, false, false, false>;
    if (d.fp8) {
        if (direct) kernel = nt ? pack_kernel<true, true, false, true> : pack_kernel<true, false, false, true>;
        else kernel = nt ? pack_kernel<true, true, false, false> : pack_kernel<true, false, false, false>;
    } else {
        if (direct) kernel = nt ? pack_kernel<false, true, false, true> : pack_kernel<false, false, false, true>;
        else kernel = nt ? pack_kernel<false, true, false, false> : pack_kernel<false, false, false, false>;
    }
    hipLaunchKernelGGL(kernel, dim3((unsigned)d.T, (unsigned)slices), dim3(B), 0, st,
                       reinterpret_cast<const uint4*>(x), ids, w, ws.bucket_rank, ws.send_off, ws.recv_off,
                       reinterpret_cast<uint4*>(dst), dst_scales,
                       reinterpret_cast<HandleRecord*>(direct ? ws.recv_meta : ws.send_meta), ws.send_to_recv,
                       ws.recv_to_send, ws.send_pos, ws.recv_pos, d.Tp, d.E, d.Ep, d.P, d.k, L, slices);
    return hipGetLastError();
}

}  // namespace moe
