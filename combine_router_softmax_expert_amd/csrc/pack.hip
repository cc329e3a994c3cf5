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
// the send <-> receive maps that the exchange uses.  Large problems load x
// nontemporally; the k row stores stay temporal (nontemporal stores of k = 8
// scattered rows ran at 60% of the temporal bandwidth on gfx950).
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

struct Meta {
    int32_t src_rank;
    int32_t src_token;
    int16_t slot;
    int16_t local_expert;
    float weight;
};
static_assert(sizeof(Meta) == 16, "handle record is 16 bytes");

template <bool FP8, bool NTL = false, bool NTS = false>
__global__ __launch_bounds__(512) void pack_kernel(const uint4* __restrict__ x, const int32_t* __restrict__ ids,
                                                   const float* __restrict__ w,
                                                   const int32_t* __restrict__ bucket_rank,
                                                   const int32_t* __restrict__ send_off,
                                                   const int32_t* __restrict__ recv_off,
                                                   uint4* __restrict__ send, float* __restrict__ send_scales,
                                                   Meta* __restrict__ send_meta, int32_t* __restrict__ send_to_recv,
                                                   int32_t* __restrict__ recv_to_send,
                                                   int32_t* __restrict__ send_pos, int32_t* __restrict__ recv_pos,
                                                   int Tp, int E, int Ep, int P, int k, int L, int slices) {
    __shared__ int32_t pos[32];
    const int t = blockIdx.x / slices;
    const int slice = blockIdx.x - t * slices;
    const int s = t / Tp;
    const int tid = threadIdx.x;

    if (tid < k) {
        const int a = t * k + tid;
        const int e = ids[a];
        const int br = bucket_rank[a];
        const int p = send_off[s * E + e] + br;
        pos[tid] = p;
        if (slice == 0) {
            const int q = recv_off[s * E + e] + br;
            send_pos[a] = p;
            recv_pos[a] = q;
            send_to_recv[p] = q;
            recv_to_send[q] = p;
            Meta m;
            m.src_rank = s;
            m.src_token = t - s * Tp;
            m.slot = (int16_t)tid;
            m.local_expert = (int16_t)(e % Ep);
            m.weight = w[a];
            send_meta[p] = m;
        }
    }
    __syncthreads();

    const int u = slice * blockDim.x + tid;   // 16-byte output unit of the row
    if (FP8) {
        // lanes u..u+7 share a 128-channel block; L % 8 == 0 and blocks start at
        // multiples of 64 lanes, so a block's lanes are all valid or all not
        if (u >= L) return;
        const uint4 a = ld16<NTL>(&x[(size_t)t * (2 * L) + 2 * u]);
        const uint4 b = ld16<NTL>(&x[(size_t)t * (2 * L) + 2 * u + 1]);
        float f[16];
        {
            float lo[8], hi[8];
            unpack8_bf16(a, lo);
            unpack8_bf16(b, hi);
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
            st16<NTS>(&send[(size_t)p * L + u], out);
            if ((u & 7) == 0) send_scales[(size_t)p * nb + (u >> 3)] = scale;
        }
    } else {
        if (u >= L) return;
        const uint4 v = ld16<NTL>(&x[(size_t)t * L + u]);
        for (int j = 0; j < k; ++j) st16<NTS>(&send[(size_t)pos[j] * L + u], v);
    }
}

}  // namespace

hipError_t launch_pack(const Dims& d, const uint16_t* x, const int32_t* ids, const float* w, const Workspace& ws,
                       void* send, float* send_scales, hipStream_t st) {
    if (d.T == 0) return hipSuccess;
    const int L = d.row_units;                 // 16-byte output units per send row
    const int B = pick_block(L);
    const int slices = (L + B - 1) / B;
    const long long blocks = (long long)d.T * slices;
    const bool nt = streaming(d, 2LL * d.H * d.T + d.Na * (16LL * L + 4LL * d.scales));
    auto kernel = d.fp8 ? (nt ? pack_kernel<true, true, false> : pack_kernel<true, false, false>)
                        : (nt ? pack_kernel<false, true, false> : pack_kernel<false, false, false>);
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(B), 0, st, reinterpret_cast<const uint4*>(x), ids, w,
                       ws.bucket_rank, ws.send_off, ws.recv_off, reinterpret_cast<uint4*>(send), send_scales,
                       reinterpret_cast<Meta*>(ws.send_meta), ws.send_to_recv, ws.recv_to_send, ws.send_pos,
                       ws.recv_pos, d.Tp, d.E, d.Ep, d.P, d.k, L, slices);
    return hipGetLastError();
}

}  // namespace moe
