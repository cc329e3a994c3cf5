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
// amax by DPP moves within the 8 lanes, scale = amax / 448 and code =
// e4m3(x / scale), each quotient the correctly rounded fp32 one (for x / scale,
// or one on the same side of every E4M3 rounding boundary; see store_rows),
// encoded by v_cvt_pk_fp8_f32 (nearest even).  The positions of the k
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
//
// Counting form (small problems, where a separate count launch costs more than
// the counting itself): every workgroup ranks its tokens' k assignments by
// itself from all N_a expert ids, which sit in the cache.  With tokens blocked
// by rank and each token's experts distinct, the stable positions have a
// closed form in counts (the send order is local expert then token, the
// receive order expert then source rank then token, as in the worked example of
// "Expert Parallel: MoE Token ..."): for assignment (t, j) with expert e on
// rank s,
//   recv_pos = #{a : id_a < e} + #{a : id_a = e, token(a) < t}
//   send_pos = s*(T/P)*k + the same two counts over rank s's assignments only.
// LDS histograms of the ids and one prefix sum give these counts (see
// count_pack_kernel).  P extra workgroups, one per source rank, write the
// counts and offsets of the handle (n, N, C, expert_off, rank_recv_off,
// send_off, recv_off) from LDS histograms in the same launch.
#include <algorithm>
#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kMaxIdsPerThread = 16;   // expert ids a thread of the counting form keeps in registers
constexpr int kMaxRanksPerStore = 32;  // row copies the all-gather writes per pass

// Maximum over each aligned group of 8 lanes, in every lane of the group, by
// three DPP moves (no LDS traffic): quad_perm [1,0,3,2] and [2,3,0,1] give
// each quad its maximum, then row_half_mirror (lane i of each group of 8 reads
// lane 7 - i, which sits in the other quad) combines the two quads.  A group
// is all active or all inactive, so no lane reads a disabled one.
template <int Ctrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), Ctrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float max8(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    return fmaxf(v, dpp_f32<0x141>(v));
}

// The token's row, loaded before anything else so its latency overlaps the
// position work (FP8 reads 32 bytes of bf16 per 16-byte output unit).
template <bool FP8, bool NTL>
__device__ __forceinline__ void load_row(const uint4* __restrict__ x, int t, int L, int u, uint4& xa, uint4& xb) {
    xa = make_uint4(0u, 0u, 0u, 0u);
    xb = xa;
    if (u < L) {
        if (FP8) {
            xa = ld16<NTL>(&x[(size_t)t * (2 * L) + 2 * u]);
            xb = ld16<NTL>(&x[(size_t)t * (2 * L) + 2 * u + 1]);
        } else {
            xa = ld16<NTL>(&x[(size_t)t * L + u]);
        }
    }
}

// Position arrays, and from the first slice the handle record and (base form)
// the send <-> receive maps, of assignment a = t*k + j.  Called by the lanes
// that own the slots as soon as they have the positions, before the block's
// LDS-only barrier (which does not wait for global stores) and before the row
// stores: issued after the row stores, these stores reused the row stores'
// registers, so the compiler first waited for all k row stores to complete.
// Every slice writes the (identical) positions, so that the token-affine
// kernels find them in the L2 of the XCD that serves their slice.
template <bool DIRECT>
__device__ __forceinline__ void write_handle(int a, int t, int s, int Tp, int j, int e, int Ep, int p, int q,
                                             float weight, bool first_slice, HandleRecord* __restrict__ dst_meta,
                                             int32_t* __restrict__ send_to_recv, int32_t* __restrict__ recv_to_send,
                                             int32_t* __restrict__ send_pos, int32_t* __restrict__ recv_pos) {
    send_pos[a] = p;
    recv_pos[a] = q;
    if (!first_slice) return;
    if (!DIRECT) {
        send_to_recv[p] = q;
        recv_to_send[q] = p;
    }
    HandleRecord m;
    m.src_rank = s;
    m.src_token = t - s * Tp;
    m.slot = (int16_t)j;
    m.local_expert = (int16_t)(e % Ep);
    m.weight = weight;
    dst_meta[DIRECT ? q : p] = m;
}

// The row (or its FP8 form and scales) to the k rows pos[0..k).
template <bool FP8, bool NTS>
__device__ __forceinline__ void store_rows(const uint4& xa, const uint4& xb, const int32_t* pos, int k, int L, int u,
                                           uint4* __restrict__ dst, float* __restrict__ dst_scales) {
    if (u >= L) return;
    if (FP8) {
        // lanes u..u+7 share a 128-channel block; L % 8 == 0 and blocks start at
        // multiples of 64 lanes, so a block's lanes are all valid or all not
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
        amax = max8(amax);
        float scale;
        uint32_t q[4];
        if (amax == 0.0f) {                       // all zeros: scale 0, codes keep each zero's sign
            scale = 0.0f;
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                q[w4] = 0u;
#pragma unroll
                for (int i = 0; i < 4; ++i) q[w4] |= ((__float_as_uint(f[4 * w4 + i]) >> 24) & 0x80u) << (8 * i);
            }
        } else if (amax >= 0x1p-64f && amax < __builtin_inff()) {
            // amax / 448 by a multiply with the rounded reciprocal of 448 and one
            // correction with the exact remainder: equal to the correctly rounded
            // quotient for every finite bf16 amax (checked exhaustively).
            constexpr float kInv448 = 1.0f / 448.0f;
            const float s0 = amax * kInv448;
            scale = fmaf(fmaf(-s0, 448.0f, amax), kInv448, s0);
            // x / scale through the reciprocal: q0 = x * r, then one correction with the
            // exact remainder x - q0 * scale (an FMA).  The corrected quotient can be one
            // ulp off the correctly rounded one, but never across an E4M3 rounding
            // boundary: checked for every bf16 amax >= 2^-64 and every bf16 |x| <= amax
            // (the remainder stays far from underflow there).  Three operations per
            // channel instead of a full division.  Every quotient has the sign of its x
            // but one: for x = -0 the correction adds +0 to -0 and gives +0, where
            // -0 / scale is -0 (code 0x80).  Each code's sign bit is therefore ORed
            // from its x: a byte permute gathers the high bytes of four bf16 values,
            // whose top bits are their signs, into the four code bytes.
            const float r = 1.0f / scale;
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float q0 = f[i] * r;
                v[i] = fmaf(fmaf(-q0, scale, f[i]), r, q0);
            }
            const uint32_t src[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
                q[w4] = pack4_e4m3(v[4 * w4], v[4 * w4 + 1], v[4 * w4 + 2], v[4 * w4 + 3]);
                // bytes 1 and 3 of the word holding values 4 w4 and 4 w4 + 1, then of the next word
                q[w4] |= __builtin_amdgcn_perm(src[2 * w4 + 1], src[2 * w4], 0x07050301u) & 0x80808080u;
            }
        } else {                                  // tiny or non-finite blocks: correctly rounded division
            scale = amax / 448.0f;
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4)
                q[w4] = pack4_e4m3(f[4 * w4] / scale, f[4 * w4 + 1] / scale, f[4 * w4 + 2] / scale,
                                   f[4 * w4 + 3] / scale);
        }
        const uint4 out = make_uint4(q[0], q[1], q[2], q[3]);
        const int nb = L / 8;
        for (int j = 0; j < k; ++j) {
            const int p = pos[j];
            st16_row<NTS>(dst, p, L, u, out);
            if ((u & 7) == 0) dst_scales[(size_t)p * nb + (u >> 3)] = scale;
        }
    } else {
        for (int j = 0; j < k; ++j) st16_row<NTS>(dst, pos[j], L, u, xa);
    }
}

template <bool FP8, bool NTL = false, bool NTS = false, bool DIRECT = false>
__global__ __launch_bounds__(512) void pack_kernel(const uint4* __restrict__ x, const int32_t* __restrict__ ids,
                                                   const int32_t* __restrict__ bucket_rank,
                                                   const int32_t* __restrict__ send_off,
                                                   const int32_t* __restrict__ recv_off, int Tp, int E, int k, int L,
                                                   int slices, int bs, const float* __restrict__ w, int Ep,
                                                   uint4* __restrict__ dst, float* __restrict__ dst_scales,
                                                   HandleRecord* __restrict__ dst_meta, int32_t* __restrict__ send_to_recv,
                                                   int32_t* __restrict__ recv_to_send,
                                                   int32_t* __restrict__ send_pos, int32_t* __restrict__ recv_pos) {
    __shared__ int32_t pos[32];
    const auto [t, slice] = row_slice(slices);
    const int s = t / Tp;
    const int tid = threadIdx.x;
    const int u = slice * bs + tid;           // 16-byte output unit of the row

    uint4 xa, xb;
    load_row<FP8, NTL>(x, t, L, u, xa, xb);
    __builtin_amdgcn_sched_barrier(0);

    const int a = t * k + tid;
    int e = 0, p = 0, q = 0;
    float wt = 0.0f;
    if (tid < k) {
        e = ids[a];
        const int br = bucket_rank[a];
        wt = w[a];
        p = send_off[s * E + e] + br;
        q = recv_off[s * E + e] + br;
        pos[tid] = DIRECT ? q : p;
        write_handle<DIRECT>(a, t, s, Tp, tid, e, Ep, p, q, wt, slice == 0, dst_meta, send_to_recv, recv_to_send,
                             send_pos, recv_pos);
    }
    lds_barrier();
    store_rows<FP8, NTS>(xa, xb, pos, k, L, u, dst, dst_scales);
}

// Positions and receive-side handle records only (no rows), one thread per
// assignment, for dispatchers that move the rows another way (the all-gather
// dispatcher of "Expert Parallel: MoE Token ...", section "为什么不用 AllGather
// 收集所有 token").
__global__ __launch_bounds__(256) void handle_kernel(const int32_t* __restrict__ ids, const float* __restrict__ w,
                                                     const int32_t* __restrict__ bucket_rank,
                                                     const int32_t* __restrict__ send_off,
                                                     const int32_t* __restrict__ recv_off,
                                                     HandleRecord* __restrict__ recv_meta,
                                                     int32_t* __restrict__ send_pos, int32_t* __restrict__ recv_pos,
                                                     int Na, int Tp, int E, int Ep, int k) {
    const int a = blockIdx.x * blockDim.x + threadIdx.x;
    if (a >= Na) return;
    const int t = a / k, s = t / Tp;
    const int e = ids[a];
    const int br = bucket_rank[a];
    const int p = send_off[s * E + e] + br;
    const int q = recv_off[s * E + e] + br;
    write_handle<true>(a, t, s, Tp, a - t * k, e, Ep, p, q, w[a], true, recv_meta, nullptr, nullptr, send_pos,
                       recv_pos);
}

// All-gather of the tokens ("Expert Parallel: MoE Token ...", section "为什么不用
// AllGather 收集所有 token": every rank gathers all tokens, then picks out its own
// assignments): token t's row, in its dispatched form (the FP8 codes and
// scales computed once), lands in row r*T + t of every rank r's copy.
template <bool FP8, bool NTL, bool NTS>
__global__ __launch_bounds__(512) void allgather_kernel(const uint4* __restrict__ x, uint4* __restrict__ gathered,
                                                        float* __restrict__ gathered_scales, int T, int P, int L,
                                                        int slices) {
    __shared__ int32_t pos[kMaxRanksPerStore];
    const auto [t, slice] = row_slice(slices);
    const int u = slice * blockDim.x + threadIdx.x;
    uint4 xa, xb;
    load_row<FP8, NTL>(x, t, L, u, xa, xb);
    for (int r0 = 0; r0 < P; r0 += kMaxRanksPerStore) {   // copies in groups of the position table
        const int n = min(kMaxRanksPerStore, P - r0);
        if ((int)threadIdx.x < n) pos[threadIdx.x] = (r0 + threadIdx.x) * T + t;
        lds_barrier();
        store_rows<FP8, NTS>(xa, xb, pos, n, L, u, gathered, gathered_scales);
        lds_barrier();
    }
}

// Exclusive prefix sum over the experts of the low halves of the histogram
// entries (two 16-bit counts side by side, each summing to at most N_a <= 8192,
// so no carry crosses between them) into prefix[0..E], prefix[E] the total.
// Run by one whole wave, 64 experts a row (lane l holds expert 64 i + l of row
// i): a DPP scan per row, the running total carried from row to row, and the
// next row's read issued before the current row's scan.  The other waves wait
// at the next block barrier.
__device__ __forceinline__ void wave_prefix_low(const uint64_t* __restrict__ hist, int32_t* __restrict__ prefix, int E) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t* low = reinterpret_cast<const uint32_t*>(hist);   // low half of entry e at 2 e
    const int rows = (E + kWave - 1) / kWave;
    auto row_value = [&](int e) { return e < E ? (int)low[2 * min(e, E - 1)] : 0; };   // clamped, unconditional
    int next = row_value(lane);
    int carry = 0;
    for (int i = 0; i < rows; ++i) {
        const int v = next;
        const int e = i * kWave + lane;
        next = row_value(e + kWave);
        const int incl = wave_inclusive_scan(v);
        if (e < E) prefix[e] = carry + incl - v;
        carry += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
    if (lane == 0) prefix[E] = carry;
    // the wave's lanes read each other's entries next: LDS accesses of one wave run in order
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
}

// Counts and offsets of source rank s for the handle (one workgroup of the
// counting form per rank): one LDS histogram entry per expert holding three
// 16-bit counts (all ids, rank s's ids, the ids of ranks below s), then one
// wave's prefix sum of the all-ranks and rank-s counts together.
template <int MI>
__device__ void rank_counts(const int32_t* __restrict__ ids, int s, int Tp, int E, int Ep, int k, int P, int Na, int bs,
                            int32_t* __restrict__ n, int32_t* __restrict__ N, int32_t* __restrict__ C,
                            int32_t* __restrict__ expert_off, int32_t* __restrict__ rank_recv_off,
                            int32_t* __restrict__ send_off, int32_t* __restrict__ recv_off) {
    extern __shared__ __align__(16) int32_t lds[];   // E 64-bit entries, then E + 1 prefix sums
    uint64_t* hist = reinterpret_cast<uint64_t*>(lds);
    int32_t* x_s = lds + 2 * E;
    const int tid = threadIdx.x;
    const int lo = s * Tp * k, hi = lo + Tp * k;   // rank s's assignments
    int id[MI];                                  // all loads in flight at once (Na <= MI * bs; clamped
#pragma unroll                                   // addresses keep the code straight-line, with no wait per load)
    for (int m = 0; m < MI; ++m) id[m] = ids[min(tid + m * bs, Na - 1)];
    for (int x = tid; x < E; x += bs) hist[x] = 0;
    lds_barrier();
#pragma unroll
    for (int m = 0; m < MI; ++m) {
        const int a = tid + m * bs;
        const int e = id[m];
        if (a >= Na || (unsigned)e >= (unsigned)E) continue;   // out-of-range ids are outside the contract: never indexed
        const uint64_t inc = 1ull | (a >= lo && a < hi ? 1ull << 16 : 0ull) | (a < lo ? 1ull << 32 : 0ull);
        atomicAdd(reinterpret_cast<unsigned long long*>(&hist[e]), (unsigned long long)inc);
    }
    lds_barrier();
    if (tid < kWave) wave_prefix_low(hist, x_s, E);
    lds_barrier();
    for (int e = tid; e < E; e += bs) {
        const uint64_t h = hist[e];
        const int all = (int)(h & 0xFFFF), cs = (int)((h >> 16) & 0xFFFF), below = (int)((h >> 32) & 0xFFFF);
        const int x = x_s[e];
        const int eo = x & 0xFFFF, xs = x >> 16;
        n[(size_t)s * E + e] = cs;
        send_off[(size_t)s * E + e] = lo + xs;
        recv_off[(size_t)s * E + e] = eo + below;
        if (s == 0) {
            N[e] = all;
            expert_off[e] = eo;
            if (e % Ep == 0) rank_recv_off[e / Ep] = eo;
        }
    }
    // C[s][r]: rank s's assignments to rank r's experts, from the scan
    for (int r = tid; r < P; r += bs) C[(size_t)s * P + r] = (x_s[(r + 1) * Ep] >> 16) - (x_s[r * Ep] >> 16);
    if (s == 0 && tid == 0) {
        expert_off[E] = x_s[E] & 0xFFFF;
        rank_recv_off[P] = x_s[E] & 0xFFFF;
    }
}

// Grid of ceil(T / TPB) + P rows of slices (row_grid): row b < ceil(T / TPB)
// packs tokens b*TPB .. b*TPB + TPB - 1 (all on one rank: TPB divides T/P),
// whose TPB * k <= 32 assignments ("slots") share one counting pass; row
// ceil(T / TPB) + s, slice 0, writes rank s's counts and offsets (the other
// slices of those rows exit).  The packing rows come first, so that workgroup
// b * slices + slice runs on the XCD the token-affine layout expects.
//
// For slot (t, j) with expert e on rank s, and t0 the block's first token:
//   recv_pos = #{a : id_a < e} + #{a < t0*k : id_a = e} + c
//   send_pos = s*(T/P)*k + #{a on rank s : id_a < e} + #{a on rank s, a < t0*k : id_a = e} + c
// with c = #{t0*k <= a < t*k : id_a = e} (earlier tokens of the same block).
// One LDS histogram entry per expert holds four 16-bit counts of the ids (all,
// rank s's, those before t0, rank s's before t0), so each id costs one 64-bit
// LDS atomic; one wave's prefix sum over the experts then gives the first term
// of both positions, and that wave's lanes own the slots.  Three block barriers
// in all: after clearing the histogram, after the atomics, after the positions.
template <bool FP8, bool DIRECT, int MI, int TPB, bool ROWS = true>
__global__ __launch_bounds__(512) void count_pack_kernel(const uint4* __restrict__ x, const int32_t* __restrict__ ids,
                                                         const float* __restrict__ w, int T, int Tp, int E, int k,
                                                         int L, int slices, int bs, int Ep, int P,
                                                         uint4* __restrict__ dst, float* __restrict__ dst_scales,
                                                         HandleRecord* __restrict__ dst_meta,
                                                         int32_t* __restrict__ send_to_recv,
                                                         int32_t* __restrict__ recv_to_send,
                                                         int32_t* __restrict__ send_pos, int32_t* __restrict__ recv_pos,
                                                         int32_t* __restrict__ counts) {
    __shared__ int32_t pos[32];
    __shared__ int32_t blk[32];                // the block's own expert ids
    const auto [b, slice] = row_slice(slices);
    const int tid = threadIdx.x;
    const int Na = T * k;
    const int groups = (T + TPB - 1) / TPB;
    if (b >= groups) {
        if (slice == 0) {                      // the count arrays from the workspace's start (count_layout)
            const CountLayout cl = count_layout(P, E);
            char* base = reinterpret_cast<char*>(counts);
            auto at = [&](size_t off) { return reinterpret_cast<int32_t*>(base + off); };
            rank_counts<MI>(ids, b - groups, Tp, E, Ep, k, P, Na, bs, at(cl.n), at(cl.N), at(cl.C), at(cl.expert_off),
                            at(cl.rank_recv_off), at(cl.send_off), at(cl.recv_off));
        }
        return;
    }
    const int t0 = b * TPB;
    const int ntok = min(TPB, T - t0);
    const int nslots = ntok * k;               // <= 32 by the launch condition
    const int s = t0 / Tp;                     // the block's rank
    const int u = slice * bs + tid;
    const int t0k = t0 * k, lo = s * Tp * k, hi = lo + Tp * k;

    // the ids first (coalesced, all in flight at once), then the tokens' rows: the
    // counting below waits for the ids only, and LDS-only barriers keep the rows'
    // loads in flight until the rows are stored
    // (MI ids per thread, MI * bs >= N_a; straight-line code with clamped
    // addresses, so the waits for the ids do not also wait for the rows)
    int raw[MI];
#pragma unroll
    for (int m = 0; m < MI; ++m) raw[m] = ids[min(tid + m * bs, Na - 1)];
    const int sl = min(tid, nslots - 1);       // threads < nslots own a slot
    const int my_e = ids[t0k + sl];
    const float wt = w[t0k + sl];
    __builtin_amdgcn_sched_barrier(0);
    uint4 xa[TPB], xb[TPB];
#pragma unroll
    for (int i = 0; i < TPB; ++i) {
        if (ROWS) load_row<FP8, false>(x, min(t0 + i, T - 1), L, u, xa[i], xb[i]);
    }
    __builtin_amdgcn_sched_barrier(0);

    extern __shared__ __align__(16) int32_t lds[];   // E 64-bit entries, then E + 1 prefix sums
    uint64_t* hist = reinterpret_cast<uint64_t*>(lds);
    int32_t* prefix = lds + 2 * E;             // exclusive prefix of (all | rank s << 16)
    for (int x = tid; x < E; x += bs) hist[x] = 0;
    if (tid < nslots) blk[tid] = my_e;
    lds_barrier();
#pragma unroll
    for (int m = 0; m < MI; ++m) {
        const int a = tid + m * bs;
        const int e = raw[m];
        if (a < Na && (unsigned)e < (unsigned)E) {   // out-of-range ids are outside the contract: never indexed
            const bool rank = a >= lo && a < hi, before = a < t0k;
            const uint64_t inc = 1ull | (rank ? 1ull << 16 : 0ull) | (before ? 1ull << 32 : 0ull) |
                                 (rank && before ? 1ull << 48 : 0ull);
            atomicAdd(reinterpret_cast<unsigned long long*>(&hist[e]), (unsigned long long)inc);
        }
    }
    lds_barrier();
    int p = 0, q = 0;
    if (tid < kWave) {                         // wave 0: the prefix sum, then the slots (nslots <= 32)
        wave_prefix_low(hist, prefix, E);
        if (tid < nslots) {
            const int e = min(max(my_e, 0), E - 1);   // in range for any input (out-of-range ids are outside the contract)
            int c = 0;                          // earlier tokens of this block with the same expert
            for (int b = 0; b < tid - tid % k; ++b) c += blk[b] == my_e ? 1 : 0;
            const int pe = prefix[e];
            const uint64_t h = hist[e];
            q = (pe & 0xFFFF) + (int)((h >> 32) & 0xFFFF) + c;
            p = lo + (pe >> 16) + (int)(h >> 48) + c;
            q = min(q, Na - 1);                 // no-ops for valid input; keep every write in bounds
            p = min(p, hi - 1);
            pos[tid] = DIRECT ? q : p;
            write_handle<DIRECT>(t0k + tid, t0 + tid / k, s, Tp, tid % k, my_e, Ep, p, q, wt, slice == 0, dst_meta,
                                 send_to_recv, recv_to_send, send_pos, recv_pos);
        }
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < TPB; ++i)
        if (ROWS && i < ntok) store_rows<FP8, false>(xa[i], xb[i], pos + i * k, k, L, u, dst, dst_scales);
}

}  // namespace

// Dynamic LDS of the counting form: E 64-bit histogram entries and E + 1 prefix sums.
static size_t count_pack_lds(int E) { return sizeof(uint64_t) * (size_t)E + sizeof(int32_t) * ((size_t)E + 1); }

// Ids each thread of the counting form loads (unrolled, all in flight): 4, 8, 12 or 16.
// Every id slot beyond N_a still costs its clamped load and its range test, so the
// count is rounded up to a multiple of 4 only (2048 tokens x top-2 over 448-thread
// workgroups, 9.1 ids per thread: 12 against 16 took the counting pack from 11.03 to
// 10.83 us on gfx950, bit-identical).
int ids_per_thread(long long Na, int B) {
    const long long m = (Na + B - 1) / B;
    return m <= 4 ? 4 : m <= 8 ? 8 : m <= 12 ? 12 : 16;
}

// Tokens per workgroup of the counting form: more tokens share one counting
// pass, as long as their slots fit the per-workgroup tables (TPB * k <= 32), the
// tokens of a workgroup share one rank (TPB divides T/P) and at least 1024
// workgroups remain (measured on gfx950 at 2048 tokens x top-2: 2 tokens per
// workgroup 13.4 us, 1 token 16.7 us, 4 tokens 13.6 us).
int tokens_per_block(const Dims& d) {
    const int B = pick_block(d.row_units);
    const long long slices = (d.row_units + B - 1) / B;
    for (int tpb = 4; tpb > 1; tpb /= 2)
        if (tpb * d.k <= 32 && d.Tp % tpb == 0 && (long long)(d.T / tpb) * slices >= 1024) return tpb;
    return 1;
}

bool pack_counts(const Dims& d) {
    if (d.T == 0 || d.count_path == CountPath::kSeparate) return false;
    const int B = pick_block(d.row_units);
    const long long blocks = (long long)d.T * ((d.row_units + B - 1) / B);
    // every thread loads at most kMaxIdsPerThread ids, and the ids all workgroups
    // read together stay well below the payload (measured on gfx950: a win at
    // 128 tokens x top-8 with 256 workgroups and at 2048 tokens x top-2 with 1024
    // workgroups reading 4096 ids each)
    if (d.Na > (long long)kMaxIdsPerThread * B) return false;
    return d.count_path == CountPath::kFused || blocks * d.Na <= (1LL << 24);
}

bool token_affine(const Dims& d) {
    if (d.fp8 || d.T == 0) return false;   // FP8 dispatch rows and bf16 output rows have different slices
    if (d.layout == Layout::kRows) return false;
    if (d.layout == Layout::kAuto && d.Na * 2LL * d.H > kAffineBytes) return false;
    const int B = pick_block(d.row_units);
    const TokenGrid g = token_grid(d, (d.row_units + B - 1) / B, true);
    return ((long long)g.rounds << g.m_log2) * B < (1LL << 32);   // one grid dimension
}

TokenGrid token_grid(const Dims& d, int slices, bool per_assignment) {
    const int tpb = pack_counts(d) ? tokens_per_block(d) : 1;   // tokens per packing workgroup: 1, 2 or 4
    TokenGrid g;
    g.tpb_log2 = tpb == 4 ? 2 : tpb == 2 ? 1 : 0;
    g.groups = (d.T + tpb - 1) / tpb;
    g.slices = slices;
    g.m_log2 = 3;
    while ((1LL << g.m_log2) < (long long)g.groups * slices) ++g.m_log2;
    g.rounds = (per_assignment ? d.k : 1) << g.tpb_log2;
    return g;
}

hipError_t launch_pack(const Dims& d, const uint16_t* x, const int32_t* ids, const float* w, const Workspace& ws,
                       void* dst, float* dst_scales, bool direct, hipStream_t st) {
    if (d.T == 0) return hipSuccess;
    const int L = d.row_units;                 // 16-byte output units per dispatched row
    const int B = pick_block(L);
    const int slices = (L + B - 1) / B;
    HandleRecord* meta = reinterpret_cast<HandleRecord*>(direct ? ws.recv_meta : ws.send_meta);
    if (pack_counts(d)) {
        const int mi = ids_per_thread(d.Na, B);
        const int tpb = tokens_per_block(d);
        auto by_tpb = [&](auto fp8, auto dir, auto m) {
            constexpr bool F = decltype(fp8)::value, D = decltype(dir)::value;
            constexpr int MI = decltype(m)::value;
            return tpb == 4 ? count_pack_kernel<F, D, MI, 4> : tpb == 2 ? count_pack_kernel<F, D, MI, 2>
                                                                        : count_pack_kernel<F, D, MI, 1>;
        };
        auto pick = [&](auto fp8, auto dir) {
            return mi == 4    ? by_tpb(fp8, dir, std::integral_constant<int, 4>{})
                   : mi == 8  ? by_tpb(fp8, dir, std::integral_constant<int, 8>{})
                   : mi == 12 ? by_tpb(fp8, dir, std::integral_constant<int, 12>{})
                              : by_tpb(fp8, dir, std::integral_constant<int, 16>{});
        };
        using T_ = std::true_type;
        using F_ = std::false_type;
        auto kernel = d.fp8 ? (direct ? pick(T_{}, T_{}) : pick(T_{}, F_{})) : (direct ? pick(F_{}, T_{}) : pick(F_{}, F_{}));
        const size_t lds = count_pack_lds(d.E);
        const unsigned blocks = (unsigned)(d.P + (d.T + tpb - 1) / tpb);
        return launch_kernel(kernel, row_grid(blocks, slices), dim3(B), lds, st, reinterpret_cast<const uint4*>(x), ids,
                             w, d.T, d.Tp, d.E, d.k, L, slices, B, d.Ep, d.P, reinterpret_cast<uint4*>(dst), dst_scales,
                             meta, ws.send_to_recv, ws.recv_to_send, ws.send_pos, ws.recv_pos, ws.n);
    }
    const bool nt = streaming(d, 2LL * d.H * d.T + d.Na * (16LL * L + 4LL * d.scales));
    auto kernel = pack_kernel<false, false, false, false>;
    if (d.fp8) {
        if (direct) kernel = nt ? pack_kernel<true, true, false, true> : pack_kernel<true, false, false, true>;
        else kernel = nt ? pack_kernel<true, true, false, false> : pack_kernel<true, false, false, false>;
    } else {
        if (direct) kernel = nt ? pack_kernel<false, true, false, true> : pack_kernel<false, false, false, true>;
        else kernel = nt ? pack_kernel<false, true, false, false> : pack_kernel<false, false, false, false>;
    }
    return launch_kernel(kernel, row_grid(d.T, slices), dim3(B), 0, st, reinterpret_cast<const uint4*>(x), ids,
                         ws.bucket_rank, ws.send_off, ws.recv_off, d.Tp, d.E, d.k, L, slices, B, w, d.Ep,
                         reinterpret_cast<uint4*>(dst), dst_scales, meta, ws.send_to_recv, ws.recv_to_send, ws.send_pos,
                         ws.recv_pos);
}

hipError_t launch_pack_handles(const Dims& d, const int32_t* ids, const float* w, const Workspace& ws,
                               hipStream_t st) {
    if (d.T == 0) return hipSuccess;
    HandleRecord* meta = reinterpret_cast<HandleRecord*>(ws.recv_meta);
    if (pack_counts(d)) {
        const int B = pick_block(d.row_units);
        const int mi = ids_per_thread(d.Na, B);
        const int tpb = tokens_per_block(d);
        auto pick = [&](auto m) {
            constexpr int MI = decltype(m)::value;
            return tpb == 4 ? count_pack_kernel<false, true, MI, 4, false>
                 : tpb == 2 ? count_pack_kernel<false, true, MI, 2, false> : count_pack_kernel<false, true, MI, 1, false>;
        };
        auto kernel = mi == 4    ? pick(std::integral_constant<int, 4>{})
                      : mi == 8  ? pick(std::integral_constant<int, 8>{})
                      : mi == 12 ? pick(std::integral_constant<int, 12>{})
                                 : pick(std::integral_constant<int, 16>{});
        const size_t lds = count_pack_lds(d.E);
        const unsigned blocks = (unsigned)(d.P + (d.T + tpb - 1) / tpb);
        return launch_kernel(kernel, row_grid(blocks, 1), dim3(B), lds, st, static_cast<const uint4*>(nullptr), ids, w,
                             d.T, d.Tp, d.E, d.k, d.row_units, 1, B, d.Ep, d.P, static_cast<uint4*>(nullptr),
                             static_cast<float*>(nullptr), meta, ws.send_to_recv, ws.recv_to_send, ws.send_pos,
                             ws.recv_pos, ws.n);
    }
    const unsigned blocks = (unsigned)((d.Na + 255) / 256);
    return launch_kernel(handle_kernel, dim3(blocks), dim3(256), 0, st, ids, w, ws.bucket_rank, ws.send_off, ws.recv_off,
                  meta, ws.send_pos, ws.recv_pos, (int)d.Na, d.Tp, d.E, d.Ep, d.k);
}

hipError_t launch_allgather(const Dims& d, const uint16_t* x, void* gathered, float* gathered_scales, hipStream_t st) {
    if (d.T == 0) return hipSuccess;
    const int L = d.row_units;
    const int B = pick_block(L);
    const int slices = (L + B - 1) / B;
    const bool nt = streaming(d, 2LL * d.H * d.T + (long long)d.P * d.T * (16LL * L + 4LL * d.scales));
    auto kernel = d.fp8 ? (nt ? allgather_kernel<true, true, false> : allgather_kernel<true, false, false>)
                        : (nt ? allgather_kernel<false, true, false> : allgather_kernel<false, false, false>);
    return launch_kernel(kernel, row_grid(d.T, slices), dim3(B), 0, st, reinterpret_cast<const uint4*>(x),
                  reinterpret_cast<uint4*>(gathered), gathered_scales, d.T, d.P, L, slices);
}

}  // namespace moe
