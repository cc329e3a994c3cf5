// route.hip -- router softmax + top-k + renormalised weights on gfx950.
//
// Follows the router paragraph of "高效且便携的专家混合通信" (pplx-kernels): the
// router's probability distribution over experts, the top-k experts, and
// weights taken from that distribution; "Expert Parallel: MoE Token ..."
// section "Dispatch 前为什么必须 count 和 permute" fixes the output as
// [num_tokens, top_k] ids and weights.
//
// E > 32: one wavefront per token, lane l holding logits l, l+64, ... (V = E/64
// rounded up), loaded on consecutive addresses.  Each of the k rounds takes the
// wave maximum with DPP row operations (pairs, quads, half rows, rows, then
// row broadcasts; a few cycles each, no LDS traffic), then a ballot per slot v
// finds the lowest expert id holding that value, so equal logits pick the lower
// id; the winner is replaced by NaN, which the IEEE maximum ignores.  NaN logits
// rank below every number (-inf included) and tie with each other: a round
// whose maximum is NaN has only NaN logits left and takes the lowest id among
// the experts not yet chosen.
// E <= 32: a group of G lanes (the next power of two >= E) owns a token, 64/G
// tokens per wave, and each round is a group arg-max over 64-bit keys
// (order-preserving logit bits, with every NaN mapped below -inf, then the
// complemented expert id) by xor-butterfly shuffles.
// A row that holds a NaN logit gets NaN weights: its softmax normaliser is NaN.
// Softmax is strictly increasing, so selecting by logit is selecting by
// probability, and the renormalised weight p_j / sum_sel p equals
// exp(l_j - l_max) / sum_sel exp(l_i - l_max): the full partition function
// cancels.  Those k exponentials (evaluated together, one per lane, after the
// selection) and the slot-order sum run in double, so the fp32 weights are the
// correctly rounded ones up to a double ulp.  The ids and weights are written
// through (st_through_row): every workgroup of the counting pack reads all of
// them next, from every XCD (whole step at 128 tokens x top-8 x 7168 on gfx950:
// 28.30 -> 28.06 us, the router 4.04 -> 3.80 us).
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// Order-preserving key of a logit: -0 ranks equal to +0, every NaN ranks below
// -inf (whose key is 0x007FFFFF) and above the 0 that marks an expert taken or
// absent.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    if (f != f) return 0u;
    uint32_t b = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

template <int G, int V>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w, int T, int E, int k) {
    constexpr int kTokensPerWave = kWave / G;
    const int lane = threadIdx.x & (kWave - 1);
    const int gl = lane % G;
    const int wave = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int t = wave * kTokensPerWave + lane / G;
    const bool valid = t < T;

    uint64_t key[V];
    const float* row = logits + (size_t)(valid ? t : 0) * E;
    int nan_seen = 0;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int e = gl + G * v;
        key[v] = 0;   // below every real key
        if (valid && e < E) {
            const float l = row[e];
            nan_seen |= l != l;
            key[v] = ((uint64_t)ordered_bits(l) << 32) | (uint32_t)~(uint32_t)e;
        }
    }
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) nan_seen |= __shfl_xor(nan_seen, off, G);

    double my_l = 0.0;
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int v = 1; v < V; ++v) best = key[v] > best ? key[v] : best;
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) {
            const uint64_t o = __shfl_xor(best, off, G);
            best = o > best ? o : best;
        }
        const int id = (int)~(uint32_t)best;
        const double lv = (double)from_ordered_bits((uint32_t)(best >> 32));
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (gl + G * v == id) key[v] = 0;
        if (gl == j) { my_id = id; my_l = lv; }
    }
    // the k exponentials at once (lanes gl < k), then their sum in slot order
    const double m = __shfl(my_l, 0, G);
    const double my_e = gl < k ? exp(my_l - m) : 0.0;
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += __shfl(my_e, j, G);
    if (valid && gl < k) {   // the wave's tokens are consecutive: one row of kTokensPerWave * k entries
        const int i = (lane / G) * k + gl;
        st_through_row(ids, wave, kTokensPerWave * k, i, my_id);
        st_through_row(w, wave, kTokensPerWave * k, i, nan_seen ? __int_as_float(0x7FC00000) : (float)(my_e / sum));
    }
}

template <int Ctrl, int RowMask = 0xF>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), Ctrl, RowMask, 0xF, false));
}

// Maximum over the 64 lanes (IEEE maxNum: NaN lanes are ignored), in every lane.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));          // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp<0x4E>(v));          // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp<0x141>(v));         // row_half_mirror
    v = fmaxf(v, dpp<0x140>(v));         // row_mirror
    v = fmaxf(v, dpp<0x142, 0xA>(v));    // row_bcast15 into rows 1 and 3
    v = fmaxf(v, dpp<0x143, 0xC>(v));    // row_bcast31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

// Lane l's double, in every lane.
__device__ __forceinline__ double readlane_f64(double v, int l) {
    const long long b = __double_as_longlong(v);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)b, l);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(b >> 32), l);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

template <int V>
__global__ __launch_bounds__(256) void route_topk_wave_kernel(const float* __restrict__ logits,
                                                              int32_t* __restrict__ ids, float* __restrict__ w,
                                                              int T, int E, int k) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;                  // whole waves leave together
    const float nan = __int_as_float(0x7FC00000);
    float val[V];
    unsigned open = 0;                   // bit v: expert lane + 64 v exists and is not chosen yet
    bool nan_here = false;
    const float* row = logits + (size_t)t * E;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int e = lane + kWave * v;
        val[v] = e < E ? row[e] : nan;
        if (e < E) open |= 1u << v;
        nan_here |= e < E && val[v] != val[v];
    }
    const bool row_nan = __ballot(nan_here) != 0;   // the same in every lane
    float my_l = 0.0f;
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
        float lm = val[0];
#pragma unroll
        for (int v = 1; v < V; ++v) lm = fmaxf(lm, val[v]);
        const float M = wave_max(lm);
        int id = -1;                     // the lowest expert id holding M
        if (M == M) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const unsigned long long hit = __ballot(val[v] == M);
                if (id < 0 && hit) id = kWave * v + __ffsll((long long)hit) - 1;
            }
        } else {                         // only NaN logits are left: the lowest id not chosen yet
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const unsigned long long hit = __ballot((open >> v) & 1u);
                if (id < 0 && hit) id = kWave * v + __ffsll((long long)hit) - 1;
            }
        }
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (lane + kWave * v == id) {
                val[v] = nan;
                open &= ~(1u << v);
            }
        if (lane == j) { my_id = id; my_l = M; }
    }
    // the k exponentials at once (lanes < k), then their sum in slot order
    const double l0 = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_l), 0));
    const double my_e = lane < k ? exp((double)my_l - l0) : 0.0;
    double sum = 0.0;
    for (int j = 0; j < k; ++j) sum += readlane_f64(my_e, j);
    if (lane < k) {
        st_through_row(ids, t, k, lane, my_id);
        st_through_row(w, t, k, lane, row_nan ? nan : (float)(my_e / sum));
    }
}

template <int V>
hipError_t launch_rtw(const Dims& d, const float* logits, int32_t* ids, float* w, hipStream_t st) {
    // one wave (one token) per workgroup: at 128 tokens the tokens spread over 128
    // compute units instead of 32 (step 30.6 -> 30.2 us measured on gfx950; no
    // change at 8192 tokens)
    constexpr int kThreads = kWave;
    const int tokens_per_block = kThreads / kWave;
    const int blocks = (d.T + tokens_per_block - 1) / tokens_per_block;
    return launch_kernel((route_topk_wave_kernel<V>), dim3(blocks), dim3(kThreads), 0, st, logits, ids, w, d.T, d.E,
                       d.k);
}

template <int G, int V>
hipError_t launch_rt(const Dims& d, const float* logits, int32_t* ids, float* w, hipStream_t st) {
    constexpr int kThreads = 256;
    const int tokens_per_block = (kThreads / kWave) * (kWave / G);
    const int blocks = (d.T + tokens_per_block - 1) / tokens_per_block;
    return launch_kernel((route_topk_kernel<G, V>), dim3(blocks), dim3(kThreads), 0, st, logits, ids, w,
                       d.T, d.E, d.k);
}

}  // namespace

hipError_t launch_route_topk(const Dims& d, const float* logits, int32_t* ids, float* w, hipStream_t st) {
    if (d.T == 0) return hipSuccess;
    const int E = d.E;
    if (E <= 1) return launch_rt<1, 1>(d, logits, ids, w, st);
    if (E <= 2) return launch_rt<2, 1>(d, logits, ids, w, st);
    if (E <= 4) return launch_rt<4, 1>(d, logits, ids, w, st);
    if (E <= 8) return launch_rt<8, 1>(d, logits, ids, w, st);
    if (E <= 16) return launch_rt<16, 1>(d, logits, ids, w, st);
    if (E <= 32) return launch_rt<32, 1>(d, logits, ids, w, st);
    if (E <= 64) return launch_rtw<1>(d, logits, ids, w, st);
    if (E <= 128) return launch_rtw<2>(d, logits, ids, w, st);
    if (E <= 256) return launch_rtw<4>(d, logits, ids, w, st);
    if (E <= 512) return launch_rtw<8>(d, logits, ids, w, st);
    return launch_rtw<16>(d, logits, ids, w, st);
}

}  // namespace moe
