// count.hip -- per-(source rank, expert) counts, the count matrix, prefix-sum
// offsets and the stable rank of every assignment inside its bucket.
//
// Follows "Expert Parallel: MoE Token 为什么要两次穿过 GPU 网络", sections
// "Dispatch 前为什么必须 count 和 permute" (count per destination, exclusive
// prefix sum into send offsets) and "All-to-All-v 才接近真实通信形状" (count
// matrix C_ij, source i -> destination j), and "[Infra-10] All-to-All
// Optimization" 3.5 (histogram -> prefix sum -> scatter).
//
// Stable ranks without sorting: a token picks an expert at most once, so the
// rank of (local token i, expert e) inside bucket (s, e) is the number of
// earlier tokens of rank s that picked e.  An LDS bitmap [E][W] words gets
// bit i of expert e set (ds_or, any order); the rank is then the exclusive
// prefix of the word popcounts (a segmented wave scan over each expert's W
// words) plus the popcount of the bits below i in i's own word.
//
// Two shapes of the same computation:
//  - count_scan_single: one workgroup does every rank, the cross-rank scan and
//    all offsets, for problems whose bitmaps fit in LDS at once (decode-sized
//    batches).  No workgroup ever waits for another, and there is one launch.
//  - count (one workgroup per source rank, its tokens in chunks of 32*W) then
//    scan (one workgroup: N[e] = sum_s n[s][e], the exclusive scan expert_off,
//    recv_off[s][e] = expert_off[e] + sum_{s'<s} n[s'][e], and rank r's receive
//    region start expert_off[r * E/P]).  The scan spreads the P x E counts over
//    the whole block, a few ranks of one expert per thread, all loaded at once
//    (32 ranks x 256 experts on gfx950: 8.3 -> 3.9 us against a thread per
//    expert walking all P ranks); where a thread would need more than
//    kMaxPerThread ranks, the counts are staged in LDS with one burst of
//    coalesced loads and a thread per expert walks them.
// Global loads are issued all at once into registers before they are used: a
// loop with a load per iteration pays one memory round trip per iteration.
// Device-scope fences between workgroups are avoided on purpose: on gfx950 each
// one writes back and invalidates the whole L2 of the XCD.
#include "device.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr size_t kLdsBudget = 64 * 1024;
constexpr int kMaxPerThread = 16;   // assignments (or counts) a thread preloads

// W: words of the per-expert bitmap chunk, a power of two <= 64 (one segment of
// the wave scan), no larger than the rank needs, bitmap + prefix within budget.
int words_per_expert(long long rows, int Tp, size_t budget) {
    const int need = (Tp + 31) / 32;
    int W = 1;
    while (W < 64 && W < need && 2 * (size_t)rows * (2 * W) * 4 <= budget) W *= 2;
    return W;
}

// Exclusive prefix of popcounts over each segment of W consecutive words
// (W | 64, so a segment never straddles a wave); every thread of the block calls it.
__device__ void segmented_word_prefix(const uint32_t* bitmap, int32_t* prefix, int n, int W) {
    for (int x0 = 0; x0 < n; x0 += blockDim.x) {
        const int x = x0 + threadIdx.x;
        const int v = x < n ? __popc(bitmap[x]) : 0;
        const int wv = x & (W - 1);
        int incl = v;
        for (int d = 1; d < W; d <<= 1) {
            const int o = __shfl_up(incl, d, W);
            if (wv >= d) incl += o;
        }
        if (x < n) prefix[x] = incl - v;
    }
}

__device__ __forceinline__ int bucket_rank_of(const uint32_t* bitmap, const int32_t* prefix, int row, int W,
                                              int i) {
    const int wd = i >> 5;
    const uint32_t below = bitmap[row * W + wd] & ((1u << (i & 31)) - 1u);
    return prefix[row * W + wd] + __popc(below);
}

__device__ __forceinline__ int word_total(const uint32_t* bitmap, const int32_t* prefix, int row, int W) {
    return prefix[row * W + W - 1] + __popc(bitmap[row * W + W - 1]);
}

// ---- one workgroup per source rank ----------------------------------------------

__global__ __launch_bounds__(kThreads) void count_kernel(const int32_t* __restrict__ ids, int Tp, int E, int Ep,
                                                         int k, int P, int W, int32_t* __restrict__ n_out,
                                                         int32_t* __restrict__ send_off, int32_t* __restrict__ C,
                                                         int32_t* __restrict__ bucket_rank) {
    extern __shared__ uint32_t lds[];
    uint32_t* bitmap = lds;                                               // [E][W]
    int32_t* prefix = reinterpret_cast<int32_t*>(lds + (size_t)E * W);   // [E][W]
    int32_t* carry = prefix + (size_t)E * W;                              // [E]
    __shared__ int32_t tmp[32];

    const int s = blockIdx.x;
    const int tid = threadIdx.x, bs = blockDim.x;
    const int EW = E * W;
    const int chunk = 32 * W;
    const int32_t* rank_ids = ids + (size_t)s * Tp * k;
    int32_t* rank_br = bucket_rank + (size_t)s * Tp * k;

    for (int e = tid; e < E; e += bs) carry[e] = 0;
    for (int c0 = 0; c0 < Tp; c0 += chunk) {
        const int ct = min(chunk, Tp - c0);
        const int na = ct * k;            // <= kMaxPerThread * bs by the choice of W
        int myid[kMaxPerThread];
#pragma unroll
        for (int j = 0; j < kMaxPerThread; ++j) {
            const int a = tid + j * bs;
            myid[j] = a < na ? rank_ids[(size_t)c0 * k + a] : 0;
        }
        for (int x = tid; x < EW; x += bs) bitmap[x] = 0;
        lds_barrier();
#pragma unroll
        for (int j = 0; j < kMaxPerThread; ++j) {
            const int a = tid + j * bs;
            if (a < na) atomicOr(&bitmap[myid[j] * W + ((a / k) >> 5)], 1u << ((a / k) & 31));
        }
        lds_barrier();
        segmented_word_prefix(bitmap, prefix, EW, W);
        lds_barrier();
#pragma unroll
        for (int j = 0; j < kMaxPerThread; ++j) {
            const int a = tid + j * bs;
            if (a < na) rank_br[(size_t)c0 * k + a] = carry[myid[j]] + bucket_rank_of(bitmap, prefix, myid[j], W, a / k);
        }
        lds_barrier();
        for (int e = tid; e < E; e += bs) carry[e] += word_total(bitmap, prefix, e, W);
        lds_barrier();
    }

    // counts and send offsets: bucket (s, e) follows rank s's buckets of lower
    // experts; E <= blockDim.x, one expert per thread
    const int c = tid < E ? carry[tid] : 0;
    const int ex = block_exclusive_scan(c, tmp, nullptr);
    if (tid < E) {
        n_out[(size_t)s * E + tid] = c;
        send_off[(size_t)s * E + tid] = s * Tp * k + ex;
    }
    for (int r = tid; r < P; r += bs) {
        int cr = 0;
        for (int e = r * Ep; e < (r + 1) * Ep; ++e) cr += carry[e];
        C[(size_t)s * P + r] = cr;
    }
}

// Cross-rank scan from the counts n (global, or LDS when staged); one expert per thread.
__device__ void cross_rank_scan(const int32_t* n, int P, int E, int Ep, int32_t* off /* LDS [E+1] */,
                                int32_t* tmp, int32_t* __restrict__ N, int32_t* __restrict__ expert_off,
                                int32_t* __restrict__ recv_off, int32_t* __restrict__ rank_recv_off) {
    const int e = threadIdx.x;
    int tot = 0;
    if (e < E)
        for (int r = 0; r < P; ++r) tot += n[(size_t)r * E + e];
    int total = 0;
    const int ex = block_exclusive_scan(tot, tmp, &total);
    if (e < E) {
        N[e] = tot;
        expert_off[e] = ex;
        off[e] = ex;
        int acc = ex;
        for (int r = 0; r < P; ++r) {
            recv_off[(size_t)r * E + e] = acc;     // source-major: coalesced over e
            acc += n[(size_t)r * E + e];
        }
    }
    if (threadIdx.x == 0) {
        expert_off[E] = total;
        off[E] = total;
    }
    lds_barrier();
    for (int r = threadIdx.x; r <= P; r += blockDim.x) rank_recv_off[r] = off[r * Ep];
}

__global__ __launch_bounds__(kThreads) void scan_kernel(const int32_t* __restrict__ n, int P, int E, int Ep,
                                                        int stage, int32_t* __restrict__ N,
                                                        int32_t* __restrict__ expert_off,
                                                        int32_t* __restrict__ recv_off,
                                                        int32_t* __restrict__ rank_recv_off) {
    extern __shared__ int32_t slds[];
    __shared__ int32_t tmp[32];
    int32_t* off = slds;                 // [E+1]
    const int32_t* src = n;
    if (stage) {                         // one burst of coalesced loads instead of 2P serial ones
        int32_t* nl = slds + E + 1;
        const int total = P * E;
        for (int x0 = 0; x0 < total; x0 += kMaxPerThread * blockDim.x) {
            int v[kMaxPerThread];
#pragma unroll
            for (int j = 0; j < kMaxPerThread; ++j) {
                const int x = x0 + j * blockDim.x + threadIdx.x;
                v[j] = x < total ? n[x] : 0;
            }
#pragma unroll
            for (int j = 0; j < kMaxPerThread; ++j) {
                const int x = x0 + j * blockDim.x + threadIdx.x;
                if (x < total) nl[x] = v[j];
            }
        }
        lds_barrier();
        src = nl;
    }
    cross_rank_scan(src, P, E, Ep, off, tmp, N, expert_off, recv_off, rank_recv_off);
}

// The same cross-rank scan with the P x E counts spread over the whole block:
// thread (g, e) = (tid / E, tid mod E) holds ranks g*R .. g*R + R - 1 of expert e
// (R ranks per group, ceil(P / R) groups), so every count loads at once into
// registers and no thread walks all P ranks: the per-group sums of each expert
// meet in LDS, one block scan over the experts gives expert_off, each group's
// start follows from the sums of the groups before it, and each thread writes
// recv_off for its own ranks.  Used when R <= kMaxPerThread (the launcher's
// choice); the staged form above takes the rest.
__global__ __launch_bounds__(kThreads) void scan_spread_kernel(const int32_t* __restrict__ n, int P, int E, int Ep,
                                                               int R, int32_t* __restrict__ N,
                                                               int32_t* __restrict__ expert_off,
                                                               int32_t* __restrict__ recv_off,
                                                               int32_t* __restrict__ rank_recv_off) {
    extern __shared__ int32_t slds[];
    __shared__ int32_t tmp[32];
    const int tid = threadIdx.x;
    const int groups = (P + R - 1) / R;
    int32_t* part = slds;                        // [groups][E]: group sums, then group starts
    int32_t* off = slds + groups * E;            // [E+1]
    const int g = tid / E, e = tid - g * E;
    const bool active = g < groups;
    int v[kMaxPerThread];
#pragma unroll
    for (int i = 0; i < kMaxPerThread; ++i) {
        const int r = g * R + i;
        v[i] = active && i < R && r < P ? n[(size_t)r * E + e] : 0;
    }
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kMaxPerThread; ++i) sum += v[i];
    if (active) part[g * E + e] = sum;
    lds_barrier();
    int tot = 0;
    if (tid < E)
        for (int h = 0; h < groups; ++h) tot += part[h * E + tid];
    int total = 0;
    const int ex = block_exclusive_scan(tot, tmp, &total);   // every thread; barriers inside
    if (tid < E) {
        N[tid] = tot;
        expert_off[tid] = ex;
        off[tid] = ex;
        int acc = ex;                            // column tid: group sums -> group starts
        for (int h = 0; h < groups; ++h) {
            const int p = part[h * E + tid];
            part[h * E + tid] = acc;
            acc += p;
        }
    }
    if (tid == 0) {
        expert_off[E] = total;
        off[E] = total;
    }
    lds_barrier();
    if (active) {
        int acc = part[g * E + e];
#pragma unroll
        for (int i = 0; i < kMaxPerThread; ++i) {
            const int r = g * R + i;
            if (i < R && r < P) {
                recv_off[(size_t)r * E + e] = acc;   // coalesced over e
                acc += v[i];
            }
        }
    }
    for (int r = tid; r <= P; r += blockDim.x) rank_recv_off[r] = off[r * Ep];
}

// ---- one workgroup for everything (small problems) --------------------------------

__global__ __launch_bounds__(kThreads) void count_scan_single_kernel(
    const int32_t* __restrict__ ids, int Tp, int E, int Ep, int k, int P, int W, int32_t* __restrict__ n_out,
    int32_t* __restrict__ send_off, int32_t* __restrict__ C, int32_t* __restrict__ bucket_rank,
    int32_t* __restrict__ N, int32_t* __restrict__ expert_off, int32_t* __restrict__ recv_off,
    int32_t* __restrict__ rank_recv_off) {
    extern __shared__ uint32_t lds[];
    const int PE = P * E;
    uint32_t* bitmap = lds;                                               // [P*E][W]
    int32_t* prefix = reinterpret_cast<int32_t*>(lds + (size_t)PE * W);  // [P*E][W]
    int32_t* nl = prefix + (size_t)PE * W;                                // [P][E]
    int32_t* off = nl + PE;                                               // [E+1]
    __shared__ int32_t tmp[32];
    const int tid = threadIdx.x, bs = blockDim.x;
    const int T = P * Tp;

    const int Na = T * k;
    int myid[kMaxPerThread];             // this thread's assignments a = tid + j * bs
#pragma unroll
    for (int j = 0; j < kMaxPerThread; ++j) {
        const int a = tid + j * bs;
        myid[j] = a < Na ? ids[a] : 0;
    }
    for (int x = tid; x < PE * W; x += bs) bitmap[x] = 0;
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kMaxPerThread; ++j) {
        const int a = tid + j * bs;
        if (a < Na) {
            const int t = a / k;
            const int s = t / Tp, i = t - s * Tp;
            atomicOr(&bitmap[(s * E + myid[j]) * W + (i >> 5)], 1u << (i & 31));
        }
    }
    lds_barrier();
    if (W > 1) {
        segmented_word_prefix(bitmap, prefix, PE * W, W);
        lds_barrier();
    } else {
        for (int x = tid; x < PE; x += bs) prefix[x] = 0;
    }
    for (int x = tid; x < PE; x += bs) {
        const int c = W > 1 ? word_total(bitmap, prefix, x, W) : __popc(bitmap[x]);
        nl[x] = c;
        n_out[x] = c;
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kMaxPerThread; ++j) {
        const int a = tid + j * bs;
        if (a < Na) {
            const int t = a / k;
            const int s = t / Tp, i = t - s * Tp;
            bucket_rank[a] = bucket_rank_of(bitmap, prefix, s * E + myid[j], W, i);
        }
    }
    // send offsets: one wave per source rank scans its E counts in chunks of 64
    {
        const int lane = tid & (kWave - 1), wave = tid / kWave, nw = bs / kWave;
        for (int s = wave; s < P; s += nw) {
            int carry = s * Tp * k;
            for (int e0 = 0; e0 < E; e0 += kWave) {
                const int e = e0 + lane;
                const int c = e < E ? nl[s * E + e] : 0;
                const int incl = wave_inclusive_scan(c);
                if (e < E) send_off[(size_t)s * E + e] = carry + incl - c;
                carry += __builtin_amdgcn_readlane(incl, kWave - 1);
            }
        }
    }
    for (int x = tid; x < P * P; x += bs) {
        const int s = x / P, r = x - s * P;
        int cr = 0;
        for (int e = r * Ep; e < (r + 1) * Ep; ++e) cr += nl[s * E + e];
        C[x] = cr;
    }
    cross_rank_scan(nl, P, E, Ep, off, tmp, N, expert_off, recv_off, rank_recv_off);
}

size_t single_lds_bytes(int P, int E, int W) { return ((size_t)P * E * (2 * W + 1) + E + 1) * 4; }

int single_words(const Dims& d) { return words_per_expert((long long)d.P * d.E, d.Tp, kLdsBudget); }

}  // namespace

bool count_is_single(const Dims& d) {
    // one workgroup handles at most kMaxPerThread assignments per thread, its LDS in budget
    if ((long long)d.T * d.k > (long long)kMaxPerThread * kThreads) return false;
    const int W = single_words(d);
    if (32 * W < d.Tp) return false;
    return single_lds_bytes(d.P, d.E, W) <= kLdsBudget;
}

hipError_t launch_count(const Dims& d, const int32_t* ids, const Workspace& ws, hipStream_t st) {
    if (count_is_single(d)) {
        const int W = single_words(d);
        return launch_kernel(count_scan_single_kernel, dim3(1), dim3(kThreads), single_lds_bytes(d.P, d.E, W), st, ids,
                           d.Tp, d.E, d.Ep, d.k, d.P, W, ws.n, ws.send_off, ws.C, ws.bucket_rank, ws.N,
                           ws.expert_off, ws.recv_off, ws.rank_recv_off);
    }
    int W = words_per_expert(d.E, d.Tp, 48 * 1024);
    while (W > 1 && 32LL * W * d.k > (long long)kMaxPerThread * kThreads) W /= 2;
    const size_t lds = (2 * (size_t)d.E * W + d.E) * 4;
    return launch_kernel(count_kernel, dim3(d.P), dim3(kThreads), lds, st, ids, d.Tp, d.E, d.Ep, d.k, d.P, W, ws.n,
                       ws.send_off, ws.C, ws.bucket_rank);
}

hipError_t launch_scan(const Dims& d, const Workspace& ws, hipStream_t st) {
    // spread form: ranks per thread group R = ceil(P / G) with G = kThreads / E groups
    const int G = kThreads / d.E;
    const int R = G > 0 ? (d.P + G - 1) / G : 0;
    if (G > 0 && R <= kMaxPerThread) {
        const int groups = (d.P + R - 1) / R;
        const size_t lds = ((size_t)groups * d.E + d.E + 1) * 4;
        return launch_kernel(scan_spread_kernel, dim3(1), dim3(kThreads), lds, st, ws.n, d.P, d.E, d.Ep, R, ws.N,
                             ws.expert_off, ws.recv_off, ws.rank_recv_off);
    }
    const bool stage = ((size_t)d.P * d.E + d.E + 1) * 4 <= kLdsBudget;
    const size_t lds = stage ? ((size_t)d.P * d.E + d.E + 1) * 4 : ((size_t)d.E + 1) * 4;
    return launch_kernel(scan_kernel, dim3(1), dim3(kThreads), lds, st, ws.n, d.P, d.E, d.Ep, stage ? 1 : 0, ws.N,
                       ws.expert_off, ws.recv_off, ws.rank_recv_off);
}

}  // namespace moe
