// count.hip -- per-(source rank, expert) counts, the count matrix, prefix-sum
// offsets and the stable rank of every assignment inside its bucket.
//
// Follows "Expert Parallel: MoE Token 为什么要两次穿过 GPU 网络", sections
// "Dispatch 前为什么必须 count 和 permute" (count per destination, exclusive
// prefix sum into send offsets) and "All-to-All-v 才接近真实通信形状" (count
// matrix C_ij, source i -> destination j), and "[Infra-10] All-to-All
// Optimization" 3.5 (histogram -> prefix sum -> scatter).
//
// count kernel: one workgroup per source rank s.  Its T/P tokens are taken in
// chunks of 32*W tokens; per chunk an LDS bitmap [E][W] words gets bit i of
// expert e set when local token i picked e (ds_or).  A token picks an expert at
// most once, so the stable rank of (token i, expert e) inside bucket (s, e) is
// the number of set bits below i: carried count of earlier chunks + exclusive
// prefix of the word popcounts (a segmented wave scan over the W words of each
// expert) + popcount of the bits below i in i's word.  Positions come out in
// token order without sorting, whatever the atomic order was.  At the end the
// counts n[s][e], the send offsets s*(T/P)*k + sum_{e'<e} n[s][e'] (block scan)
// and the row C[s][.] are written.
//
// scan kernel: one workgroup; thread e sums n[.][e] into N[e], a block scan
// gives expert_off, a walk over the source ranks gives recv_off[e][s], and
// rank r's receive region starts at expert_off[r * E/P].
#include "device.hpp"
#include "kernels.hpp"

namespace moe {

int count_words_per_expert(int E, int Tp) {
    // bitmap + prefix: 2 * E * W words of LDS, kept within 48 KiB; W is a power
    // of two <= 64 (a segment of the wave scan) and no larger than the rank needs
    int need = (Tp + 31) / 32;
    int W = 1;
    while (W < 64 && W < need && 2 * (size_t)E * (2 * W) * 4 + (size_t)E * 4 <= 48 * 1024) W *= 2;
    return W;
}

size_t count_lds_bytes(int E, int W) { return (2 * (size_t)E * W + (size_t)E + 32) * 4; }

namespace {

constexpr int kCountThreads = 1024;

__global__ __launch_bounds__(kCountThreads) void count_kernel(const int32_t* __restrict__ ids, int Tp, int E,
                                                              int Ep, int k, int P, int W,
                                                              int32_t* __restrict__ n_out,
                                                              int32_t* __restrict__ send_off,
                                                              int32_t* __restrict__ C,
                                                              int32_t* __restrict__ bucket_rank) {
    extern __shared__ uint32_t lds[];
    uint32_t* bitmap = lds;                                   // [E][W]
    int32_t* prefix = reinterpret_cast<int32_t*>(lds + (size_t)E * W);  // [E][W]
    int32_t* carry = prefix + (size_t)E * W;                  // [E]
    int32_t* tmp = carry + E;                                 // scan scratch (<= 17 ints)

    const int s = blockIdx.x;
    const int tid = threadIdx.x, bs = blockDim.x;
    const int EW = E * W;
    const int chunk = 32 * W;
    const int32_t* rank_ids = ids + (size_t)s * Tp * k;
    int32_t* rank_br = bucket_rank + (size_t)s * Tp * k;

    for (int e = tid; e < E; e += bs) carry[e] = 0;
    for (int c0 = 0; c0 < Tp; c0 += chunk) {
        const int ct = min(chunk, Tp - c0);
        for (int x = tid; x < EW; x += bs) bitmap[x] = 0;
        __syncthreads();
        for (int a = tid; a < ct * k; a += bs) {
            const int i = a / k;
            const int e = rank_ids[(size_t)c0 * k + a];
            atomicOr(&bitmap[e * W + (i >> 5)], 1u << (i & 31));
        }
        __syncthreads();
        // exclusive scan of popcounts over each expert's W words; EW is a multiple
        // of W and bs of 64, so a segment never straddles a wave or a pass
        for (int x = tid; x < EW; x += bs) {
            const int wv = x & (W - 1);
            const int v = __popc(bitmap[x]);
            int incl = v;
            for (int d = 1; d < W; d <<= 1) {
                const int o = __shfl_up(incl, d, W);
                if (wv >= d) incl += o;
            }
            prefix[x] = incl - v;
        }
        __syncthreads();
        for (int a = tid; a < ct * k; a += bs) {
            const int i = a / k;
            const int e = rank_ids[(size_t)c0 * k + a];
            const int wd = i >> 5;
            const uint32_t below = bitmap[e * W + wd] & ((1u << (i & 31)) - 1u);
            rank_br[(size_t)c0 * k + a] = carry[e] + prefix[e * W + wd] + __popc(below);
        }
        __syncthreads();
        for (int e = tid; e < E; e += bs)
            carry[e] += prefix[e * W + W - 1] + __popc(bitmap[e * W + W - 1]);
        __syncthreads();
    }

    // counts, send offsets (bucket (s, e) starts after rank s's buckets of lower
    // experts); E <= blockDim.x, one expert per thread
    {
        const int c = tid < E ? carry[tid] : 0;
        int total = 0;
        const int ex = block_exclusive_scan(c, tmp, &total);
        if (tid < E) {
            n_out[(size_t)s * E + tid] = c;
            send_off[(size_t)s * E + tid] = s * Tp * k + ex;
        }
    }
    for (int r = tid; r < P; r += bs) {
        int c = 0;
        for (int e = r * Ep; e < (r + 1) * Ep; ++e) c += carry[e];
        C[(size_t)s * P + r] = c;
    }
}

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ n, int P, int E, int Ep,
                                                            int32_t* __restrict__ N,
                                                            int32_t* __restrict__ expert_off,
                                                            int32_t* __restrict__ recv_off,
                                                            int32_t* __restrict__ rank_recv_off) {
    __shared__ int32_t off[1025];
    __shared__ int32_t tmp[32];
    const int e = threadIdx.x;      // E <= 1024 == blockDim.x
    int tot = 0;
    if (e < E)
        for (int s = 0; s < P; ++s) tot += n[(size_t)s * E + e];
    int total = 0;
    const int ex = block_exclusive_scan(tot, tmp, &total);
    if (e < E) {
        N[e] = tot;
        expert_off[e] = ex;
        off[e] = ex;
        int acc = ex;
        for (int s = 0; s < P; ++s) {
            recv_off[(size_t)e * P + s] = acc;
            acc += n[(size_t)s * E + e];
        }
    }
    if (e == 0) {
        expert_off[E] = total;
        off[E] = total;
    }
    __syncthreads();
    for (int r = threadIdx.x; r <= P; r += blockDim.x) rank_recv_off[r] = off[r * Ep];
}

}  // namespace

hipError_t launch_count(const Dims& d, const int32_t* ids, const Workspace& ws, hipStream_t st) {
    const int W = count_words_per_expert(d.E, d.Tp);
    const size_t lds = count_lds_bytes(d.E, W);
    hipLaunchKernelGGL(count_kernel, dim3(d.P), dim3(kCountThreads), lds, st, ids, d.Tp, d.E, d.Ep, d.k, d.P, W,
                       ws.n, ws.send_off, ws.C, ws.bucket_rank);
    return hipGetLastError();
}

hipError_t launch_scan(const Dims& d, const Workspace& ws, hipStream_t st) {
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, st, ws.n, d.P, d.E, d.Ep, ws.N,
                       ws.expert_off, ws.recv_off, ws.rank_recv_off);
    return hipGetLastError();
}

}  // namespace moe
