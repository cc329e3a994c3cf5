// validate.hip -- the debug check of the routing input.  Expert ids outside
// [0, E) or repeated within one token's k slots are outside the dispatch
// contract: the fast path neither detects nor survives them, so under the
// library's debug mode dispatch runs this check first and refuses such input
// before any payload kernel is launched.  One workgroup walks every token,
// checking its k ids for range and pairwise distinctness, and writes the number
// of offending assignments to one workspace word (a plain store, so nothing
// needs clearing first).
#include "device.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void validate_ids_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                           int32_t* __restrict__ bad_out) {
    __shared__ int32_t tmp[17];
    int bad = 0;
    for (int t = threadIdx.x; t < T; t += blockDim.x) {
        const int32_t* row = ids + (size_t)t * k;
        for (int j = 0; j < k; ++j) {
            const int e = row[j];
            bool ok = (unsigned)e < (unsigned)E;
            for (int i = 0; i < j && ok; ++i) ok = row[i] != e;
            bad += ok ? 0 : 1;
        }
    }
    int total = 0;
    block_exclusive_scan(bad, tmp, &total);
    if (threadIdx.x == 0) *bad_out = total;
}

}  // namespace

hipError_t launch_validate_ids(const Dims& d, const int32_t* ids, int32_t* bad_out, hipStream_t st) {
    return launch_kernel(validate_ids_kernel, dim3(1), dim3(256), 0, st, ids, d.T, d.E, d.k, bad_out);
}

}  // namespace moe
