// Packed variable-length batches ("FlashAttention-3 : une attention plus
// rapide et plus precise ...", section "Optimisations restantes et
// integration future": variable-length sequences): sequence s owns tokens
// [cu[s], cu[s + 1]) of one packed sequence, and a token attends only within
// its own sequence -- the document mask of "FlexAttention de PyTorch avec
// FlashAttention-4 change la donne" (opening section) over the concatenation.
// This kernel writes the per-token sequence index that the forward's document
// path reads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// ids[t] = the largest s in [0, num_seqs] with cu[s] <= t (binary search over
// the num_seqs + 1 offsets). Non-decreasing in t for any cu.
__global__ __launch_bounds__(256) void seq_ids_kernel(const int32_t* __restrict__ cu, int num_seqs, int total,
                                                      int32_t* __restrict__ ids) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= total) return;
    int lo = 0, hi = num_seqs;   // answer in [lo, hi]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid;
        else hi = mid - 1;
    }
    ids[t] = lo;
}

hipError_t launch_seq_ids(const int32_t* cu, int num_seqs, int total, int32_t* ids, hipStream_t st) {
    hipLaunchKernelGGL(seq_ids_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, cu, num_seqs,
                       total, ids);
    return hipGetLastError();
}

}  // namespace attn
