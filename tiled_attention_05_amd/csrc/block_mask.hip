// Block-mask builder: classifies every (query tile, key tile) pair of a
// block_m x block_n tiling as empty / partial / full ("FlexAttention de
// PyTorch avec FlashAttention-4 change la donne", section "Limitations
// actuelles": block sparsity).
//
// One workgroup per (batch row, query tile). Each row i of the tile has one
// contiguous interval of allowed keys [lo_i, hi_i] (causal / window bounds
// intersected with the interval of its document, documents being contiguous),
// staged in LDS; a tile's allowed-pair count is the sum of the row intervals
// clipped to the tile's key range, so the classification is exact.
#include "common.h"
#include "fwd_params.h"

namespace attn {

constexpr int kBmMax = 4096;

__global__ void block_mask_clear(int32_t* flags) { *flags = 0; }

__global__ __launch_bounds__(256) void block_mask_kernel(int Nq, int Nk, int mask, int window,
                                                         const int32_t* doc, int bm, int bn,
                                                         int8_t* kinds, int32_t* counts,
                                                         int32_t* flags) {
    __shared__ int lo_s[kBmMax];
    __shared__ int hi_s[kBmMax];
    __shared__ int cnt_s[3];
    const int nqt = (Nq + bm - 1) / bm, nkt = (Nk + bn - 1) / bn;
    const int b = blockIdx.x / nqt, qt = blockIdx.x % nqt;
    const int i0 = qt * bm, rows = min(bm, Nq - i0);
    const int off = Nk - Nq;
    const int32_t* drow = doc ? doc + (size_t)b * Nk : nullptr;
    if (threadIdx.x < 3) cnt_s[threadIdx.x] = 0;

    for (int r = threadIdx.x; r < rows; r += blockDim.x) {
        const int i = i0 + r;
        int lo = 0, hi = Nk - 1;
        if (mask & kMaskCausal) hi = min(hi, i + off);
        if (mask & kMaskWindow) lo = max(lo, i + off - window + 1);
        if (drow) {
            const int x = drow[i];
            lo = max(lo, lower_bound_i32(drow, Nk, x));
            hi = min(hi, upper_bound_i32(drow, Nk, x) - 1);
            if (i + 1 < Nk && drow[i + 1] < x) atomicOr(flags, 1);
        }
        lo_s[r] = lo;
        hi_s[r] = hi;
    }
    __syncthreads();

    for (int kt = threadIdx.x; kt < nkt; kt += blockDim.x) {
        const int j0 = kt * bn, j1 = min(j0 + bn, Nk) - 1;
        long long n = 0;
        for (int r = 0; r < rows; ++r) {
            const int a = max(lo_s[r], j0), z = min(hi_s[r], j1);
            if (z >= a) n += z - a + 1;
        }
        const long long cells = (long long)rows * (j1 - j0 + 1);
        const int kind = n == 0 ? 0 : (n == cells ? 2 : 1);
        kinds[((size_t)b * nqt + qt) * nkt + kt] = (int8_t)kind;
        atomicAdd(&cnt_s[kind], 1);
    }
    __syncthreads();
    if (threadIdx.x < 3) counts[((size_t)b * nqt + qt) * 3 + threadIdx.x] = cnt_s[threadIdx.x];
}

hipError_t launch_block_mask(int B, int Nq, int Nk, int mask, int window, const int32_t* doc, int bm,
                             int bn, void* out, hipStream_t st) {
    const size_t nqt = (Nq + bm - 1) / bm, nkt = (Nk + bn - 1) / bn;
    const size_t kinds_bytes = (B * nqt * nkt + 15) / 16 * 16;
    int8_t* kinds = (int8_t*)out;
    int32_t* counts = (int32_t*)((char*)out + kinds_bytes);
    int32_t* flags = counts + B * nqt * 3;
    hipLaunchKernelGGL(block_mask_clear, dim3(1), dim3(1), 0, st, flags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(block_mask_kernel, dim3((unsigned)(B * nqt)), dim3(256), 0, st, Nq, Nk, mask,
                       window, doc, bm, bn, kinds, counts, flags);
    return hipGetLastError();
}

}  // namespace attn
