// Packed variable-length batches ("FlashAttention-3 : une attention plus
// rapide et plus precise ...", section "Optimisations restantes et
// integration future": variable-length sequences): sequence s owns tokens
// [cu[s], cu[s + 1]) of one packed sequence, and a token attends only within
// its own sequence -- the document mask of "FlexAttention de PyTorch avec
// FlashAttention-4 change la donne" (opening section) over the concatenation.
// seq_ids_kernel writes the per-token sequence index that the forward's
// document path reads; varlen_tiles_kernel the per-sequence tile list of the
// bf16 path.
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

// Per-sequence tiling of a packed batch for the bf16 forward: one list entry
// per (sequence s, query tile t of bm rows), the entry being the tile's first
// packed row cu[s] + t bm. Order: sequences by tile count, descending (ties:
// lower index first), and within a sequence its tiles from the last (the
// heaviest: it attends to the most keys) to the first. The tiles in flight at
// once then come from one or two sequences and share their keys and values in
// the L2 of each XCD, and the grid ends on the light tiles of the shortest
// sequences. Entries past the tile count are -1. One workgroup; n_seq <=
// kVarlenMaxSeqs (the caller checks it); tile counts are cut at
// kVarlenMaxTiles, and no write leaves the n_list entries.
constexpr int kVarlenMaxSeqs = 4096, kVarlenMaxTiles = 4096;

__global__ __launch_bounds__(1024) void varlen_tiles_kernel(const int32_t* __restrict__ cu, int n_seq, int bm,
                                                            int32_t* __restrict__ items, int n_list) {
    __shared__ int nt[kVarlenMaxSeqs];    // tiles of sequence s
    __shared__ int rk[kVarlenMaxSeqs];    // rank of s by tile count, descending
    __shared__ int at[kVarlenMaxSeqs];    // tiles of the sequence of rank r, then its first list entry
    __shared__ int part[1024];
    const int tid = threadIdx.x;
    for (int s = tid; s < n_seq; s += 1024)
        nt[s] = min((max(cu[s + 1] - cu[s], 0) + bm - 1) / bm, kVarlenMaxTiles);
    for (int r = tid; r < kVarlenMaxSeqs; r += 1024) at[r] = 0;
    __syncthreads();
    for (int s = tid; s < n_seq; s += 1024) {
        const int n = nt[s];
        int r = 0;
        for (int c = 0; c < n_seq; ++c) r += (nt[c] > n || (nt[c] == n && c < s)) ? 1 : 0;
        rk[s] = r;
        at[r] = n;   // ranks are a permutation of 0 .. n_seq - 1
    }
    __syncthreads();
    // first entry of rank r: exclusive scan of the tile counts in rank order
    constexpr int PER = kVarlenMaxSeqs / 1024;
    int a[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        a[i] = at[PER * tid + i];
        sum += a[i];
    }
    part[tid] = sum;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int x = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += x;
        __syncthreads();
    }
    int run = part[tid] - sum;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        at[PER * tid + i] = run;
        run += a[i];
    }
    const int n_tiles = part[1023];
    __syncthreads();
    for (int s = tid; s < n_seq; s += 1024) {
        const int first = at[rk[s]], n = nt[s];
        for (int t = 0; t < n; ++t) {
            const int e = first + (n - 1 - t);
            if (e < n_list) items[e] = cu[s] + t * bm;
        }
    }
    for (int i = n_tiles + tid; i < n_list; i += 1024) items[i] = -1;
}

hipError_t launch_varlen_tiles(const int32_t* cu, int n_seq, int bm, int32_t* items, int n_list, hipStream_t st) {
    if (n_seq < 1 || n_seq > kVarlenMaxSeqs || bm < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(varlen_tiles_kernel, dim3(1), dim3(1024), 0, st, cu, n_seq, bm, items, n_list);
    return hipGetLastError();
}

}  // namespace attn
