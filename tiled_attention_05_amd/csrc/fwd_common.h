// Pieces shared by the forward kernels: key-tile geometry and LDS swizzles,
// the wave-parallel search over document ids, and the K/V tile copy.
#pragma once
#include <climits>

#include "common.h"
#include "fwd_params.h"

namespace attn {

constexpr int BN = 64;   // keys per tile

template <int D>
struct Tile {
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int CPR = D / 8;          // 16-byte chunks per row
    static constexpr int RPB = 16 / CPR;       // rows sharing one 256-byte bank window
    static constexpr int BYTES = BN * ROW_BYTES;
    // K tile: 16-byte reads of 32 rows at one chunk column must hit distinct
    // banks within every 16 lanes -> XOR the chunk index with the row.
    static __device__ __forceinline__ int swz_k(int r) { return (r / RPB) % CPR; }
    // V tile: transposed 8-byte reads touch 4 rows x 64 bytes per 32 lanes ->
    // rotate 64-byte groups by the row.
    static __device__ __forceinline__ int swz_v(int r) { return 4 * ((r / RPB) % (CPR / 4)); }
};

// Wave-parallel search over a non-decreasing int array: first j in [0, n)
// with a[j] >= x (STRICT = false) or a[j] > x (STRICT = true); n if none.
// Each step probes 64 evenly spaced entries, so n = 32768 needs 3 loads.
template <bool STRICT>
__device__ int wave_search(const int32_t* a, int n, int x, int lane) {
    int lo = 0, hi = n;   // answer in [lo, hi]
    while (hi - lo > 64) {
        const int step = (hi - lo + 63) / 64;
        const int j = lo + lane * step;
        bool hit = true;
        if (j < hi) hit = STRICT ? (a[j] > x) : (a[j] >= x);
        const uint64_t bal = __ballot(hit);
        const int first = bal ? __builtin_ctzll(bal) : 64;
        const int nlo = first > 0 ? lo + (first - 1) * step + 1 : lo;
        const int nhi = first < 64 ? min(hi, lo + first * step) : hi;
        lo = nlo;
        hi = nhi;
    }
    const int j = lo + lane;
    bool hit = true;
    if (j < hi) hit = STRICT ? (a[j] > x) : (a[j] >= x);
    const uint64_t bal = __ballot(hit);
    return bal ? min(hi, lo + __builtin_ctzll(bal)) : hi;
}

// Keys a block of query rows [r0, r1] (inclusive, r1 < Nq) may attend to: one
// contiguous range [lo, hi), the union of the rows' allowed keys (causal: up
// to r1 + off; window: from r0 + off - W + 1; documents: from the first key of
// the first row's document to the last key of the last row's document, ids
// being non-decreasing). Every key of the range is allowed for some row of
// the block, so a key tile that meets the range is not empty. An empty range
// comes back as lo = INT_MAX, hi = INT_MIN. dq0 / dq1: the document ids of
// rows r0 and r1 (0 without documents). Called by a whole wave (the document
// search is wave-parallel).
struct KeyRange {
    int lo, hi, dq0, dq1;
};
template <bool DOC>
__device__ __forceinline__ KeyRange rows_key_range(int r0, int r1, int Nk, int off, int mask, int W,
                                                   const int32_t* docrow, int lane) {
    KeyRange k{0, Nk, 0, 0};
    if (mask & kMaskCausal) k.hi = min(k.hi, r1 + off + 1);
    if (mask & kMaskWindow) k.lo = max(k.lo, r0 + off - W + 1);
    if (DOC) {
        k.dq0 = docrow[r0];
        k.dq1 = docrow[r1];
        k.lo = max(k.lo, wave_search<false>(docrow, Nk, k.dq0, lane));
        k.hi = min(k.hi, wave_search<true>(docrow, Nk, k.dq1, lane));
    }
    if (k.hi <= k.lo) {
        k.lo = INT_MAX;
        k.hi = INT_MIN;
    }
    return k;
}

// Whether every pair of rows [r0, r1] x keys of the tile starting at j0 is
// allowed, so the tile needs no element mask ("full"); a ragged last tile
// (fewer than BN keys) is never full, its missing keys being masked. dj0 / dj1:
// document ids of the tile's first and last key.
template <bool DOC>
__device__ __forceinline__ bool tile_full(int j0, int Nk, int r0, int r1, int off, int mask, int W,
                                          const KeyRange& k, int dj0, int dj1) {
    const int j1 = min(j0 + BN, Nk) - 1;
    bool full = j0 + BN <= Nk;
    if (mask & kMaskCausal) full &= j1 <= r0 + off;
    if (mask & kMaskWindow) full &= (r1 + off) - j0 < W;
    if (DOC) full &= dj0 == dj1 && k.dq0 == k.dq1 && dj0 == k.dq0;
    return full;
}

// Copy of one BN-row tile of K (or V) into LDS with its swizzle: LDS slot s
// of the tile (16 bytes) receives logical chunk (s % CPR) ^ swz(row) of row
// s / CPR. A wave moves 64 slots per instruction; the lane's byte offset
// within the tile is fixed, the tile base moves in scalar registers.
template <int D, int NW>
struct TileCopy {
    using T = Tile<D>;
    static constexpr int ROUNDS = BN * T::CPR / (NW * 64);
    static constexpr int ROWS_PER_ROUND = NW * 64 / T::CPR;
    static_assert(ROUNDS * NW * 64 == BN * T::CPR, "tile must split evenly over the waves");
    static_assert(ROUNDS == 1 || ROWS_PER_ROUND % 16 == 0, "swizzle must repeat across rounds");
    int r0;             // tile row of this lane in round 0
    unsigned k_chunk;   // swizzled byte offset within the row, K layout
    unsigned v_chunk;   // same, V layout

    __device__ __forceinline__ void init(int wave, int lane) {
        const int s = wave * 64 + lane;
        r0 = s / T::CPR;
        const int pc = s % T::CPR;
        k_chunk = (pc ^ T::swz_k(r0)) * 16;
        v_chunk = (pc ^ T::swz_v(r0)) * 16;
    }

    // Rows past Nk re-read row Nk - 1 (finite data the mask then ignores).
    template <bool IS_V>
    __device__ __forceinline__ void issue(const __bf16* X, int kv0, int Nk, unsigned tile_lds, int wave) const {
        const char* base = (const char*)X + (size_t)kv0 * T::ROW_BYTES;
        const unsigned chunk = IS_V ? v_chunk : k_chunk;
        if (kv0 + BN <= Nk) {
#pragma unroll
            for (int rd = 0; rd < ROUNDS; ++rd)
                dma16s(base + rd * ROWS_PER_ROUND * T::ROW_BYTES, r0 * T::ROW_BYTES + chunk,
                       tile_lds + (rd * NW + wave) * 1024);
        } else {
#pragma unroll
            for (int rd = 0; rd < ROUNDS; ++rd) {
                const int row = min(rd * ROWS_PER_ROUND + r0, Nk - 1 - kv0);
                dma16s(base, row * T::ROW_BYTES + chunk, tile_lds + (rd * NW + wave) * 1024);
            }
        }
    }
};

// Document ids of one key tile: every wave keeps its own copy (64 x 4 bytes).
__device__ __forceinline__ void issue_docs(const int32_t* docrow, int kv0, int Nk, unsigned docs_lds, int wave,
                                           int lane) {
    const int j = min(lane, Nk - 1 - kv0);
    dma4s(docrow + kv0, j * 4, docs_lds + wave * BN * 4);
}

}  // namespace attn
