// Pieces shared by the forward kernels: key-tile geometry and LDS swizzles,
// the wave-parallel search over document ids, and the K/V tile copy.
#pragma once
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
