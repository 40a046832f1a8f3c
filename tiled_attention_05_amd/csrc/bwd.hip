// Attention backward: dQ, dK, dV from Q, K, V, O, dO and the forward's LSE.
//
// With P_ij = exp(scale q_i.k_j - LSE_i) recomputed from the saved LSE (the
// N x N matrix is never stored) and D_i = sum_c dO_ic O_ic:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
// The result is exact and deterministic ("FlashAttention-2 (FR)", section
// "Performance et efficacite"); FlexAttention's backward loses determinism with
// block sparsity ("FlexAttention de PyTorch avec FlashAttention-4 change la
// donne", section "Limitations actuelles") -- here no gradient is accumulated
// with atomics: dK / dV are owned by one wave per key block (looping over the
// queries and the group's query heads), dQ by one wave per query block.
//
// Products are 32x32x16 bf16 MFMAs (A: lane l holds row l % 32, k = 8 (l / 32)
// + 0..7; B: column l % 32; C: lane l, register r holds row 8 (r / 4) +
// 4 (l / 32) + r % 4, column l % 32). A wave's own block is read once: into
// registers (K for dK / dV, Q and dO for dQ) or into the wave's part of LDS
// (V for dK / dV). The streamed chunks (Q and dO for dK / dV, K and V for dQ)
// go through LDS tiles shared by the workgroup's 4 waves, read row-wise (16-byte
// reads) and, where an operand is needed transposed (Q^T, dO^T, K^T), with the
// transposed reads of the prefill kernel's V layout; the probabilities are
// packed in the matching permuted order.
#include <climits>
#include <type_traits>

#include "fwd_common.h"

namespace attn {

struct BwdParams {
    const __bf16 *q, *k, *v, *o, *dout;   // BHSD bf16
    const float* lse;                     // [B][Hq][N] natural log
    float* dsum;                          // [B][Hq][N] scratch: D_i
    __bf16 *dq, *dk, *dv;
    int B, Hq, Hkv, G, N;
    float scale, scale_log2;
    int causal;
    int xg_kv, xg_q;   // heads per XCD dispatch group of the dK/dV and dQ parts, 0 = plain order
    int n_kv;          // dK/dV workgroups of the gradient grid (a multiple of 8), the dQ ones follow
};

// Work item of a grid of n_heads x ng workgroups, group index heaviest first
// (the caller maps it to its blocks). Round-robin dispatch puts workgroup w
// on XCD w % 8; with xg > 0 each XCD takes its heads xg at a time, all groups
// of those heads before the next ones, so the workgroups in flight on one XCD
// share the few heads' rows in its L2.
__device__ inline void grid_item(int w, int n_heads, int ng, int xg, int& head, int& grp) {
    if (xg > 0) {
        const int x = w % 8, k = w / 8, per = xg * ng, r = k % per;
        grp = r / xg;
        head = x + 8 * ((k / per) * xg + r % xg);
    } else {
        grp = w / n_heads;
        head = w % n_heads;
    }
}

constexpr int kBD = 128, kBC = 32;   // head dim, rows per block / chunk

// D_i = sum_c dO_ic O_ic (float32): 16 lanes per row (16 bytes each, so a
// wave reads 4 whole rows per instruction), 16 rows per 256-thread block.
__global__ __launch_bounds__(256) void bwd_dsum_kernel(BwdParams p) {
    const size_t rows = (size_t)p.B * p.Hq * p.N;
    const size_t row = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    float s = 0.f;
    if (row < rows) {
        const bf16x8 x = *(const bf16x8*)(p.dout + row * kBD + 8 * c);
        const bf16x8 y = *(const bf16x8*)(p.o + row * kBD + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) s = __builtin_fmaf((float)x[e], (float)y[e], s);
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m);   // within the 16-lane group
    if (row < rows && c == 0) p.dsum[row] = s;
}

// Transposed-read offsets of the prefill kernel (one 32-row tile): lane L of a
// 16-lane group addresses row 4 hh + L / 4 (+ 16 u, + 8 for the high half),
// columns 32 t + 16 cg + 4 (L % 4).
__device__ __forceinline__ void tr_offsets(int lane, int ofs[4]) {
    using T = Tile<kBD>;
    const int hh = lane >> 5, Ln = lane & 15, cg = (lane >> 4) & 1;
    const int r = 4 * hh + (Ln >> 2);
    const int col = 16 * cg + 4 * (Ln & 3);
    const int v0 = r * T::ROW_BYTES + ((((col * 2) >> 4) ^ T::swz_v(r)) << 4) + ((col * 2) & 15);
#pragma unroll
    for (int t = 0; t < 4; ++t) ofs[t] = v0 ^ (64 * t);
}

// Rows r0 .. r0 + 31 of one head (row-major [N][128], rows clamped to N - 1)
// into an LDS tile shared by the 4 waves of a workgroup: wave w copies the 4
// rows of slots i = 2 w, 2 w + 1 of 8. A tile read transposed (by itself or
// also row-wise) takes the prefill kernel's V swizzle (chunk c of row r at
// c ^ 4 (r mod 4)); a tile read only row-wise (ROWS) chunk c ^ (r mod 16),
// in which the 16 rows of a quarter-wave's 16-byte reads hit 16 bank groups
// instead of 4.
template <bool ROWS = false>
__device__ __forceinline__ void tile_part_to_lds(const __bf16* head, int r0, int N, unsigned base, int lane,
                                                 int wave) {
    using T = Tile<kBD>;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int i = 2 * wave + k;
        const int slot = i * 64 + lane, r = slot >> 4, pc = slot & 15;
        const __bf16* src = head + (size_t)min(r0 + r, N - 1) * kBD + 8 * (pc ^ (ROWS ? T::swz_k(r) : T::swz_v(r)));
        dma16(src, base + i * 1024);
    }
}

// Wait for this wave's copies, then meet the other waves: after it, every
// wave's share of the tiles has landed and every wave has finished reading
// the buffer the next copies refill.
__device__ __forceinline__ void copies_landed_barrier() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A-operand (or B-operand) fragments of rows r0 + l32: dims 16 s + 8 hh + 0..7.
__device__ __forceinline__ void row_frags(const __bf16* head, int r0, int N, int lane, bf16x8 f[8]) {
    const __bf16* rp = head + (size_t)min(r0 + (lane & 31), N - 1) * kBD + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = *(const bf16x8*)(rp + 16 * s);
}

// Row fragments (A or B operand: row l32 of the tile, dims 16 s + 8 hh + 0..7)
// read from an LDS tile in the layout (ROWS or not) of tile_part_to_lds.
template <bool ROWS = false>
__device__ __forceinline__ void lds_row_frags(const ATTN_LDS char* tile, int lane, bf16x8 f[8]) {
    using T = Tile<kBD>;
    const int r = lane & 31, hh = lane >> 5;
    const ATTN_LDS char* rp = tile + r * T::ROW_BYTES;
#pragma unroll
    for (int s = 0; s < 8; ++s)
        f[s] = *(const ATTN_LDS bf16x8*)(rp + (((2 * s + hh) ^ (ROWS ? T::swz_k(r) : T::swz_v(r))) << 4));
}

// Product of a tile read transposed from LDS (A: 32 d-rows x 16 tile rows, per
// output tile t and step u) with packed values (B): acc[t] += A_t,u B_u.
__device__ __forceinline__ void tr_gemm(const ATTN_LDS char* tile, const int ofs[4], const bf16x8 pk[2],
                                        f32x16 acc[4]) {
    constexpr int RB = Tile<kBD>::ROW_BYTES;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const ATTN_LDS char* a = tile + ofs[t] + 16 * u * RB;
            const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4*)a);
            const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4*)(a + 8 * RB));
            acc[t] = mfma_bf16(__builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7), pk[u], acc[t]);
        }
}

// The fragments of tr_gemm, all requested at once (f[4 u + t]), and its
// products from them: for a caller with registers to hold the 8 fragments, so
// that their reads overlap its vector work.
__device__ __forceinline__ void tr_frags(const ATTN_LDS char* tile, const int ofs[4], bf16x8 f[8]) {
    constexpr int RB = Tile<kBD>::ROW_BYTES;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const ATTN_LDS char* a = tile + ofs[t] + 16 * u * RB;
            const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4*)a);
            const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4*)(a + 8 * RB));
            f[4 * u + t] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        }
}
__device__ __forceinline__ void tr_products(const bf16x8 f[8], const bf16x8 pk[2], f32x16 acc[4]) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[t] = mfma_bf16(f[4 * u + t], pk[u], acc[t]);
}

// Writes acc (C layout: rows = d, column = lane's row r0 + l32) scaled by f as
// bf16 rows of [N][128].
__device__ __forceinline__ void store_rows(__bf16* head, int r0, int N, int lane, const f32x16 acc[4], float f) {
    const int row = r0 + (lane & 31);
    if (row >= N) return;
    __bf16* orow = head + (size_t)row * kBD + 4 * (lane >> 5);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[t][4 * gq + e] * f);
            *(bf16x4*)(orow + 32 * t + 8 * gq) = w;
        }
}

// LDS of a gradient workgroup: two buffers of two 32-row chunk tiles (dK / dV:
// Q and dO; dQ: K and V), each wave's own V block (dK / dV) and the chunk's LSE
// and D values (dK / dV). 65 KB: two workgroups fit a CU.
struct BwdLds {
    __attribute__((aligned(1024))) char tiles[2][2][kBC * Tile<kBD>::ROW_BYTES];
    __attribute__((aligned(1024))) char vblk[4][kBC * Tile<kBD>::ROW_BYTES];
    __attribute__((aligned(16))) float stat[2][2 * kBC];
};

// dK, dV: one wave per (batch, key/value head, 32-key block), looping over
// the query chunks of every query head of the group. The 4 waves of a
// workgroup own 4 consecutive key blocks of one head, so they need the same
// Q / dO chunks: the chunk tiles are shared, each wave copying a quarter (a
// wave past the last key block still copies and meets the barriers; its keys
// are masked out and it stores nothing). Under a causal mask the group starts
// at the first chunk its first block sees; for the later blocks the first
// chunks are fully masked and add exact zeros. The next chunk's tiles are
// requested before the current chunk is computed (two LDS buffer sets, one
// barrier per chunk); the loop has no load the compiler counts. Two
// workgroups per CU (two waves per SIMD, 256 registers each; the wave's K
// block in registers, its V block in LDS) hide the latency of each wave's
// serial chain S -> P -> dV, dK about 1.35x better than one wave per SIMD.
__device__ __forceinline__ void dkdv_block(const BwdParams& p, int bid, BwdLds& sm) {
    auto& lds = sm.tiles;   // [buffer][Q, dO]
    auto& stat = sm.stat;   // [buffer]: LSE then D of the chunk
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nkb = (p.N + kBC - 1) / kBC, nkg = (nkb + 3) / 4;
    // heavy groups first: under a causal mask the first key blocks see the most query chunks
    int kg, bg;
    if (bid >= p.B * p.Hkv * nkg) return;   // padding of the dK/dV part to a multiple of 8
    grid_item(bid, p.B * p.Hkv, nkg, p.xg_kv, bg, kg);
    const int g = bg % p.Hkv, b = bg / p.Hkv;
    const int kb = 4 * kg + wave;   // may be >= nkb: then every key of the block is masked
    const int l32 = lane & 31, hh = lane >> 5;
    const int j0 = kb * kBC;
    const size_t kvh = ((size_t)b * p.Hkv + g) * p.N * kBD;
    bf16x8 kf[8];
    row_frags(p.k + kvh, j0, p.N, lane, kf);   // B operand of S = Q K^T: column = key
    // The V block (B operand of dP = dO V^T) stays in this wave's LDS, read
    // each chunk: held in registers it pushed the loop past the 256-register
    // cap (values reloaded from scratch every chunk). Chunk c of row r at
    // c ^ (r mod 16), so the 16 rows of a 16-byte row read hit 16 bank groups.
    ATTN_LDS char* vb = (ATTN_LDS char*)sm.vblk[wave];
    {
        using T = Tile<kBD>;
#pragma unroll
        for (int i = 0; i < 8; ++i) {   // 4 rows of 16 chunks per copy
            const int r = 4 * i + (lane >> 4), pc = lane & 15;
            dma16(p.v + kvh + (size_t)min(j0 + r, p.N - 1) * kBD + 8 * (pc ^ T::swz_k(r)), lds_addr(vb + i * 1024));
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no compiler-counted load stays pending into the loop
    int ofs[4];
    tr_offsets(lane, ofs);
    f32x16 dv[4], dk[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) dv[t] = dk[t] = f32x16{};
    const int key = j0 + l32;
    const int qc0 = p.causal ? 4 * kg : 0;   // the first query chunk that sees the group's first block
    const int nqc = (p.N + kBC - 1) / kBC;
    const int per_head = nqc - qc0, total = p.G * per_head;

    auto issue = [&](int it, int buf) __attribute__((always_inline)) {
        const int h = g * p.G + it / per_head, i0 = (qc0 + it % per_head) * kBC;
        const size_t qh = ((size_t)b * p.Hq + h) * p.N * kBD;
        tile_part_to_lds(p.q + qh, i0, p.N, lds_addr((ATTN_LDS char*)lds[buf][0]), lane, wave);
        tile_part_to_lds(p.dout + qh, i0, p.N, lds_addr((ATTN_LDS char*)lds[buf][1]), lane, wave);
        // wave 0, lanes 0-31: LSE of the chunk's queries, lanes 32-63: D (one 4-byte copy each)
        if (wave == 0) {
            const size_t qr = ((size_t)b * p.Hq + h) * p.N + min(i0 + l32, p.N - 1);
            dma4(hh ? (const void*)(p.dsum + qr) : (const void*)(p.lse + qr), lds_addr((ATTN_LDS float*)stat[buf]));
        }
    };
    auto compute = [&](int it, int buf) __attribute__((always_inline)) {
        const int i0 = (qc0 + it % per_head) * kBC;
        // S = Q K^T and dP = dO V^T: lane = key, registers = queries 8 (r / 4) + 4 hh + r % 4
        bf16x8 af[8];
        f32x16 s = f32x16{}, dp = f32x16{};
        lds_row_frags((const ATTN_LDS char*)lds[buf][0], lane, af);
#pragma unroll
        for (int st = 0; st < 8; ++st) s = mfma_bf16(af[st], kf[st], s);
        lds_row_frags((const ATTN_LDS char*)lds[buf][1], lane, af);
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            using T = Tile<kBD>;
            const bf16x8 vf = *(const ATTN_LDS bf16x8*)(vb + l32 * T::ROW_BYTES + (((2 * st + hh) ^ T::swz_k(l32)) << 4));
            dp = mfma_bf16(af[st], vf, dp);
        }
        bf16x8 pk[2], sk[2];
        // Element r of the lane is query i0 + 4 hh + c, c = 8 (r / 4) + r % 4:
        // allowed when lo <= c < lo + range (one unsigned compare per element;
        // range 0 when the lane's key is past N)
        const int base = i0 + 4 * hh;
        const int lo = p.causal ? key - base : -kBC;
        const int range = key < p.N ? max(p.N - base - lo, 0) : 0;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int q4 = 8 * r4 + 4 * hh;   // queries q4 .. q4 + 3 of the chunk
            const f32x4 l4 = *(const ATTN_LDS f32x4*)((const ATTN_LDS float*)stat[buf] + q4);
            const f32x4 d4 = *(const ATTN_LDS f32x4*)((const ATTN_LDS float*)stat[buf] + kBC + q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * r4 + e;
                // branch-free: the exponential of every element, then a select
                // (a short-circuit condition around it became per-element
                // exec-mask branches); keys and queries past N are clamped rows,
                // so the discarded values are finite or +inf, never read
                const bool ok = (unsigned)(8 * r4 + e - lo) < (unsigned)range;
                const float ex = fast_exp2(s[r] * p.scale_log2 - l4[e] * kLog2e);
                const float pr = ok ? ex : 0.f;
                pk[r >> 3][r & 7] = (__bf16)pr;
                sk[r >> 3][r & 7] = (__bf16)(pr * (dp[r] - d4[e]));
            }
        }
        tr_gemm((const ATTN_LDS char*)lds[buf][1], ofs, pk, dv);   // dV^T += dO^T P
        tr_gemm((const ATTN_LDS char*)lds[buf][0], ofs, sk, dk);   // dK^T += Q^T dS
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next barrier
    };
    if (total > 0) issue(0, 0);
    for (int it = 0; it < total; ++it) {
        copies_landed_barrier();   // chunk it is in LDS; buffer (it + 1) & 1 is no longer read
        if (it + 1 < total) issue(it + 1, (it + 1) & 1);
        compute(it, it & 1);
    }
    store_rows(p.dk + kvh, j0, p.N, lane, dk, p.scale);
    store_rows(p.dv + kvh, j0, p.N, lane, dv, 1.f);
}

// dQ: one wave per (batch, query head, 32-query block). The next key chunk's
// K and V tiles are requested before the current chunk is computed (two LDS
// buffer pairs, one barrier per chunk); K and V fragments are read from them.
// The 4 waves of a workgroup own 4 consecutive query blocks of one head and
// share the K / V chunk tiles, each wave copying a quarter (a wave past the
// last query block still copies and meets the barriers, and stores nothing);
// under a causal mask the group runs to the last chunk its last block sees,
// the chunks beyond a block's diagonal being fully masked (exact zeros).
__device__ __forceinline__ void dq_block(const BwdParams& p, int bid, BwdLds& sm) {
    auto& lds = sm.tiles;   // [buffer][K, V]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nqb = (p.N + kBC - 1) / kBC, nqg = (nqb + 3) / 4;
    // heavy groups first: under a causal mask the last query blocks see the most key chunks
    int qg, bh;
    grid_item(bid, p.B * p.Hq, nqg, p.xg_q, bh, qg);
    qg = nqg - 1 - qg;
    const int h = bh % p.Hq, b = bh / p.Hq;
    const int qb = 4 * qg + wave;   // may be >= nqb: then every query of the block is masked
    const int g = h / p.G;
    const int l32 = lane & 31, hh = lane >> 5;
    const int i0 = qb * kBC;
    const size_t qh = ((size_t)b * p.Hq + h) * p.N;
    const size_t kvh = ((size_t)b * p.Hkv + g) * p.N * kBD;
    bf16x8 qf[8], df[8];
    row_frags(p.q + qh * kBD, i0, p.N, lane, qf);      // B operand of S^T = K Q^T: column = query
    row_frags(p.dout + qh * kBD, i0, p.N, lane, df);   // B operand of dP^T = V dO^T
    const int qrow = i0 + l32;
    const float lse2 = p.lse[qh + min(qrow, p.N - 1)] * kLog2e;
    const float dd = p.dsum[qh + min(qrow, p.N - 1)];
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no compiler-counted load stays pending into the loop
    int ofs[4];
    tr_offsets(lane, ofs);
    f32x16 dq[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) dq[t] = f32x16{};
    const int nkc = p.causal ? min(4 * qg + 4, nqb) : nqb;   // key chunks of the group (chunk = block size)

    auto issue = [&](int kc, int buf) __attribute__((always_inline)) {
        tile_part_to_lds(p.k + kvh, kc * kBC, p.N, lds_addr((ATTN_LDS char*)lds[buf][0]), lane, wave);
        tile_part_to_lds<true>(p.v + kvh, kc * kBC, p.N, lds_addr((ATTN_LDS char*)lds[buf][1]), lane, wave);
    };
    auto compute = [&](int kc, int buf) __attribute__((always_inline)) {
        const int j0 = kc * kBC;
        // every (query, key) pair of the chunk allowed (see the dK / dV kernel)
        const bool full = i0 + kBC <= p.N && j0 + kBC <= p.N && (!p.causal || j0 + kBC - 1 <= i0);
        // S^T = K Q^T, dP^T = V dO^T: lane = query, registers = keys 8 (r / 4) + 4 hh + r % 4
        // both fragment sets requested before the products (the registers are there)
        bf16x8 kr[8], vr[8];
        f32x16 s = f32x16{}, dp = f32x16{};
        lds_row_frags((const ATTN_LDS char*)lds[buf][0], lane, kr);
        lds_row_frags<true>((const ATTN_LDS char*)lds[buf][1], lane, vr);
#pragma unroll
        for (int st = 0; st < 8; ++st) s = mfma_bf16(kr[st], qf[st], s);
#pragma unroll
        for (int st = 0; st < 8; ++st) dp = mfma_bf16(vr[st], df[st], dp);
        // K^T fragments of the dQ products, read while the probabilities are computed
        bf16x8 ktf[8];
        tr_frags((const ATTN_LDS char*)lds[buf][0], ofs, ktf);
        asm volatile("" ::: "memory");
        bf16x8 sk[2];
        auto probs = [&](auto mask_c) __attribute__((always_inline)) {
            constexpr bool MASK = decltype(mask_c)::value;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = j0 + 8 * (r >> 2) + 4 * hh + (r & 3);
                const bool ok = !MASK || ((qrow < p.N) & (key < p.N) & (!p.causal | (key <= qrow)));
                const float ex = fast_exp2(s[r] * p.scale_log2 - lse2);   // branch-free, as in dK / dV
                const float pr = ok ? ex : 0.f;
                sk[r >> 3][r & 7] = (__bf16)(pr * (dp[r] - dd));
            }
        };
        if (full) probs(std::integral_constant<bool, false>{});
        else probs(std::integral_constant<bool, true>{});
        tr_products(ktf, sk, dq);   // dQ^T += K^T dS^T
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next barrier
    };
    if (nkc > 0) issue(0, 0);
    for (int kc = 0; kc < nkc; ++kc) {
        copies_landed_barrier();   // chunk kc is in LDS; buffer (kc + 1) & 1 is no longer read
        if (kc + 1 < nkc) issue(kc + 1, (kc + 1) & 1);
        compute(kc, kc & 1);
    }
    store_rows(p.dq + qh * kBD, i0, p.N, lane, dq, p.scale);
}

// dK/dV and dQ need only the inputs and D, not each other: one grid holds the
// dK/dV workgroups first and the dQ workgroups after them, so the dQ work
// fills the CUs the end of the dK/dV part leaves idle. Two workgroups per CU
// (two waves per SIMD, 256 registers each) hide the latency of each wave's
// serial product chain.
// The dK/dV part is padded to a multiple of 8 workgroups, so that workgroup
// n_kv + w of the dQ part runs on the XCD w would (round-robin dispatch).
__global__ __launch_bounds__(256, 2) void bwd_grad_kernel(BwdParams p) {
    __shared__ BwdLds sm;
    const int bid = blockIdx.x;
    if (bid < p.n_kv) dkdv_block(p, bid, sm);
    else dq_block(p, bid - p.n_kv, sm);
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, float* workspace, int B, int Hq, int Hkv, int N, float scale,
                      int causal, hipStream_t st) {
    BwdParams p{};
    p.q = (const __bf16*)q; p.k = (const __bf16*)k; p.v = (const __bf16*)v;
    p.o = (const __bf16*)o; p.dout = (const __bf16*)dout;
    p.lse = lse; p.dsum = workspace;
    p.dq = (__bf16*)dq; p.dk = (__bf16*)dk; p.dv = (__bf16*)dv;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.N = N;
    p.scale = scale; p.scale_log2 = scale * kLog2e; p.causal = causal;
    const size_t rows = (size_t)p.B * p.Hq * p.N;
    hipLaunchKernelGGL(bwd_dsum_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // one workgroup per 4 consecutive blocks of 32 rows of one head
    const long long ng = ((p.N + kBC - 1) / kBC + 3) / 4;
    // Dispatch groups of as many heads as fill an XCD's resident workgroups
    // (32 CUs, two workgroups each), when the heads split evenly over the 8
    // XCDs and into groups of at least two.
    auto xcd_group = [&](long long n_heads) {
        if (n_heads % 8 || ng > 32) return 0;
        int g = (int)(64 / ng);
        while (g > 1 && (n_heads / 8) % g) --g;
        return g >= 2 ? g : 0;
    };
    p.xg_kv = xcd_group((long long)p.B * p.Hkv);
    p.xg_q = xcd_group((long long)p.B * p.Hq);
    const long long n_kv = ((long long)p.B * p.Hkv * ng + 7) / 8 * 8;
    p.n_kv = (int)n_kv;
    hipLaunchKernelGGL(bwd_grad_kernel, dim3((unsigned)(n_kv + (long long)p.B * p.Hq * ng)), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace attn
