// Fused attention forward for gfx950, bf16 inputs.
//
// One workgroup computes a BM = NW * QB * 32 row query tile of one (batch,
// query head). Key / value tiles of BN = 64 rows stream HBM -> LDS with direct
// global->LDS copies; the score tile lives only in registers and the output is
// rescaled on chip, so no score matrix is ever written to device memory ("Les
// kernels d'attention rapide et la fusion d'operateurs ...", section "Attention
// de type FlashAttention et attention paginee"; "FlashAttention-3 : ...",
// section "Rappel du fonctionnement de FlashAttention").
//
// Matrix-core formulation (CDNA4 32x32x16 bf16 MFMA, 64-wide waves):
//   GEMM0  S^T = K Q^T   A = K rows from LDS, B = Q rows kept in registers.
//          The accumulator holds one query per lane (lane & 31) and 16 keys,
//          so row max / row sum are in-lane plus one half-wave exchange.
//   GEMM1  O^T = V^T P^T A = V read transposed from LDS (ds_read_b64_tr_b16),
//          B = P straight from the GEMM0 accumulator registers (bf16). The
//          output accumulator again holds one query per lane.
// Each wave owns 32 query rows; eight waves (two per SIMD) make a 256-row tile.
//
// Softmax/GEMM overlap between the two waves of each SIMD, the counterpart of
// the ping-pong schedule of "FlashAttention-3 : ...", section "Ping-pong
// scheduling entre warpgroups". Every wave runs the same loop body
//     softmax(j), GEMM1(j), GEMM0(j + 1)
// but meets the per-tile workgroup barrier at a different point: waves 4-7
// (group B) before the softmax, waves 0-3 (group A, one per SIMD next to a B
// wave) before GEMM0. Between two barriers group A therefore runs GEMM0(i),
// softmax(i), GEMM1(i) while group B runs softmax(i-1), GEMM1(i-1), GEMM0(i):
// while one wave of a SIMD is in its exp / max / sum phase the other keeps the
// matrix core busy. Sharing one body keeps the register assignment identical
// for both groups. Key tiles are double-buffered, value tiles (read for two
// consecutive tiles) triple-buffered; one workgroup barrier per tile.
//
// Softmax: exp2 with scale * log2(e) folded into one FMA per score, running
// max / running sum per row, a single division at the end ("FlashAttention-2
// (FR)", section "Architecture technique", item 1). The running max used as
// the exponent reference is only moved when the row max has grown by more than
// 2^8 ("lazy" rescale): the output accumulator is then rescaled rarely, and the
// result is unchanged because O / l and the LSE use the same reference. The
// exponents are first taken against the current references; the row max is
// computed only when one of a lane's partial sums of p (a bound on each p in
// it) shows that a reference may have to move.
// Masked tiles and score modifiers first rewrite the scores in place (exp2
// units, -inf where not allowed); the softmax code is then the same.
//
// Register files: the matrix instructions are issued as inline assembly with
// the output accumulator and the Q fragments in AGPRs (only the matrix core
// reads them) and the scores / probabilities in VGPRs, so no copies between
// the two files appear in the loop. Each wave runs its own loops around its
// key range (the same number of barriers as every other wave), so the
// steady-state body has no per-tile branches around the matrix work.
//
// Tiles are classified per wave as empty (outside the wave's contiguous key
// range, skipped), partial (element mask) or full (no mask code): closed form
// for causal / window, from the tile's first / last document id for packed
// documents.
#include <climits>
#include <cstdlib>
#include <type_traits>

#include "fwd_common.h"

namespace attn {
// Degree-3 fit of tanh(u) / u in t = u^2 on |u| <= kTanhPolyU (weighted least
// squares on Chebyshev nodes, reweighted toward equal relative error).
constexpr float kTanhPolyU = 0.5f;
constexpr float kTanhP0 = 0.999999463558197f, kTanhP1 = -0.33326318860054016f;
constexpr float kTanhP2 = 0.13190290331840515f, kTanhP3 = -0.04440207779407501f;
// Degree-2 fit of the same on |u| <= kTanhPoly2U (same method; relative error
// 4.5e-7 evaluated in float32), one FMA fewer per score.
constexpr float kTanhPoly2U = 0.25f;
constexpr float kTanhQ0 = 0.9999995827674866f, kTanhQ1 = -0.33321908116340637f;
constexpr float kTanhQ2 = 0.12841613590717316f;
// Degree-1 fit of the same on |u| <= kTanhPoly1U (same method; relative error
// 4.2e-6 evaluated in float32), for the small scores most tiles hold.
constexpr float kTanhPoly1U = 0.125f;
constexpr float kTanhL0 = 0.9999959468841553f, kTanhL1 = -0.33126187324523926f;
}  // namespace attn

#ifdef ATTN_SINGLE_STAGE
// Debug build: one key/value tile in flight, each copy waited for as soon as it
// is issued, fragments read just before their product. The arithmetic is the
// same as in the pipelined build, so the results must be equal bit for bit.
#define ATTN_PREFETCH 1
#define ATTN_LDS_AHEAD 1
#define ATTN_LATE_COPY_A 0
#define ATTN_LATE_COPY_B 0
#endif
#ifndef ATTN_LDS_AHEAD
#define ATTN_LDS_AHEAD 4   // matrix fragments read from LDS ahead of their product
#endif
#ifndef ATTN_LATE_COPY_A
#define ATTN_LATE_COPY_A 1
#endif
#ifndef ATTN_LATE_COPY_B
#define ATTN_LATE_COPY_B 1
#endif
#ifndef ATTN_PREFETCH
#define ATTN_PREFETCH 2   // key/value tiles in flight ahead of the matrix work (1..3)
#endif

namespace attn {

constexpr float kLazyTau = 8.f;     // log2 units: rescale O only when the max grows by > 2^8
constexpr float kNoMax = -1e30f;    // initial reference: finite, below any score
// Each of a lane's partial sums of p (8 p each) bounds the p it holds; at or
// below this limit every p is below 2^(kLazyTau - 0.005): no reference moves.
constexpr float kSpecSumLimit = 255.f;

// LDS of one workgroup of the bf16 forward.
template <int D, bool DOC>
struct Bf16Lds {
    static constexpr int NW = 8, PF = ATTN_PREFETCH, NKB = PF + 1, NVB = PF + 2;
    __attribute__((aligned(1024))) char tiles[(NKB + NVB) * Tile<D>::BYTES];
    __attribute__((aligned(16))) int docs[DOC ? NVB * NW * BN : 4];
    int range[NW][2];
};

// One work item (query tile qt of one (batch, head)) of the bf16 forward,
// run by the whole workgroup; wid is the item's index in the launch order.
template <int D, bool SOFTCAP, bool ALIBI, bool DOC, bool PERSIST = false>
__device__ __attribute__((always_inline)) void fwd_bf16_item(const FwdParams& p, int wid,
                                                             Bf16Lds<D, DOC>& sm) {
    using T = Tile<D>;
    constexpr int NW = 8;        // waves: 4 in group A, 4 in group B
    constexpr int BM = NW * 32;
    constexpr int DS = D / 16;   // GEMM0 k-steps
    constexpr int DT = D / 32;   // output d-subtiles
    constexpr bool MODS = SOFTCAP || ALIBI;
    // Copies run PF tiles ahead of the matrix work; key tiles need PF + 1
    // buffers, value tiles (read during two consecutive intervals) PF + 2.
    constexpr int PF = ATTN_PREFETCH;
    static_assert(PF >= 1 && PF <= 3, "prefetch distance 1 to 3");
    constexpr int NKB = PF + 1, NVB = PF + 2;
    // LDS fragments are read LA products ahead of their use; a fragment
    // register is refilled two products after the product that read it.
    constexpr int LA = ATTN_LDS_AHEAD, NB = LA + 2;
    static_assert(LA >= 1 && LA <= 7, "read-ahead 1..7 (lgkmcnt range)");
    // Without modifiers or document ids, group A issues all the copies (its
    // waves wait at the barrier while group B finishes its matrix phase, so
    // the issue time is hidden there) and group B none; else every wave
    // issues its share.
    constexpr bool A_ONLY = !MODS && !DOC;
    using Copy = TileCopy<D, A_ONLY ? NW / 2 : NW>;
    constexpr int LOADS_PER_TILE = 2 * Copy::ROUNDS + (DOC ? 1 : 0);   // per copying wave

    char* tiles_lds = sm.tiles;
    int* docs_lds = sm.docs;
    auto& range_lds = sm.range;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool group_b = wave >= NW / 2;
    const int l32 = lane & 31, hh = lane >> 5;

    // ---- work item: heavy (late) query tiles first for causal balance
    int qt = p.n_qt - 1 - wid / p.n_bh;
    // (batch, head) slot j. Round-robin dispatch puts workgroup w on XCD
    // w % 8. With xgrp > 0 each XCD takes its heads xgrp at a time, all
    // query tiles of those heads (heaviest first) before the next ones, so
    // the tiles in flight on one XCD read the same few K / V heads from its
    // L2. With grouped heads, the heads of one key / value head are put 8
    // slots apart, i.e. on the same XCD, for the same reason.
    int j = wid % p.n_bh;
    if (p.xgrp > 0) {
        const int x = wid % 8, k = wid / 8, per = p.xgrp * p.n_qt;
        const int r = k % per;
        qt = p.n_qt - 1 - r / p.xgrp;
        j = x + 8 * ((k / per) * p.xgrp + r % p.xgrp);
    }
    int bh = j;
    const int n_u = p.B * p.Hkv;   // key / value heads
    if (p.group > 1 && n_u % 8 == 0) {
        const int u = (j / (8 * p.group)) * 8 + j % 8, q = (j / 8) % p.group;
        bh = (u / p.Hkv) * p.Hq + (u % p.Hkv) * p.group + q;
    }
    const int b = bh / p.Hq, h = bh % p.Hq, g = h / p.group;
    int Nq = p.Nq, Nk = p.Nk;
    // Packed variable-length batch tiled per sequence: the k-th heaviest
    // query tile is entry k of the item list (its first packed row); rows,
    // keys and pointers are then those of its sequence alone. Offsets are
    // clamped into the packed length, so any list stays in bounds.
    int row0 = 0;
    if (!DOC && p.items) {
        const int r = p.items[p.n_qt - 1 - qt];
        if (r < 0) return;   // list padding: the whole workgroup leaves before any barrier
        const int s = min(max(wave_search<true>(p.cu, p.n_seq + 1, r, lane) - 1, 0), p.n_seq - 1);
        const int s0 = min(max(p.cu[s], 0), p.Nq), s1 = min(max(p.cu[s + 1], s0), p.Nq);
        if (r < s0 || r >= s1) return;   // only with offsets that do not partition the batch
        Nq = Nk = s1 - s0;
        qt = (r - s0) / BM;
        row0 = s0;
    }
    const int off = Nk - Nq;
    const bool causal = p.mask & kMaskCausal, windowed = p.mask & kMaskWindow;
    const int W = p.window;
    const int q0 = qt * BM;

    // row 0 of this (batch, head) in Q / O (and LSE), and in K / V
    const size_t qbase = (size_t)(b * p.Hq + h) * p.Nq + row0;
    const size_t kbase = (size_t)(b * p.Hkv + g) * p.Nk + row0;
    const __bf16* Q = (const __bf16*)p.q + qbase * D;
    const __bf16* K = (const __bf16*)p.k + kbase * D;
    const __bf16* V = (const __bf16*)p.v + kbase * D;
    const int32_t* docrow = DOC ? p.doc + (size_t)b * Nk : nullptr;

    // ---- this wave's rows and its contiguous key range [w_lo, w_hi)
    const int wq0 = q0 + wave * 32;
    const bool wave_active = wq0 < Nq;
    const int wq1 = min(wq0 + 32, Nq) - 1;
    KeyRange kr{INT_MAX, INT_MIN, 0, 0};
    if (wave_active) kr = rows_key_range<DOC>(wq0, wq1, Nk, off, p.mask, W, docrow, lane);
    const int w_lo = kr.lo, w_hi = kr.hi;
    if (lane == 0) { range_lds[wave][0] = w_lo; range_lds[wave][1] = w_hi; }
    __syncthreads();
    int kv_lo = INT_MAX, kv_hi = INT_MIN;
#pragma unroll
    for (int w = 0; w < NW; ++w) { kv_lo = min(kv_lo, range_lds[w][0]); kv_hi = max(kv_hi, range_lds[w][1]); }
    const int kt_begin = kv_hi > kv_lo ? kv_lo / BN : 0;
    const int n_tiles = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN - kt_begin : 0;
    const int wt_begin = w_hi > w_lo ? w_lo / BN : 0;
    const int wt_end = w_hi > w_lo ? (w_hi + BN - 1) / BN : 0;
    // Order of the key tiles. With ALiBi under a causal mask the bias grows by
    // slope * 64 per tile toward the diagonal (up to about 65 in exp2 units
    // for the steepest head), so walking the keys forward would move the
    // exponent reference, and rescale the output, on almost every tile; from
    // the diagonal backward the row max is met first and rarely grows.
    const bool rev = ALIBI && causal;
    auto ktile = [&](int i) __attribute__((always_inline)) {   // key tile of step i
        return rev ? kt_begin + n_tiles - 1 - i : kt_begin + i;
    };

    const int row = wq0 + l32;
    const int doc_i = DOC ? docrow[min(row, Nq - 1)] : 0;
    const float c = p.scale_log2;
    const float slope_l2 = ALIBI ? p.slopes[h] * kLog2e : 0.f;
    const float cap_l2 = SOFTCAP ? p.softcap * kLog2e : 0.f;        // cap in exp2 units
    const float cap_in = SOFTCAP ? p.scale * 2.f * kLog2e / p.softcap : 0.f;
    // Soft-cap on small scores: cap tanh(v / cap) = v P((v / cap)^2) with
    // v = c x (exp2 units), P a degree-3 fit of tanh(u) / u on |u| <= 1/2
    // (relative error 6.2e-7 evaluated in float32). The coefficients are
    // rescaled so that x P'(x^2) gives the capped score straight from the raw
    // one (P'(t) = c P(c^2 t / cap^2)). Used for a tile when every raw score of
    // the wave satisfies |x| <= tc_xmax; when every |x| <= tq_xmax (|u| <= 1/4)
    // the degree-2 fit instead, when every |x| <= tl_xmax (|u| <= 1/8) the
    // degree-1 fit.
    float tc0 = 0.f, tc1 = 0.f, tc2 = 0.f, tc3 = 0.f, tc_xmax = 0.f;
    float tq0 = 0.f, tq1 = 0.f, tq2 = 0.f, tq_xmax = 0.f;   // the degree-2 form, |x| <= tq_xmax
    float tl0 = 0.f, tl1 = 0.f, tl_xmax = 0.f;              // the degree-1 form, |x| <= tl_xmax
    if (SOFTCAP) {
        const float k = c * c / (cap_l2 * cap_l2);   // u^2 = k x^2
        tc0 = kTanhP0 * c;
        tc1 = kTanhP1 * k * c;
        tc2 = kTanhP2 * k * k * c;
        tc3 = kTanhP3 * k * k * k * c;
        tc_xmax = kTanhPolyU * p.softcap / p.scale;
        tq0 = kTanhQ0 * c;
        tq1 = kTanhQ1 * k * c;
        tq2 = kTanhQ2 * k * k * c;
        tq_xmax = kTanhPoly2U * p.softcap / p.scale;
        tl0 = kTanhL0 * c;
        tl1 = kTanhL1 * k * c;
        tl_xmax = kTanhPoly1U * p.softcap / p.scale;
    }

    // ---- Q fragments (B operand of GEMM0): lane holds row l32, d = 16 s + 8 hh + 0..7
    bf16x8 qf[DS];
    {
        const __bf16* qr = Q + (size_t)min(row, Nq - 1) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < DS; ++s) qf[s] = *(const bf16x8*)(qr + 16 * s);
    }
    // Retire every compiler-visible global load here. The tile copies below
    // are inline asm the compiler does not count, so a load still pending at
    // the loop would get in-loop vmcnt waits that also drain the prefetches.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    f32x16 o[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) o[t] = f32x16{};
    float m = kNoMax, l = 0.f;
    // Matrix operands written by vector code: set here, pinned in their
    // register files and followed by wait states, so none of these writes
    // lands right before the first matrix instruction that reads it.
#pragma unroll
    for (int s = 0; s < DS; ++s) pin_a(qf[s]);
#pragma unroll
    for (int t = 0; t < DT; ++t) pin_a(o[t]);
    mfma_guard();

    // ---- lane-constant LDS offsets. With both swizzles, the offset of K-read
    // step s is koff0 ^ (32 s) and of V d-subtile t is voff0 ^ (64 t).
    // K reads: row 32 kb + l32, logical chunk 2 s + hh.
    const int koff0 = l32 * T::ROW_BYTES + ((hh ^ T::swz_k(l32)) * 16);
    // V transposed reads: in each 16-lane group lane L addresses row R0 + L/4
    // (R0 = 32 kb + 16 u + 8 part + 4 hh), columns 32 t + 16 cg + 4 (L % 4).
    int voff0;
    {
        const int L = lane & 15, cg = (lane >> 4) & 1;
        const int r = 4 * hh + (L >> 2);
        const int col = 16 * cg + 4 * (L & 3);
        voff0 = r * T::ROW_BYTES + ((((col * 2) >> 4) ^ T::swz_v(r)) << 4) + ((col * 2) & 15);
    }
    int kofs[DS], vofs[DT];
#pragma unroll
    for (int s = 0; s < DS; ++s) kofs[s] = koff0 ^ (32 * s);
#pragma unroll
    for (int t = 0; t < DT; ++t) vofs[t] = voff0 ^ (64 * t);

    ATTN_LDS char* lds = (ATTN_LDS char*)tiles_lds;
    auto kbuf = [&](int i) __attribute__((always_inline)) { return lds + (i % NKB) * T::BYTES; };
    auto vbuf = [&](int i) __attribute__((always_inline)) { return lds + (NKB + i % NVB) * T::BYTES; };
    auto dbuf = [&](int i) __attribute__((always_inline)) {
        return (ATTN_LDS int*)docs_lds + (i % NVB) * (NW * BN);
    };
    // Per-lane fragment addresses of one tile: the tile base is added once
    // and pinned there; the kb / u / row-half parts are immediate offsets.
    auto tile_addr = [&](const ATTN_LDS char* base, const int* ofs, int* a, int n) __attribute__((always_inline)) {
        // one scalar base (the buffer index arithmetic stays on the scalar unit)
        const int sb = __builtin_amdgcn_readfirstlane((int)lds_addr(base));
#pragma unroll
        for (int i = 0; i < n; ++i) {
            a[i] = sb + ofs[i];
            pin(a[i]);
        }
    };
    auto at = [](int addr, int imm) __attribute__((always_inline)) {
        return (const ATTN_LDS char*)(uintptr_t)addr + imm;
    };

    // ---------------------------------------------------------------- stages
    f32x16 sacc[2];   // S^T of the tile: [kb] keys 32 kb .. + 31, one query per lane
    bf16x8 pf[2][2];  // P fragments [kb][u]
    // GEMM0 of one tile: fragment i = (kb, s) read two fragments ahead.
    auto gemm0 = [&](const ATTN_LDS char* kl) __attribute__((always_inline)) {
        int ka[DS];
        tile_addr(kl, kofs, ka, DS);
        constexpr int NF = 2 * DS;
        bf16x8 kf[NB];
        auto rd = [&](int i) __attribute__((always_inline)) {
            return *(const ATTN_LDS bf16x8*)at(ka[i % DS], (i / DS) * 32 * T::ROW_BYTES);
        };
#pragma unroll
        for (int f = 0; f < LA && f < NF; ++f) kf[f] = rd(f);
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            const int kb = i / DS, st = i % DS;
            if (st == 0) mfma_bf16_va0(sacc[kb], kf[i % NB], qf[st]);
            else mfma_bf16_va(sacc[kb], kf[i % NB], qf[st]);
            if (i >= 2) keep(kf[(i - 2) % NB]);
            if (i + LA < NF) kf[(i + LA) % NB] = rd(i + LA);
        }
        keep(kf[(NF - 2) % NB]);
        keep(kf[(NF - 1) % NB]);
        mfma_guard();   // the scores may be read right after
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) pin(sacc[kb]);
    };
    // GEMM1 of one tile: fragment i = (kb, u, t) read two fragments ahead.
    auto gemm1 = [&](const ATTN_LDS char* vl) __attribute__((always_inline)) {
        int va[DT];
        tile_addr(vl, vofs, va, DT);
        constexpr int NF = 4 * DT;
        bf16x8 vf[NB];
        auto rd = [&](int i) __attribute__((always_inline)) {
            const int kb = i / (2 * DT), u = (i / DT) % 2, t = i % DT;
            const int imm = (32 * kb + 16 * u) * T::ROW_BYTES;
            const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4*)at(va[t], imm));
            const bf16x4 hi4 =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4*)at(va[t], imm + 8 * T::ROW_BYTES));
            return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        };
#pragma unroll
        for (int f = 0; f < LA && f < NF; ++f) vf[f] = rd(f);
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            const int kb = i / (2 * DT), u = (i / DT) % 2, t = i % DT;
            mfma_bf16_a(o[t], vf[i % NB], pf[kb][u]);
            if (i >= 2) keep(vf[(i - 2) % NB]);
            if (i + LA < NF) vf[(i + LA) % NB] = rd(i + LA);
        }
        keep(vf[(NF - 2) % NB]);
        keep(vf[(NF - 1) % NB]);
        keep(pf[1][0]);
        keep(pf[1][1]);
    };

    auto is_full = [&](int kt, const ATTN_LDS int* dl) __attribute__((always_inline)) -> bool {
        const int j0 = kt * BN;
        int dj0 = 0, dj1 = 0;
        if (DOC) {
            dj0 = dl[wave * BN];
            dj1 = dl[wave * BN + (min(j0 + BN, Nk) - 1 - j0)];
        }
        return tile_full<DOC>(j0, Nk, wq0, wq1, off, p.mask, W, kr, dj0, dj1);
    };

    // Score modifiers and / or the element mask, in place: the scores become
    // exp2-unit values plus zoff (the same for all scores of the lane), -inf
    // where the key is not allowed for the row.
    auto prepare_scores = [&](bool full, int kt, const ATTN_LDS int* dl, float zoff) __attribute__((always_inline)) {
        const int j0 = kt * BN;
        int dk[2][16];
        if (DOC && !full) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const i32x4 dv = *(const ATTN_LDS i32x4*)(dl + wave * BN + 32 * kb + 8 * gq + 4 * hh);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dk[kb][4 * gq + e] = dv[e];
                }
        }
        // allowed keys of this row within the tile: jl_lo <= jl <= jl_hi
        const int jl_hi = full ? BN : min(Nk - 1 - j0, causal ? row + off - j0 : INT_MAX / 2);
        const int jl_lo = (windowed && !full) ? row + off - W + 1 - j0 : 0;
        if (SOFTCAP) {
            // cap tanh(x / cap) in exp2 units, in place: the polynomial when
            // every raw score of the wave is in its range, else the exact form
            float a0 = max3_abs(sacc[0][0], sacc[0][1], sacc[0][2]);
            float a1 = max3_abs(sacc[1][0], sacc[1][1], sacc[1][2]);
#pragma unroll
            for (int r = 3; r < 15; r += 2) {
                a0 = max3_abs(a0, sacc[0][r], sacc[0][r + 1]);
                a1 = max3_abs(a1, sacc[1][r], sacc[1][r + 1]);
            }
            a0 = max3_abs(a0, sacc[0][15], a1);
            a0 = max3_abs(a0, sacc[1][15], sacc[1][15]);
            if (__builtin_amdgcn_ballot_w64(!(a0 <= tl_xmax)) == 0) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float x = sacc[kb][r], t = x * x;
                        sacc[kb][r] = __builtin_fmaf(x, __builtin_fmaf(tl1, t, tl0), zoff);
                    }
            } else if (__builtin_amdgcn_ballot_w64(!(a0 <= tq_xmax)) == 0) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float x = sacc[kb][r], t = x * x;
                        sacc[kb][r] = __builtin_fmaf(x, __builtin_fmaf(__builtin_fmaf(tq2, t, tq1), t, tq0), zoff);
                    }
            } else if (__builtin_amdgcn_ballot_w64(!(a0 <= tc_xmax)) == 0) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float x = sacc[kb][r], t = x * x;
                        sacc[kb][r] = __builtin_fmaf(
                            x, __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(tc3, t, tc2), t, tc1), t, tc0), zoff);
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        // cap - 2 cap / (exp(2 x / cap) + 1)
                        const float e = fast_exp2(sacc[kb][r] * cap_in);
                        sacc[kb][r] = __builtin_fmaf(-2.f * cap_l2, fast_rcp(e + 1.f), cap_l2 + zoff);
                    }
            }
        }
        // ALiBi: the bias slope (j - row) = slope jc + slope (j0 + 4 hh - row)
        // with jc = 32 kb + 8 (r / 4) + r % 4 (key within tile less the lane's
        // 4 hh): the first part is added here, one FMA with a literal per
        // score; the second, the same for all scores of the lane, is folded
        // into the row max and the exponent reference (alibi_lane).
        // The same pass on every tile, then the element mask on partial ones,
        // both in place (separate full / partial versions of the first pass
        // made the compiler merge their results through register copies).
        if (MODS) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if ((r & 3) == 0) pin(sacc[kb]);   // four elements at a time
                    const int jc = 32 * kb + 8 * (r >> 2) + (r & 3);
                    const float x = sacc[kb][r];
                    float y = SOFTCAP ? x : __builtin_fmaf(x, c, zoff);
                    if (ALIBI && jc != 0) y = __builtin_fmaf((float)jc, slope_l2, y);
                    sacc[kb][r] = y;
                }
        }
        if (!full) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int jl = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);   // key within tile
                    if ((r & 3) == 0) pin(sacc[kb]);
                    const float y = MODS ? sacc[kb][r] : sacc[kb][r] * c;
                    bool ok = jl <= jl_hi && jl >= jl_lo;
                    if (DOC) ok &= dk[kb][r] == doc_i;
                    sacc[kb][r] = ok ? y : -INFINITY;
                }
        } else if (!MODS) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    if ((r & 3) == 0) pin(sacc[kb]);
                    sacc[kb][r] *= c;
                }
        }
    };

    float rescale_by = 1.f;      // output factor of the last softmax (1 for most rows)
    bool rescale_any = false;    // some row of the wave needs it
    // Online softmax of tile kt: scores -> P, running max / sum. Plain full
    // tiles keep raw scores (scale folded into the exponent FMA).
    auto softmax = [&](int kt, const ATTN_LDS int* dl) __attribute__((always_inline)) {
        const bool full = is_full(kt, dl);
        const bool pre = MODS || !full || !(c > 0.f);
        float ls0 = -0.f, ls1 = -0.f, ls2 = -0.f, ls3 = -0.f;   // -0 + p folds to p
        auto exps = [&](auto arg) __attribute__((always_inline)) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float p0 = fast_exp2(arg(sacc[kb][r]));
                    const float p1 = fast_exp2(arg(sacc[kb][r + 1]));
                    if (r & 2) { ls2 += p0; ls3 += p1; } else { ls0 += p0; ls1 += p1; }
                    pf[kb][r >> 3][(r & 7)] = (__bf16)p0;
                    pf[kb][r >> 3][(r & 7) + 1] = (__bf16)p1;
                }
        };
        // lane part of the ALiBi bias (see prepare_scores), 0 without ALiBi
        const float alibi_lane = ALIBI ? slope_l2 * (float)(kt * BN + 4 * hh - row) : 0.f;
        // With score modifiers, once every row of the wave has a reference the
        // scores are prepared relative to it (the modifier's last FMA adds
        // alibi_lane - m), so that the exponent needs no argument instruction
        // on tiles where no row's reference moves.
        const bool rel = MODS && __builtin_amdgcn_ballot_w64(!(m > kNoMax)) == 0;
        if (__builtin_expect(pre, MODS)) prepare_scores(full, kt, dl, rel ? alibi_lane - m : 0.f);
        const float ce = pre ? 1.f : c;
        // The exponents against the current references first. When no partial
        // sum of p exceeds kSpecSumLimit, no row's reference would move and
        // these are the values the pass with the tile's row max gives, without
        // that pass; otherwise (the first tile of a row too, its reference
        // still kNoMax) that pass recomputes the tile.
        if (rel) {
            exps([](float x) __attribute__((always_inline)) { return x; });
        } else {
            const float mneg0 = alibi_lane - m;
            exps([&](float x) __attribute__((always_inline)) { return __builtin_fmaf(x, ce, mneg0); });
        }
        bool need = false;
        float alpha = 1.f;
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(max2(max3(ls0, ls1, ls2), ls3) <= kSpecSumLimit)) != 0, 0)) {
            ls0 = ls1 = ls2 = ls3 = -0.f;
            float a0 = max3(sacc[0][0], sacc[0][1], sacc[0][2]), a1 = max3(sacc[1][0], sacc[1][1], sacc[1][2]);
#pragma unroll
            for (int r = 3; r < 15; r += 2) {
                a0 = max3(a0, sacc[0][r], sacc[0][r + 1]);
                a1 = max3(a1, sacc[1][r], sacc[1][r + 1]);
            }
            a0 = max3(a0, sacc[0][15], max2(a1, sacc[1][15]));
            float ce2, mneg;   // p = exp2(s ce2 + mneg)
            if (rel) {
                const float mx = xhalf_max(a0);   // the tile's max over the reference
                need = mx > kLazyTau;
                alpha = need ? fast_exp2(-mx) : 1.f;
                m = need ? m + mx : m;
                ce2 = 1.f;
                mneg = need ? -mx : 0.f;
            } else {
                const float mx = xhalf_max(a0 + alibi_lane) * ce;
                const float mn = max2(m, mx);
                need = mn > m + kLazyTau;
                alpha = need ? fast_exp2(m - mn) : 1.f;
                m = need ? mn : m;
                ce2 = ce;
                mneg = alibi_lane - m;
            }
            // relative scores and no reference moved: the exponent of the score itself
            const bool plain = rel && __builtin_amdgcn_ballot_w64(need) == 0;
            if (plain)
                exps([](float x) __attribute__((always_inline)) { return x; });
            else
                exps([&](float x) __attribute__((always_inline)) { return __builtin_fmaf(x, ce2, mneg); });
        }
        // P is complete here; GEMM1 reads it only after the wait states below
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            pin(pf[kb][0]);
            pin(pf[kb][1]);
        }
        l = l * alpha + ((ls0 + ls1) + (ls2 + ls3));
        // take the sums here, while the other wave of the SIMD is in its matrix
        // phase (left alone, the compiler sinks them below GEMM0, onto the
        // path to the next barrier)
        pin(l);
        rescale_by = alpha;
        rescale_any = __builtin_amdgcn_ballot_w64(need) != 0;
        if (__builtin_expect(rescale_any, 0)) {   // rare: the reference max moved
            mfma_guard();
#pragma unroll
            for (int t = 0; t < DT; ++t) {
                // one output tile at a time through VGPRs
                pin_a(o[t]);
                f32x16 x = o[t];
                pin(x);
                x *= rescale_by;
                o[t] = x;
                pin_a(o[t]);
            }
            mfma_guard();
        }
    };

    Copy copy;
    copy.init(wave, lane);
    auto tile_k = [&](int i) __attribute__((always_inline)) {
        copy.template issue<false>(K, ktile(i) * BN, Nk, lds_addr(kbuf(i)), wave);
    };
    auto tile_v = [&](int i) __attribute__((always_inline)) {
        copy.template issue<true>(V, ktile(i) * BN, Nk, lds_addr(vbuf(i)), wave);
        if (DOC) issue_docs(docrow, ktile(i) * BN, Nk, lds_addr(dbuf(i)), wave, lane);
    };

    // ---------------------------------------------------------------- ping-pong loops
    // Barrier i (i >= 1) is passed by group B at the top of iteration i - 1,
    // by group A between its softmax and GEMM1 of tile i - 1: on each SIMD one
    // wave's products (GEMM1 of tile i - 1, GEMM0 of tile i) then overlap the
    // other wave's softmax. Before the barrier each wave waits for its copies
    // of tile i only (up to PF - 1 later tiles may stay in flight); after it,
    // it issues its share of tile i + PF. Between barriers i and i + 1 the
    // waves read K(i), V(i - 1), the document ids of tiles i - 1 and i, and
    // refill K(i - 1), V(i - 2): never a buffer being read.
    auto copies = [&](int i) __attribute__((always_inline)) {
        if (A_ONLY && group_b) return;
        if (i + PF < n_tiles) {
            tile_k(i + PF);
            tile_v(i + PF);
#ifdef ATTN_SINGLE_STAGE
            __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
#endif
        }
    };
    auto barrier_and_copy = [&](int i, bool copy = true) __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        static_assert((PF - 1) * LOADS_PER_TILE <= 15, "vmcnt immediate");
        const int ahead = min(PF - 1, n_tiles - 1 - i);   // later tiles whose copies may stay in flight
        if (PF >= 3 && ahead >= 2) __builtin_amdgcn_s_waitcnt(0x0070 | (2 * LOADS_PER_TILE));
        else if (PF >= 2 && ahead >= 1) __builtin_amdgcn_s_waitcnt(0x0070 | LOADS_PER_TILE);
        else __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (copy) copies(i);
    };
    // Copies of tile i + PF may go out anywhere between barriers i and i + 1.
    // Issued by all waves right after the barrier they queue up behind each
    // other (the CU's vector-memory path drains about 64 bytes per cycle) and
    // hold every wave; in the kernels without score modifiers they go out at
    // the end of the interval instead. (The modifier kernels run out of
    // registers with the copies there.)
    constexpr bool LATE_A = ATTN_LATE_COPY_A && !MODS, LATE_B = ATTN_LATE_COPY_B && !MODS;
    // Iteration it over a tile of this wave's key range: softmax and GEMM1 of
    // tile it, GEMM0 of tile it + 1 (when it is also in the range).
    auto body = [&](int it, bool next) __attribute__((always_inline)) {
        const int kt = ktile(it);
        if (group_b) barrier_and_copy(it + 1, !LATE_B);
        softmax(kt, dbuf(it));
        if (!group_b) barrier_and_copy(it + 1, !LATE_A);
        operand_guard();   // P was written by vector code just before
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            pin(pf[kb][0]);
            pin(pf[kb][1]);
        }
        gemm1(vbuf(it));
        if (next) gemm0(kbuf(it + 1));
        if (group_b ? LATE_B : LATE_A) copies(it + 1);
    };

    // this wave's tiles: [wb, we) relative to kt_begin
    int wb = n_tiles, we = n_tiles;
    if (wt_end > wt_begin) {
        wb = rev ? kt_begin + n_tiles - wt_end : wt_begin - kt_begin;
        we = rev ? kt_begin + n_tiles - wt_begin : wt_end - kt_begin;
    }
    if (n_tiles > 0) {
#pragma unroll
        for (int i = 0; i < PF; ++i)
            if (i < n_tiles && !(A_ONLY && group_b)) {
                tile_k(i);
                tile_v(i);
            }
        barrier_and_copy(0);
    }
    int it = 0;
    if (wb < we) {
        if (wb == 0) gemm0(kbuf(0));
        for (; it < wb; ++it) {   // before the range: barriers and copies only
            barrier_and_copy(it + 1);
            if (it + 1 == wb) gemm0(kbuf(wb));
        }
        for (; it < we - 1; ++it) body(it, true);
        body(it, false);
        ++it;
    }
    for (; it < n_tiles; ++it) barrier_and_copy(it + 1);   // after the range

    // ---- epilogue: O / l, LSE = (m + log2 l) ln 2
    if (!wave_active) return;
    mfma_guard();
#pragma unroll
    for (int t = 0; t < DT; ++t) pin_a(o[t]);
    __bf16* O = (__bf16*)p.o + qbase * D;
    const float lt = xhalf_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    // The output goes to HBM through this wave's own half of a tile buffer:
    // in registers each lane holds a quarter-row of d values (4 of every 8),
    // which stored directly writes 16-byte pieces of 32 rows per instruction;
    // read back row-wise, each store writes whole contiguous rows (the wave's
    // 32 rows are one contiguous block of O). After the last barrier no wave
    // reads the key buffers or any value buffer but the last tile's.
    static_assert(2 * 32 * T::ROW_BYTES <= T::BYTES && NKB + NVB - 1 >= NW / 2, "output staging space");
    int sbuf = wave / 2;
    if (n_tiles > 0 && sbuf >= NKB + (n_tiles - 1) % NVB) ++sbuf;
    ATTN_LDS char* stage = lds + sbuf * T::BYTES + (wave & 1) * (32 * T::ROW_BYTES);
    // In a persistent workgroup the lane-only offsets are computed here, not
    // hoisted out of its item loop (where they would be kept in scratch).
    int ln = lane;
    if (PERSIST) pin(ln);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[t][4 * gq + e] * inv);
            // d = 32 t + 8 gq + 4 hh + e: chunk 4 t + gq of row l32, bytes 8 hh ..
            const int r = ln & 31;
            const int ch = (4 * t + gq) ^ T::swz_k(r);
            *(ATTN_LDS bf16x4*)(stage + r * T::ROW_BYTES + ch * 16 + 8 * (ln >> 5)) = w;
        }
    asm volatile("" ::: "memory");
    {
        constexpr int RPI = 64 / T::CPR;   // rows per 16-byte-per-lane instruction
        const int rr = ln / T::CPR, cc = ln % T::CPR;
#pragma unroll
        for (int k = 0; k < 32 / RPI; ++k) {
            const int r = k * RPI + rr;
            const bf16x8 x = *(const ATTN_LDS bf16x8*)(stage + r * T::ROW_BYTES + ((cc ^ T::swz_k(r)) * 16));
            if (wq0 + r < Nq) *(bf16x8*)(O + (size_t)(wq0 + r) * D + cc * 8) = x;
        }
    }
    if (row < Nq && p.lse && hh == 0)
        p.lse[qbase + row] = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
}

// One workgroup per work item (the grid is every item of the launch).
template <int D, bool SOFTCAP, bool ALIBI, bool DOC>
__global__ __launch_bounds__(512) void fwd_bf16_kernel(FwdParams p) {
    __shared__ Bf16Lds<D, DOC> sm;
    fwd_bf16_item<D, SOFTCAP, ALIBI, DOC>(p, blockIdx.x, sm);
}

// Persistent form: a grid of as many workgroups as are resident at once, each
// walking the items w, w + G, w + 2G, ... of the same heavy-first, XCD-grouped
// order (a static schedule, no atomics); a barrier separates consecutive items
// so no wave refills LDS buffers another wave still reads.
template <int D, bool SOFTCAP, bool ALIBI, bool DOC>
__global__ __launch_bounds__(512) void fwd_bf16_persistent_kernel(FwdParams p) {
    __shared__ Bf16Lds<D, DOC> sm;
    const int n_items = p.n_qt * p.n_bh, G = gridDim.x, w = blockIdx.x;
    // Snake order: in odd rounds the items are taken in reverse within this
    // workgroup's XCD class (w % 8; item r G + j runs on XCD j % 8 as in the
    // plain launch), so a workgroup that took a heavy item takes a light one
    // next and the workgroups' totals stay close.
    const bool snake = G % 8 == 0;
    for (int r = 0; r * G < n_items; ++r) {
        const int j = (snake && (r & 1)) ? (G / 8 - 1 - w / 8) * 8 + w % 8 : w;
        const int wid = r * G + j;
        if (wid >= n_items) continue;
        fwd_bf16_item<D, SOFTCAP, ALIBI, DOC, true>(p, wid, sm);
        __syncthreads();
    }
}

// -----------------------------------------------------------------------------
// The forward's own tile schedule, written out for inspection: for every
// block of 32 query rows (one wave of the forward) and every 64-key tile,
// 0 = empty (skipped), 1 = partial (element mask), 2 = full (no mask code),
// from the same range and full-tile functions the forward kernel calls. One
// wave per (batch row, row block).
template <bool DOC>
__global__ __launch_bounds__(64) void fwd_plan_kernel(int Nq, int Nk, int mask, int W, const int32_t* doc,
                                                      int n_rb, int n_kt, int8_t* kinds) {
    const int b = blockIdx.x / n_rb, rb = blockIdx.x % n_rb, lane = threadIdx.x;
    const int r0 = rb * 32, r1 = min(r0 + 32, Nq) - 1, off = Nk - Nq;
    const int32_t* docrow = DOC ? doc + (size_t)b * Nk : nullptr;
    const KeyRange kr = rows_key_range<DOC>(r0, r1, Nk, off, mask, W, docrow, lane);
    const int t0 = kr.hi > kr.lo ? kr.lo / BN : 0, t1 = kr.hi > kr.lo ? (kr.hi + BN - 1) / BN : 0;
    int8_t* out = kinds + ((size_t)b * n_rb + rb) * n_kt;
    for (int kt = lane; kt < n_kt; kt += 64) {
        int kind = 0;
        if (kt >= t0 && kt < t1) {
            const int j0 = kt * BN, j1 = min(j0 + BN, Nk) - 1;
            kind = tile_full<DOC>(j0, Nk, r0, r1, off, mask, W, kr, DOC ? docrow[j0] : 0, DOC ? docrow[j1] : 0)
                       ? 2 : 1;
        }
        out[kt] = (int8_t)kind;
    }
}

hipError_t launch_fwd_plan(int B, int Nq, int Nk, int mask, int window, const int32_t* doc, int8_t* kinds,
                           hipStream_t st) {
    const int n_rb = (Nq + 31) / 32, n_kt = (Nk + BN - 1) / BN;
    const long long grid = (long long)B * n_rb;
    if (grid > INT_MAX) return hipErrorInvalidValue;
    if (mask & kMaskDoc)
        hipLaunchKernelGGL(fwd_plan_kernel<true>, dim3((unsigned)grid), dim3(64), 0, st, Nq, Nk, mask, window,
                           doc, n_rb, n_kt, kinds);
    else
        hipLaunchKernelGGL(fwd_plan_kernel<false>, dim3((unsigned)grid), dim3(64), 0, st, Nq, Nk, mask, window,
                           doc, n_rb, n_kt, kinds);
    return hipGetLastError();
}

// -----------------------------------------------------------------------------
// ATTN_PERSISTENT=1 (read once) selects the persistent form of the bf16
// forward, for comparing the two launch forms; results are identical.
static bool persistent_launch() {
    static const bool on = [] {
        const char* e = std::getenv("ATTN_PERSISTENT");
        return e && e[0] && e[0] != '0';
    }();
    return on;
}

// Compute units of the current device (one resident workgroup each).
static int resident_workgroups() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
        n = 256;
    return n;
}

template <int D, bool SC, bool AL, bool DC>
static hipError_t launch_bf16_inst(const FwdParams& p0, hipStream_t st) {
    FwdParams p = p0;
    constexpr int BM = 256;
    p.n_qt = p.items ? p.n_list : (p.Nq + BM - 1) / BM;
    p.n_bh = p.B * p.Hq;
    // Head groups per XCD: as many heads as fill two rounds of its resident
    // workgroups (32 CUs, one workgroup each; one round measured slower),
    // when the heads split evenly over the 8 XCDs and into groups of at
    // least two. With one head per group (long sequences) the plain order
    // measured faster.
    p.xgrp = 0;
    if (p.n_bh % 8 == 0) {
        const int per_xcd = p.n_bh / 8;
        int g = 64 / p.n_qt;
        while (g > 1 && per_xcd % g) --g;
        p.xgrp = g >= 2 ? g : 0;
    }
    const int n_items = p.n_qt * p.n_bh;
    if (persistent_launch()) {
        // one workgroup per CU is resident (the LDS holds one workgroup's buffers)
        const int grid = n_items < resident_workgroups() ? n_items : resident_workgroups();
        hipLaunchKernelGGL((fwd_bf16_persistent_kernel<D, SC, AL, DC>), dim3(grid), dim3(512), 0, st, p);
    } else {
        hipLaunchKernelGGL((fwd_bf16_kernel<D, SC, AL, DC>), dim3(n_items), dim3(512), 0, st, p);
    }
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bf16_d(const FwdParams& p, hipStream_t st) {
    const bool sc = p.softcap > 0.f, al = p.slopes != nullptr, dc = (p.mask & kMaskDoc) != 0;
    if (!sc && !al && !dc) return launch_bf16_inst<D, false, false, false>(p, st);
    if (!sc && !al && dc) return launch_bf16_inst<D, false, false, true>(p, st);
    if (sc && al && dc) return launch_bf16_inst<D, true, true, true>(p, st);
    if (sc && !al && !dc) return launch_bf16_inst<D, true, false, false>(p, st);
    if (!sc && al && !dc) return launch_bf16_inst<D, false, true, false>(p, st);
    if (sc && al && !dc) return launch_bf16_inst<D, true, true, false>(p, st);
    if (sc && !al && dc) return launch_bf16_inst<D, true, false, true>(p, st);
    return launch_bf16_inst<D, false, true, true>(p, st);
}

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t st) {
    if (d == 128) return launch_bf16_d<128>(p, st);
    return launch_bf16_d<64>(p, st);
}

}  // namespace attn
