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
// result is unchanged because O / l and the LSE use the same reference.
//
// Tiles are classified per wave as empty (outside the wave's contiguous key
// range, skipped), partial (element mask) or full (no mask code): closed form
// for causal / window, from the tile's first / last document id for packed
// documents.
#include <climits>
#include <type_traits>

#include "fwd_common.h"

#ifndef ATTN_PREFETCH
#define ATTN_PREFETCH 2   // key/value tiles in flight ahead of the matrix work (1..3)
#endif

namespace attn {

constexpr float kLazyTau = 8.f;   // log2 units: rescale O only when the max grows by > 2^8

template <int D, bool SOFTCAP, bool ALIBI, bool DOC>
__global__ __launch_bounds__(512) void fwd_bf16_kernel(FwdParams p) {
    using T = Tile<D>;
    constexpr int NW = 8;        // waves: 4 in group A, 4 in group B
    constexpr int BM = NW * 32;
    constexpr int DS = D / 16;   // GEMM0 k-steps
    constexpr int DT = D / 32;   // output d-subtiles
    constexpr bool MODS = SOFTCAP || ALIBI;
    // Copies run PF tiles ahead of the matrix work; key tiles need PF + 1
    // buffers, value tiles (read during two consecutive intervals) PF + 2.
    constexpr int PF = ATTN_PREFETCH;
    static_assert(PF >= 1 && PF <= 2, "prefetch distance 1 or 2");
    constexpr int NKB = PF + 1, NVB = PF + 2;
    using Copy = TileCopy<D, NW>;
    constexpr int LOADS_PER_TILE = 2 * Copy::ROUNDS + (DOC ? 1 : 0);   // per wave

    __shared__ __attribute__((aligned(1024))) char tiles_lds[(NKB + NVB) * T::BYTES];
    __shared__ __attribute__((aligned(16))) int docs_lds[DOC ? NVB * NW * BN : 4];
    __shared__ int range_lds[NW][2];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool group_b = wave >= NW / 2;
    const int l32 = lane & 31, hh = lane >> 5;

    // ---- work item: heavy (late) query tiles first for causal balance
    const int wid = blockIdx.x;
    const int qt = p.n_qt - 1 - wid / p.n_bh;
    const int bh = wid % p.n_bh;
    const int b = bh / p.Hq, h = bh % p.Hq, g = h / p.group;
    const int Nq = p.Nq, Nk = p.Nk, off = Nk - Nq;
    const bool causal = p.mask & kMaskCausal, windowed = p.mask & kMaskWindow;
    const int W = p.window;
    const int q0 = qt * BM;

    const __bf16* Q = (const __bf16*)p.q + (size_t)(b * p.Hq + h) * Nq * D;
    const __bf16* K = (const __bf16*)p.k + (size_t)(b * p.Hkv + g) * Nk * D;
    const __bf16* V = (const __bf16*)p.v + (size_t)(b * p.Hkv + g) * Nk * D;
    const int32_t* docrow = DOC ? p.doc + (size_t)b * Nk : nullptr;

    // ---- this wave's rows and its contiguous key range [w_lo, w_hi)
    const int wq0 = q0 + wave * 32;
    const bool wave_active = wq0 < Nq;
    const int wq1 = min(wq0 + 32, Nq) - 1;
    int w_lo = INT_MAX, w_hi = INT_MIN;
    int dq0 = 0, dq1 = 0;
    if (wave_active) {
        w_lo = 0;
        w_hi = Nk;
        if (causal) w_hi = min(w_hi, wq1 + off + 1);
        if (windowed) w_lo = max(w_lo, wq0 + off - W + 1);
        if (DOC) {
            dq0 = docrow[wq0];
            dq1 = docrow[wq1];
            w_lo = max(w_lo, wave_search<false>(docrow, Nk, dq0, lane));
            w_hi = min(w_hi, wave_search<true>(docrow, Nk, dq1, lane));
        }
        if (w_hi <= w_lo) { w_lo = INT_MAX; w_hi = INT_MIN; }
    }
    if (lane == 0) { range_lds[wave][0] = w_lo; range_lds[wave][1] = w_hi; }
    __syncthreads();
    int kv_lo = INT_MAX, kv_hi = INT_MIN;
#pragma unroll
    for (int w = 0; w < NW; ++w) { kv_lo = min(kv_lo, range_lds[w][0]); kv_hi = max(kv_hi, range_lds[w][1]); }
    const int kt_begin = kv_hi > kv_lo ? kv_lo / BN : 0;
    const int n_tiles = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN - kt_begin : 0;
    const int wt_begin = w_hi > w_lo ? w_lo / BN : 0;
    const int wt_end = w_hi > w_lo ? (w_hi + BN - 1) / BN : 0;

    const int row = wq0 + l32;
    const int doc_i = DOC ? docrow[min(row, Nq - 1)] : 0;
    const float c = p.scale_log2;
    const float slope_l2 = ALIBI ? p.slopes[h] * kLog2e : 0.f;
    const float cap_l2 = SOFTCAP ? p.softcap * kLog2e : 0.f;        // cap in exp2 units
    const float cap_in = SOFTCAP ? p.scale * 2.f * kLog2e / p.softcap : 0.f;

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
    float m = -INFINITY, l = 0.f;

    // ---- lane-constant LDS offsets. With both swizzles, the offset of K-read
    // step s is koff0 ^ (32 s) and of V d-subtile t is voff0 ^ (64 t): one base
    // register each.
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

    ATTN_LDS char* lds = (ATTN_LDS char*)tiles_lds;
    auto kbuf = [&](int i) __attribute__((always_inline)) { return lds + (i % NKB) * T::BYTES; };
    auto vbuf = [&](int i) __attribute__((always_inline)) { return lds + (NKB + i % NVB) * T::BYTES; };
    auto dbuf = [&](int i) __attribute__((always_inline)) {
        return (ATTN_LDS int*)docs_lds + (i % NVB) * (NW * BN);
    };

    // ---------------------------------------------------------------- stages
    f32x16 sacc[2];
    // Matrix phases keep at most two fragments in flight: the instruction
    // groups below order them as read, read, then (mfma, read) pairs.
    auto gemm0 = [&](const ATTN_LDS char* kl) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s = 0; s < DS; ++s) {
                const bf16x8 kf = *(const ATTN_LDS bf16x8*)(kl + (koff0 ^ (32 * s)) + kb * 32 * T::ROW_BYTES);
                sacc[kb] = mfma_bf16(kf, qf[s], s == 0 ? f32x16{} : sacc[kb]);
            }
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < 2 * DS - 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    auto is_full = [&](int kt, const ATTN_LDS int* dl) __attribute__((always_inline)) -> bool {
        const int j0 = kt * BN;
        const int j1 = min(j0 + BN, Nk) - 1;
        bool full = j0 + BN <= Nk;
        if (causal) full &= j1 <= wq0 + off;
        if (windowed) full &= (wq1 + off) - j0 < W;
        if (DOC) {
            const int dj0 = dl[wave * BN], dj1 = dl[wave * BN + (j1 - j0)];
            full &= dj0 == dj1 && dq0 == dq1 && dj0 == dq0;
        }
        return full;
    };

    bf16x8 pf[2][2];
    float rescale_by = 1.f;      // output factor of the last softmax (1 for most rows)
    bool rescale_any = false;    // some row of the wave needs it
    // Online-softmax update shared by both softmax variants: new reference max,
    // rescale factor, then p = exp2(y - m) into bf16 P and the running sum. The
    // reference only moves when the row max grew by more than 2^kLazyTau.
    auto finish = [&](float mx, auto&& ys) __attribute__((always_inline)) {
        const float mold = m;
        const float mn = fmaxf(mold, mx);
        const bool upd = mold == -INFINITY || mn > mold + kLazyTau;
        const float mref = mn == -INFINITY ? 0.f : mn;
        const float alpha = upd ? fast_exp2(mold - mref) : 1.f;
        const bool need = upd && mold != -INFINITY;
        m = upd ? mn : mold;
        const float mu = m == -INFINITY ? 0.f : m;
        float ls0 = 0.f, ls1 = 0.f, ls2 = 0.f, ls3 = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float p0 = fast_exp2(ys(kb, r, mu)), p1 = fast_exp2(ys(kb, r + 1, mu));
                if (r & 2) { ls2 += p0; ls3 += p1; } else { ls0 += p0; ls1 += p1; }
                pf[kb][r >> 3][(r & 7)] = (__bf16)p0;
                pf[kb][r >> 3][(r & 7) + 1] = (__bf16)p1;
            }
        l = l * alpha + ((ls0 + ls1) + (ls2 + ls3));
        rescale_by = need ? alpha : 1.f;
        rescale_any = __builtin_amdgcn_ballot_w64(need) != 0;
    };

    // Full tile, no score modifier: the max is taken on raw q.k and the scale
    // is folded into the exponent argument, one FMA per score.
    auto softmax_plain = [&]() __attribute__((always_inline)) {
        float a0 = max3(sacc[0][0], sacc[0][1], sacc[0][2]), a1 = max3(sacc[1][0], sacc[1][1], sacc[1][2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) {
            a0 = max3(a0, sacc[0][r], sacc[0][r + 1]);
            a1 = max3(a1, sacc[1][r], sacc[1][r + 1]);
        }
        a0 = max3(a0, sacc[0][15], a1);
        const float mx = xhalf_max(fmaxf(a0, sacc[1][15])) * c;
        finish(mx, [&](int kb, int r, float mu) __attribute__((always_inline)) {
            return __builtin_fmaf(sacc[kb][r], c, -mu);
        });
    };

    // Score modifiers and / or the element mask (partial tiles): the modified
    // score in exp2 units replaces the raw one, masked entries become -inf.
    auto softmax_general = [&](bool full, int kt, const ATTN_LDS int* dl) __attribute__((always_inline)) {
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
        const bool mask_doc = DOC && !full;
        float a0 = -INFINITY, a1 = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int jl = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);   // key within tile
                float y;
                if (SOFTCAP) {
                    // cap * tanh(x / cap) = cap - 2 cap / (exp(2 x / cap) + 1), in exp2 units
                    const float e = fast_exp2(sacc[kb][r] * cap_in);
                    y = cap_l2 - 2.f * cap_l2 * fast_rcp(e + 1.f);
                } else {
                    y = sacc[kb][r] * c;
                }
                if (ALIBI) y -= slope_l2 * (float)(row - (j0 + jl));
                bool ok = jl <= jl_hi && jl >= jl_lo;
                if (DOC) ok &= !mask_doc || dk[kb][r] == doc_i;
                y = ok ? y : -INFINITY;
                sacc[kb][r] = y;
                if (kb == 0) a0 = fmaxf(a0, y); else a1 = fmaxf(a1, y);
            }
        }
        const float mx = xhalf_max(fmaxf(a0, a1));
        finish(mx, [&](int kb, int r, float mu) __attribute__((always_inline)) { return sacc[kb][r] - mu; });
    };

    auto softmax = [&](bool full, int kt, const ATTN_LDS int* dl) __attribute__((always_inline)) {
        if (!MODS && full) softmax_plain();
        else softmax_general(full, kt, dl);
    };


    auto gemm1 = [&](const ATTN_LDS char* vl) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    const int base = (32 * kb + 16 * u) * T::ROW_BYTES + (voff0 ^ (64 * t));
                    const bf16x4 lo4 =
                        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4*)(vl + base));
                    const bf16x4 hi4 =
                        __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4*)(vl + base + 8 * T::ROW_BYTES));
                    const bf16x8 vf = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
                    o[t] = mfma_bf16(vf, pf[kb][u], o[t]);
                }
        constexpr int NM = 4 * DT;   // matrix instructions in this phase
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < NM - 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_barrier(0);
    };

    auto in_w = [&](int kt) __attribute__((always_inline)) { return kt >= wt_begin && kt < wt_end; };
    Copy copy;
    copy.init(wave, lane);
    auto tile_k = [&](int i) __attribute__((always_inline)) {
        copy.template issue<false>(K, (kt_begin + i) * BN, Nk, lds_addr(kbuf(i)), wave);
    };
    auto tile_v = [&](int i) __attribute__((always_inline)) {
        copy.template issue<true>(V, (kt_begin + i) * BN, Nk, lds_addr(vbuf(i)), wave);
        if (DOC) issue_docs(docrow, (kt_begin + i) * BN, Nk, lds_addr(dbuf(i)), wave, lane);
    };

    // ---------------------------------------------------------------- ping-pong loop
    // Barrier i (i >= 1) is passed by group B at the top of body(i - 1) and by
    // group A in the middle of body(i - 1). Before it, each wave waits for its
    // copies of tile i only (tile i + 1 may still be in flight when PF = 2);
    // after it, it issues its share of tile i + PF. Between barriers i and i + 1
    // the waves read K(i), V(i - 1) and V(i), never a buffer being refilled.
    auto barrier_and_copy = [&](int i) __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        if (PF >= 2 && i + 1 < n_tiles) __builtin_amdgcn_s_waitcnt(0x0070 | LOADS_PER_TILE);
        else __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (i + PF < n_tiles) {
            tile_k(i + PF);
            tile_v(i + PF);
        }
    };
    if (n_tiles > 0) {
#pragma unroll
        for (int i = 0; i < PF; ++i)
            if (i < n_tiles) {
                tile_k(i);
                tile_v(i);
            }
        barrier_and_copy(0);
        if (in_w(kt_begin)) gemm0(kbuf(0));
    }

    for (int it = 0; it < n_tiles; ++it) {
        const int kt = kt_begin + it;
        if (group_b) barrier_and_copy(it + 1);
        if (in_w(kt)) {
            softmax(is_full(kt, dbuf(it)), kt, dbuf(it));
            if (__builtin_expect(rescale_any, 0)) {   // rare: the reference max moved
#pragma unroll
                for (int t = 0; t < DT; ++t) o[t] *= rescale_by;
            }
            gemm1(vbuf(it));
        }
        if (!group_b) barrier_and_copy(it + 1);
        if (it + 1 < n_tiles && in_w(kt + 1)) gemm0(kbuf(it + 1));
    }

    // ---- epilogue: O / l, LSE = (m + log2 l) ln 2
    if (!wave_active) return;
    __bf16* O = (__bf16*)p.o + (size_t)(b * p.Hq + h) * Nq * D;
    const float lt = xhalf_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (row < Nq) {
        __bf16* orow = O + (size_t)row * D + 4 * hh;
#pragma unroll
        for (int t = 0; t < DT; ++t)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                bf16x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[t][4 * gq + e] * inv);
                *(bf16x4*)(orow + 32 * t + 8 * gq) = w;
            }
        if (p.lse && hh == 0)
            p.lse[(size_t)(b * p.Hq + h) * Nq + row] = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    }
}

// -----------------------------------------------------------------------------
template <int D, bool SC, bool AL, bool DC>
static hipError_t launch_bf16_inst(const FwdParams& p0, hipStream_t st) {
    FwdParams p = p0;
    constexpr int BM = 256;
    p.n_qt = (p.Nq + BM - 1) / BM;
    p.n_bh = p.B * p.Hq;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, SC, AL, DC>), dim3(p.n_qt * p.n_bh), dim3(512), 0, st, p);
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
