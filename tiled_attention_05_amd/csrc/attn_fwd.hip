// Fused attention forward for gfx950 (bf16 and fp32 inputs).
//
// One workgroup computes a BM-row query tile of one (batch, query head). Key /
// value tiles of BN = 64 rows stream HBM -> LDS with direct global->LDS copies
// into a double buffer while the previous tile is being multiplied; the score
// tile lives only in registers and the output is rescaled on chip, so no
// score matrix is ever written to device memory ("Les kernels d'attention
// rapide et la fusion d'operateurs ...", section "Attention de type
// FlashAttention et attention paginee"; "FlashAttention-3 : ...", section
// "Rappel du fonctionnement de FlashAttention").
//
// Matrix-core formulation (CDNA4 32x32 MFMA, 64-wide waves):
//   GEMM0  S^T = K Q^T   A = K rows from LDS, B = Q rows kept in registers.
//          The accumulator puts one query per lane (lane & 31) and 16 keys per
//          lane, so the row max / row sum are in-lane reductions plus one
//          exchange between the two half-waves.
//   GEMM1  O^T = V^T P^T A = V read transposed from LDS (ds_read_b64_tr_b16),
//          B = P straight from the GEMM0 accumulator registers (bf16). The
//          output accumulator again holds one query per lane, so the per-row
//          rescale factor is a per-lane scalar.
// Each wave owns QB blocks of 32 query rows, so every K / V fragment read from
// LDS feeds QB MFMAs (halves LDS traffic per FLOP at QB = 2).
//
// Softmax: exp2 with scale * log2(e) folded into one FMA per score, running
// max / running sum per row, a single division at the end (the non-matmul
// work reduction of "FlashAttention-2 (FR)", section "Architecture technique",
// item 1). Tiles are classified per wave as empty (skipped), partial (element
// mask) or full (no mask code), closed-form for causal / window and from the
// tile's first / last document id for packed documents.
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

template <int D, int NW, bool DOC>
__device__ __forceinline__ void issue_tile(const __bf16* K, const __bf16* V, const int32_t* docrow,
                                           int kv0, int Nk, ATTN_LDS char* kl, ATTN_LDS char* vl,
                                           ATTN_LDS int* dl, int wave, int lane) {
    using T = Tile<D>;
    constexpr int ROUNDS = BN * T::CPR / (NW * 64);
    static_assert(ROUNDS * NW * 64 == BN * T::CPR, "tile must split evenly over the waves");
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
        const int s = (rd * NW + wave) * 64 + lane;
        const int row = s / T::CPR, pc = s % T::CPR;
        const int grow = min(kv0 + row, Nk - 1);   // rows past Nk: any finite row, masked later
        load_lds16(K + (size_t)grow * D + (pc ^ T::swz_k(row)) * 8, kl + (rd * NW + wave) * 1024);
        load_lds16(V + (size_t)grow * D + (pc ^ T::swz_v(row)) * 8, vl + (rd * NW + wave) * 1024);
    }
    if (DOC) load_lds4(docrow + min(kv0 + lane, Nk - 1), dl + wave * BN);
}

template <int D, int QB, int NW, bool SOFTCAP, bool ALIBI, bool DOC>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdParams p) {
    using T = Tile<D>;
    constexpr int BM = NW * QB * 32;
    constexpr int DS = D / 16;   // GEMM0 k-steps
    constexpr int DT = D / 32;   // output d-subtiles

    __shared__ __attribute__((aligned(1024))) char k_lds0[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char k_lds1[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char v_lds0[T::BYTES];
    __shared__ __attribute__((aligned(1024))) char v_lds1[T::BYTES];
    __shared__ __attribute__((aligned(16))) int d_lds0[DOC ? NW * BN : 4];
    __shared__ __attribute__((aligned(16))) int d_lds1[DOC ? NW * BN : 4];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    const int qlast = min(q0 + BM, Nq) - 1;

    const __bf16* Q = (const __bf16*)p.q + (size_t)(b * p.Hq + h) * Nq * D;
    const __bf16* K = (const __bf16*)p.k + (size_t)(b * p.Hkv + g) * Nk * D;
    const __bf16* V = (const __bf16*)p.v + (size_t)(b * p.Hkv + g) * Nk * D;
    const int32_t* docrow = DOC ? p.doc + (size_t)b * Nk : nullptr;

    // ---- key range of the whole query tile
    int kv_lo = 0, kv_hi = Nk;
    if (causal) kv_hi = min(kv_hi, qlast + off + 1);
    if (windowed) kv_lo = max(kv_lo, q0 + off - W + 1);
    if (DOC) {
        kv_lo = max(kv_lo, wave_search<false>(docrow, Nk, docrow[q0], lane));
        kv_hi = min(kv_hi, wave_search<true>(docrow, Nk, docrow[qlast], lane));
    }
    const int kt_begin = kv_lo / BN;
    const int n_tiles = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN - kt_begin : 0;

    // ---- this wave's rows
    const int wq0 = q0 + wave * QB * 32;
    const bool wave_active = wq0 < Nq;
    const int wq1 = min(wq0 + QB * 32, Nq) - 1;
    int row[QB];
    int doc_i[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        row[qb] = wq0 + qb * 32 + l32;
        doc_i[qb] = DOC ? docrow[min(row[qb], Nq - 1)] : 0;
    }
    const int dq0 = DOC && wave_active ? docrow[wq0] : 0;
    const int dq1 = DOC && wave_active ? docrow[wq1] : 0;

    const float c = p.scale_log2;
    const float slope_l2 = ALIBI ? p.slopes[h] * kLog2e : 0.f;
    const float cap_l2 = SOFTCAP ? p.softcap * kLog2e : 0.f;        // cap in exp2 units
    const float cap_in = SOFTCAP ? p.scale * 2.f * kLog2e / p.softcap : 0.f;

    // ---- Q fragments (B operand of GEMM0): lane holds row l32, d = 16 s + 8 hh + 0..7
    bf16x8 qf[QB][DS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const __bf16* qr = Q + (size_t)min(row[qb], Nq - 1) * D + 8 * hh;
#pragma unroll
        for (int s = 0; s < DS; ++s) qf[qb][s] = *(const bf16x8*)(qr + 16 * s);
    }

    f32x16 o[QB][DT];
    float m[QB], l[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m[qb] = -INFINITY;
        l[qb] = 0.f;
#pragma unroll
        for (int t = 0; t < DT; ++t) o[qb][t] = f32x16{};
    }

    // ---- lane-constant LDS offsets
    // K reads: row 32 kb + l32, logical chunk 2 s + hh
    int koff[DS];
    {
        const int r = l32;
#pragma unroll
        for (int s = 0; s < DS; ++s) koff[s] = r * T::ROW_BYTES + (((2 * s + hh) ^ T::swz_k(r)) * 16);
    }
    // V transposed reads: within each 16-lane group, lane L addresses row
    // R0 + L/4 (R0 = 32 kb + 16 u + 8 part + 4 hh), columns 32 t + 16 cg + 4 (L % 4).
    int voff[DT];
    {
        const int L = lane & 15, cg = (lane >> 4) & 1;
        const int r = 4 * hh + (L >> 2);   // row modulo 32, swizzle-relevant part
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            const int col = 32 * t + 16 * cg + 4 * (L & 3);
            const int chunk = (col * 2) >> 4;
            voff[t] = r * T::ROW_BYTES + ((chunk ^ T::swz_v(r)) << 4) + ((col * 2) & 15);
        }
    }

    auto compute_tile = [&](const ATTN_LDS char* kl, const ATTN_LDS char* vl, const ATTN_LDS int* dl,
                            int kt) __attribute__((always_inline)) {
        const int j0 = kt * BN;
        const bool ragged = j0 + BN > Nk;
        const int j1 = min(j0 + BN, Nk) - 1;
        bool empty = false, full = !ragged;
        if (causal) { empty |= j0 > wq1 + off; full &= j1 <= wq0 + off; }
        if (windowed) { empty |= (wq0 + off) - j1 >= W; full &= (wq1 + off) - j0 < W; }
        if (DOC) {
            const int dj0 = dl[wave * BN], dj1 = dl[wave * BN + (j1 - j0)];
            empty |= dj1 < dq0 || dj0 > dq1;
            full &= dj0 == dj1 && dq0 == dq1 && dj0 == dq0;
        }
        if (empty) return;

        // GEMM0: S^T[key][query] for 2 key blocks of 32
        f32x16 sacc[QB][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int s = 0; s < DS; ++s) {
                const bf16x8 kf = *(const ATTN_LDS bf16x8*)(kl + koff[s] + kb * 32 * T::ROW_BYTES);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    sacc[qb][kb] = mfma_bf16(kf, qf[qb][s], s == 0 ? f32x16{} : sacc[qb][kb]);
            }
        }

        constexpr bool MODS = SOFTCAP || ALIBI;
        const bool general = MODS || !full;
        bf16x8 pf[QB][2][2];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = -INFINITY;
            if (!general) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][kb][r]);
                mx = xhalf_max(mx) * c;
            } else {
                // modified score in exp2 units, masked entries -inf
                const int i = row[qb];
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
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int jl = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);   // key within tile
                        float y;
                        if (SOFTCAP) {
                            // cap * tanh(x / cap) = cap - 2 cap / (exp(2 x / cap) + 1), in exp2 units
                            const float e = fast_exp2(sacc[qb][kb][r] * cap_in);
                            y = cap_l2 - 2.f * cap_l2 * fast_rcp(e + 1.f);
                        } else {
                            y = sacc[qb][kb][r] * c;
                        }
                        if (ALIBI) y -= slope_l2 * (float)(i - (j0 + jl));
                        if (!full) {
                            const int j = j0 + jl;
                            bool ok = j < Nk;
                            if (causal) ok &= j <= i + off;
                            if (windowed) ok &= i + off - j < W;
                            if (DOC) ok &= dk[kb][r] == doc_i[qb];
                            y = ok ? y : -INFINITY;
                        }
                        sacc[qb][kb][r] = y;
                        mx = fmaxf(mx, y);
                    }
                }
                mx = xhalf_max(mx);
            }
            const float mnew = fmaxf(m[qb], mx);
            const float mu = mnew == -INFINITY ? 0.f : mnew;
            const float alpha = fast_exp2(m[qb] - mu);
            m[qb] = mnew;
            float ls = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x = general ? sacc[qb][kb][r] - mu : __builtin_fmaf(sacc[qb][kb][r], c, -mu);
                    const float pe = fast_exp2(x);
                    sacc[qb][kb][r] = pe;
                    ls += pe;
                }
            l[qb] = l[qb] * alpha + ls;
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                for (int t = 0; t < DT; ++t) o[qb][t] *= alpha;
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    bf16x8 v8;
#pragma unroll
                    for (int e = 0; e < 8; ++e) v8[e] = (__bf16)sacc[qb][kb][8 * u + e];
                    pf[qb][kb][u] = v8;
                }
        }

        // GEMM1: O^T += V^T P^T
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int t = 0; t < DT; ++t) {
                    const int base = (32 * kb + 16 * u) * T::ROW_BYTES + voff[t];
                    const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (ATTN_LDS bf16x4*)(vl + base));
                    const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (ATTN_LDS bf16x4*)(vl + base + 8 * T::ROW_BYTES));
                    const bf16x8 vf = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) o[qb][t] = mfma_bf16(vf, pf[qb][kb][u], o[qb][t]);
                }
    };

    // ---- main loop: tile i is multiplied while tile i + 1 lands in the other buffer
    ATTN_LDS char* kl0 = (ATTN_LDS char*)k_lds0;
    ATTN_LDS char* kl1 = (ATTN_LDS char*)k_lds1;
    ATTN_LDS char* vl0 = (ATTN_LDS char*)v_lds0;
    ATTN_LDS char* vl1 = (ATTN_LDS char*)v_lds1;
    ATTN_LDS int* dl0 = (ATTN_LDS int*)d_lds0;
    ATTN_LDS int* dl1 = (ATTN_LDS int*)d_lds1;
    if (n_tiles > 0)
        issue_tile<D, NW, DOC>(K, V, docrow, kt_begin * BN, Nk, kl0, vl0, dl0, wave, lane);
    for (int it = 0; it < n_tiles; it += 2) {
        wait_all_and_barrier();
        if (it + 1 < n_tiles)
            issue_tile<D, NW, DOC>(K, V, docrow, (kt_begin + it + 1) * BN, Nk, kl1, vl1, dl1, wave, lane);
        if (wave_active) compute_tile(kl0, vl0, dl0, kt_begin + it);
        if (it + 1 >= n_tiles) break;
        wait_all_and_barrier();
        if (it + 2 < n_tiles)
            issue_tile<D, NW, DOC>(K, V, docrow, (kt_begin + it + 2) * BN, Nk, kl0, vl0, dl0, wave, lane);
        if (wave_active) compute_tile(kl1, vl1, dl1, kt_begin + it + 1);
    }

    // ---- epilogue: O / l, LSE = (m + log2 l) ln 2
    if (!wave_active) return;
    __bf16* O = (__bf16*)p.o + (size_t)(b * p.Hq + h) * Nq * D;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float lt = xhalf_sum(l[qb]);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        const int i = row[qb];
        if (i < Nq) {
            __bf16* orow = O + (size_t)i * D + 4 * hh;
#pragma unroll
            for (int t = 0; t < DT; ++t)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    bf16x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[qb][t][4 * gq + e] * inv);
                    *(bf16x4*)(orow + 32 * t + 8 * gq) = w;
                }
            if (p.lse && hh == 0)
                p.lse[(size_t)(b * p.Hq + h) * Nq + i] =
                    lt > 0.f ? (m[qb] + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
        }
    }
}

// -----------------------------------------------------------------------------
// fp32 inputs: the same tiling on the fp32 matrix cores (32x32x2), one wave per
// 32 query rows, K / V tiles staged through LDS with plain loads. No operand is
// ever rounded below fp32.
template <int D, bool SOFTCAP, bool ALIBI, bool DOC>
__global__ __launch_bounds__(256) void fwd_f32_kernel(FwdParams p) {
    constexpr int NW = 4, BM = NW * 32, DT = D / 32;
    __shared__ float k_lds[BN][D + 1];
    __shared__ float v_lds[BN][D + 1];
    __shared__ int d_lds[BN];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    const int wid = blockIdx.x;
    const int qt = p.n_qt - 1 - wid / p.n_bh;
    const int bh = wid % p.n_bh;
    const int b = bh / p.Hq, h = bh % p.Hq, g = h / p.group;
    const int Nq = p.Nq, Nk = p.Nk, off = Nk - Nq;
    const bool causal = p.mask & kMaskCausal, windowed = p.mask & kMaskWindow;
    const int W = p.window;
    const int q0 = qt * BM;
    const int qlast = min(q0 + BM, Nq) - 1;
    const float* Q = (const float*)p.q + (size_t)(b * p.Hq + h) * Nq * D;
    const float* K = (const float*)p.k + (size_t)(b * p.Hkv + g) * Nk * D;
    const float* V = (const float*)p.v + (size_t)(b * p.Hkv + g) * Nk * D;
    const int32_t* docrow = DOC ? p.doc + (size_t)b * Nk : nullptr;

    int kv_lo = 0, kv_hi = Nk;
    if (causal) kv_hi = min(kv_hi, qlast + off + 1);
    if (windowed) kv_lo = max(kv_lo, q0 + off - W + 1);
    if (DOC) {
        kv_lo = max(kv_lo, wave_search<false>(docrow, Nk, docrow[q0], lane));
        kv_hi = min(kv_hi, wave_search<true>(docrow, Nk, docrow[qlast], lane));
    }
    const int kt_begin = kv_lo / BN;
    const int n_tiles = kv_hi > kv_lo ? (kv_hi + BN - 1) / BN - kt_begin : 0;

    const int i = q0 + wave * 32 + l32;
    const bool valid = i < Nq;
    const float* qr = Q + (size_t)min(i, Nq - 1) * D;
    const int doc_i = DOC ? docrow[min(i, Nq - 1)] : 0;
    const float c = p.scale_log2;
    const float slope_l2 = ALIBI ? p.slopes[h] * kLog2e : 0.f;
    const float cap_l2 = SOFTCAP ? p.softcap * kLog2e : 0.f;
    const float cap_in = SOFTCAP ? p.scale * 2.f * kLog2e / p.softcap : 0.f;

    f32x16 o[DT];
    for (int t = 0; t < DT; ++t) o[t] = f32x16{};
    float m = -INFINITY, l = 0.f;

    for (int it = 0; it < n_tiles; ++it) {
        const int j0 = (kt_begin + it) * BN;
        __syncthreads();
        for (int e = threadIdx.x; e < BN * D; e += NW * 64) {
            const int r = e / D, cc = e % D;
            const int gr = min(j0 + r, Nk - 1);
            k_lds[r][cc] = K[(size_t)gr * D + cc];
            v_lds[r][cc] = V[(size_t)gr * D + cc];
        }
        if (DOC && threadIdx.x < BN) d_lds[threadIdx.x] = docrow[min(j0 + (int)threadIdx.x, Nk - 1)];
        __syncthreads();

        f32x16 s[2];
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{};
            for (int st = 0; st < D / 2; ++st)
                s[kb] = mfma_f32(k_lds[32 * kb + l32][2 * st + hh], qr[2 * st + hh], s[kb]);
        }
        float mx = -INFINITY;
        for (int kb = 0; kb < 2; ++kb)
            for (int r = 0; r < 16; ++r) {
                const int jl = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                const int j = j0 + jl;
                float y;
                if (SOFTCAP) {
                    const float e = exp2f(s[kb][r] * cap_in);
                    y = cap_l2 - 2.f * cap_l2 / (e + 1.f);
                } else {
                    y = s[kb][r] * c;
                }
                if (ALIBI) y -= slope_l2 * (float)(i - j);
                bool ok = j < Nk;
                if (causal) ok &= j <= i + off;
                if (windowed) ok &= i + off - j < W;
                if (DOC) ok &= d_lds[jl] == doc_i;
                y = ok ? y : -INFINITY;
                s[kb][r] = y;
                mx = fmaxf(mx, y);
            }
        mx = xhalf_max(mx);
        const float mnew = fmaxf(m, mx);
        const float mu = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = exp2f(m - mu);
        m = mnew;
        float ls = 0.f;
        for (int kb = 0; kb < 2; ++kb)
            for (int r = 0; r < 16; ++r) {
                const float pe = exp2f(s[kb][r] - mu);
                s[kb][r] = pe;
                ls += pe;
            }
        l = l * alpha + ls;
        for (int t = 0; t < DT; ++t) o[t] *= alpha;
        // O^T += V^T P^T, two keys (one per half-wave) per step
        for (int kb = 0; kb < 2; ++kb)
            for (int r = 0; r < 16; ++r) {
                const int jl = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
                for (int t = 0; t < DT; ++t) o[t] = mfma_f32(v_lds[jl][32 * t + l32], s[kb][r], o[t]);
            }
    }

    const float lt = xhalf_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (valid) {
        float* orow = (float*)p.o + ((size_t)(b * p.Hq + h) * Nq + i) * D + 4 * hh;
        for (int t = 0; t < DT; ++t)
            for (int gq = 0; gq < 4; ++gq) {
                f32x4 w;
                for (int e = 0; e < 4; ++e) w[e] = o[t][4 * gq + e] * inv;
                *(f32x4*)(orow + 32 * t + 8 * gq) = w;
            }
        if (p.lse && hh == 0)
            p.lse[(size_t)(b * p.Hq + h) * Nq + i] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
    }
}

// -----------------------------------------------------------------------------
// Host-side launchers (called by the C ABI after validation).
template <int D, int QB, int NW, bool SC, bool AL, bool DC>
static hipError_t launch_bf16_inst(const FwdParams& p0, hipStream_t st) {
    FwdParams p = p0;
    constexpr int BM = NW * QB * 32;
    p.n_qt = (p.Nq + BM - 1) / BM;
    p.n_bh = p.B * p.Hq;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, NW, SC, AL, DC>), dim3(p.n_qt * p.n_bh), dim3(NW * 64),
                       0, st, p);
    return hipGetLastError();
}

template <int D, int QB, int NW>
static hipError_t launch_bf16_d(const FwdParams& p, hipStream_t st) {
    const bool sc = p.softcap > 0.f, al = p.slopes != nullptr, dc = (p.mask & kMaskDoc) != 0;
    if (!sc && !al && !dc) return launch_bf16_inst<D, QB, NW, false, false, false>(p, st);
    if (!sc && !al && dc) return launch_bf16_inst<D, QB, NW, false, false, true>(p, st);
    if (sc && al && dc) return launch_bf16_inst<D, QB, NW, true, true, true>(p, st);
    if (sc && !al && !dc) return launch_bf16_inst<D, QB, NW, true, false, false>(p, st);
    if (!sc && al && !dc) return launch_bf16_inst<D, QB, NW, false, true, false>(p, st);
    if (sc && al && !dc) return launch_bf16_inst<D, QB, NW, true, true, false>(p, st);
    if (sc && !al && dc) return launch_bf16_inst<D, QB, NW, true, false, true>(p, st);
    return launch_bf16_inst<D, QB, NW, false, true, true>(p, st);
}

hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t st) {
    if (d == 128) return launch_bf16_d<128, 2, 4>(p, st);
    return launch_bf16_d<64, 2, 4>(p, st);
}

template <int D, bool SC, bool AL, bool DC>
static hipError_t launch_f32_inst(const FwdParams& p0, hipStream_t st) {
    FwdParams p = p0;
    p.n_qt = (p.Nq + 127) / 128;
    p.n_bh = p.B * p.Hq;
    hipLaunchKernelGGL((fwd_f32_kernel<D, SC, AL, DC>), dim3(p.n_qt * p.n_bh), dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_f32_d(const FwdParams& p, hipStream_t st) {
    const bool sc = p.softcap > 0.f, al = p.slopes != nullptr, dc = (p.mask & kMaskDoc) != 0;
    if (!sc && !al && !dc) return launch_f32_inst<D, false, false, false>(p, st);
    if (!sc && !al && dc) return launch_f32_inst<D, false, false, true>(p, st);
    if (sc && al && dc) return launch_f32_inst<D, true, true, true>(p, st);
    if (sc && !al && !dc) return launch_f32_inst<D, true, false, false>(p, st);
    if (!sc && al && !dc) return launch_f32_inst<D, false, true, false>(p, st);
    if (sc && al && !dc) return launch_f32_inst<D, true, true, false>(p, st);
    if (sc && !al && dc) return launch_f32_inst<D, true, false, true>(p, st);
    return launch_f32_inst<D, false, true, true>(p, st);
}

hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t st) {
    if (d == 128) return launch_f32_d<128>(p, st);
    return launch_f32_d<64>(p, st);
}

}  // namespace attn
