// fp8 (OCP e4m3) path: the incoherent-processing prepare step and the fused
// forward on fp8 matrix cores.
//
// "FlashAttention-3 : une attention plus rapide ...", section "Basse precision
// FP8 et incoherent processing": Q and K are multiplied by a Hadamard transform
// with random signs, per head, in O(d log d), which spreads outlier channels
// before quantisation; section "Fonctionnalites des GPU Hopper : WGMMA, TMA,
// FP8": fp8 doubles matrix throughput; section "Chevauchement de GEMM et
// softmax grace a l'asynchronisme": the exponential does not get faster in fp8,
// so the softmax / matrix overlap matters even more.
#include <climits>
#include <type_traits>

#include "fwd_common.h"

namespace attn {

constexpr float kFp8NoMax = -1e30f;   // initial exponent reference: finite, below any score

constexpr int kFp8Tile = 128;        // tokens per quantisation scale
constexpr float kE4m3Max = 448.f;
constexpr float kFp8PShift = 4.f;    // P is stored as e4m3(p * 2^4 * s_v / s_vmax), p <= 2^4

// -----------------------------------------------------------------------------
// Prepare: one workgroup (4 waves) per (tensor, batch, head, 128-token tile).
// Lane layout: 4 lanes per token; lane c of a quad holds the 8-dim chunks
// c, c + 4, c + 8, c + 12, i.e. dims 8c + 32j + e (j, e < 4, 8): every load
// instruction reads 64 contiguous bytes of each of 16 token rows, and of the
// 7 index bits of a dim, bits 0-2 (e) and 5-6 (j) are in the lane's registers
// and bits 3-4 (c) across the quad. A wave covers 16 tokens per step, the 4
// waves 64, two steps the tile. Q and K rows: x <- (x * signs) H / sqrt(d),
// the Walsh-Hadamard transform in Sylvester order: butterflies on bits 0-2 and
// 5-6 in registers, on bits 3-4 with quad permutes (xor 1, xor 2); butterflies
// on different bits commute, so their order does not change the result. Then
// the tile's amax gives scale = amax / 448 and the codes are the round-to-
// nearest-even e4m3 values of x / scale (clamped to +-448 first, so nothing
// saturates to NaN). Q and K also get a residual code on the same scale,
// e4m3(x / scale - value(code)): the difference is exact in float32 (the code
// is within a factor 17/16 of x / scale), so value + residual carries about
// six mantissa bits. V is not rotated, has one code and is written
// transposed, [d][tokens], so the attention kernel reads contiguous keys per
// lane.
// With rotary tables (rope_cos / rope_sin, float32 [N][d/2]) Q and K rows are
// first turned pairwise, (x_i, x_{i+d/2}) by the token's angle (the pair sits
// in one lane: j and j + 2): both passes are memory-bound over the same rows,
// so they share one read and one write ("FlashAttention-3 : ...", section
// "Basse precision FP8 et incoherent processing").
__device__ __forceinline__ float quad_xor(float v, int m) {
    // DPP quad permutes: xor 1 = [1, 0, 3, 2] (0xB1), xor 2 = [2, 3, 0, 1] (0x4E)
    const int i = __float_as_int(v);
    return __int_as_float(m == 1 ? __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true)
                                 : __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true));
}

__global__ __launch_bounds__(256) void fp8_prepare_kernel(const __bf16* __restrict__ q,
                                                          const __bf16* __restrict__ k,
                                                          const __bf16* __restrict__ v, int B, int Hq,
                                                          int Hkv, int N, int Np, const int8_t* __restrict__ signs,
                                                          const float* __restrict__ rope_cos,
                                                          const float* __restrict__ rope_sin,
                                                          uint8_t* __restrict__ q8, uint8_t* __restrict__ k8,
                                                          uint8_t* __restrict__ v8) {
    constexpr int D = 128, STEPS = kFp8Tile / 64;   // 64 tokens per step over the 4 waves
    __shared__ float red[4];
    __shared__ __attribute__((aligned(16))) uint8_t vt[D][kFp8Tile];
    const int nt = Np / kFp8Tile;
    const int nq = B * Hq * nt, nk = B * Hkv * nt;
    int id = blockIdx.x;
    int which, H;
    const __bf16* src;
    uint8_t* dst;
    if (id < nq) { which = 0; src = q; dst = q8; H = Hq; }
    else if (id < nq + nk) { which = 1; id -= nq; src = k; dst = k8; H = Hkv; }
    else { which = 2; id -= nq + nk; src = v; dst = v8; H = Hkv; }
    const int tile = id % nt, bh = id / nt;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane & 3;              // quad lane: chunks c + 4 j
    const int tq = lane >> 2;            // token of the wave's 16
    const bool rot = which < 2 && signs != nullptr;
    const bool rope = which < 2 && rope_cos != nullptr;

    float sg[4][8];
    if (rot) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) sg[j][e] = signs[8 * c + 32 * j + e] < 0 ? -1.f : 1.f;
    }

    float x[STEPS][4][8];   // [step][j][e]: dim 8c + 32j + e
    float am = 0.f;
    // The rows of every step are loaded first, all loads in flight together;
    // rows past N read row N - 1 and are zeroed (no branch around the loads).
    bf16x8 raw[STEPS][4];
#pragma unroll
    for (int it = 0; it < STEPS; ++it) {
        const int row = tile * kFp8Tile + it * 64 + wave * 16 + tq;
        const __bf16* rp = src + ((size_t)bh * N + min(row, N - 1)) * D + 8 * c;
#pragma unroll
        for (int j = 0; j < 4; ++j) raw[it][j] = *(const bf16x8*)(rp + 32 * j);
    }
#pragma unroll
    for (int it = 0; it < STEPS; ++it) {
        const int t = it * 64 + wave * 16 + tq;   // token within the tile
        const int row = tile * kFp8Tile + t;
        float (*y)[8] = x[it];
        {
            const bool in = row < N;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) y[j][e] = in ? (float)raw[it][j][e] : 0.f;
        }
        if (rope && row < N) {
            // pair (i, i + 64) = (j, j + 2) of this lane, i = 8c + 32j + e, j < 2
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float4* c4 = (const float4*)(rope_cos + (size_t)row * (D / 2) + 8 * c + 32 * j);
                const float4* s4 = (const float4*)(rope_sin + (size_t)row * (D / 2) + 8 * c + 32 * j);
                const float4 c0 = c4[0], c1 = c4[1], s0 = s4[0], s1 = s4[1];
                const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
                const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float a0 = y[j][e], b0 = y[j + 2][e];
                    y[j][e] = __builtin_fmaf(a0, cs[e], -b0 * sn[e]);
                    y[j + 2][e] = __builtin_fmaf(a0, sn[e], b0 * cs[e]);
                }
            }
        }
        if (rot) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) y[j][e] *= sg[j][e];
            // index bits 0-2 (e) and 5-6 (j): in registers
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int len = 1; len < 8; len <<= 1)
#pragma unroll
                    for (int i = 0; i < 8; i += 2 * len)
#pragma unroll
                        for (int e = i; e < i + len; ++e) {
                            const float a0 = y[j][e], b0 = y[j][e + len];
                            y[j][e] = a0 + b0;
                            y[j][e + len] = a0 - b0;
                        }
#pragma unroll
            for (int lj = 1; lj < 4; lj <<= 1)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if ((j & lj) == 0)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float a0 = y[j][e], b0 = y[j + lj][e];
                            y[j][e] = a0 + b0;
                            y[j + lj][e] = a0 - b0;
                        }
            // index bits 3-4 (c): across the quad
#pragma unroll
            for (int m = 1; m < 4; m <<= 1) {
                const float sgn = (c & m) ? -1.f : 1.f;   // upper lane of the pair: partner - self
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[j][e] = __builtin_fmaf(sgn, y[j][e], quad_xor(y[j][e], m));
            }
            const float r = 0.08838834764831845f;   // 1 / sqrt(128)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 8; ++e) y[j][e] *= r;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(y[j][e]));
    }
#pragma unroll
    for (int s2 = 32; s2 >= 1; s2 >>= 1) am = fmaxf(am, __shfl_xor(am, s2));
    if (lane == 0) red[wave] = am;
    __syncthreads();
    am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = am > 0.f ? am / kE4m3Max : 1.f;
    const float inv = 1.f / sc;
    const size_t plane = (size_t)B * H * Np * D;   // bytes of one code plane
    float* scales = (float*)(dst + 2 * plane);
    if (threadIdx.x == 0) scales[(size_t)bh * nt + tile] = sc;

#pragma unroll
    for (int it = 0; it < STEPS; ++it) {
        const int t = it * 64 + wave * 16 + tq;
        const int row = tile * kFp8Tile + t;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t w2[2], r2[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const float* z = x[it][j] + 4 * h2;
                const float a0 = fminf(fmaxf(z[0] * inv, -kE4m3Max), kE4m3Max);
                const float a1 = fminf(fmaxf(z[1] * inv, -kE4m3Max), kE4m3Max);
                const float a2 = fminf(fmaxf(z[2] * inv, -kE4m3Max), kE4m3Max);
                const float a3 = fminf(fmaxf(z[3] * inv, -kE4m3Max), kE4m3Max);
                int pk = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
                pk = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, pk, true);
                w2[h2] = (uint32_t)pk;
                if (which < 2) {   // residual of the rounding, on the same scale
                    const auto v01 = __builtin_amdgcn_cvt_pk_f32_fp8(pk, false);
                    const auto v23 = __builtin_amdgcn_cvt_pk_f32_fp8(pk, true);
                    int rk = __builtin_amdgcn_cvt_pk_fp8_f32(a0 - v01[0], a1 - v01[1], 0, false);
                    rk = __builtin_amdgcn_cvt_pk_fp8_f32(a2 - v23[0], a3 - v23[1], rk, true);
                    r2[h2] = (uint32_t)rk;
                }
            }
            if (which < 2) {
                uint8_t* rp = dst + ((size_t)bh * Np + row) * D + 8 * c + 32 * j;
                *(uint2*)rp = make_uint2(w2[0], w2[1]);
                *(uint2*)(rp + plane) = make_uint2(r2[0], r2[1]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) vt[8 * c + 32 * j + e][t] = (uint8_t)(w2[e >> 2] >> (8 * (e & 3)));
            }
        }
    }
    if (which == 2) {
        __syncthreads();
        // thread i stores half (i & 1) of d-row i / 2 of the transposed tile
        const int dr = threadIdx.x >> 1, half = threadIdx.x & 1;
        const uint4* src4 = (const uint4*)&vt[dr][64 * half];
        uint4* o = (uint4*)(dst + ((size_t)bh * D + dr) * Np + (size_t)tile * kFp8Tile + 64 * half);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = src4[i];
    }
}

hipError_t launch_fp8_prepare(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int N, int d,
                              const int8_t* signs, const float* rope_cos, const float* rope_sin, void* q8,
                              void* k8, void* v8, hipStream_t st) {
    if (d != 128) return hipErrorNotSupported;
    const int Np = (N + kFp8Tile - 1) / kFp8Tile * kFp8Tile;
    const int nt = Np / kFp8Tile;
    const long long blocks = (long long)B * (Hq + 2 * Hkv) * nt;
    if (blocks > INT_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fp8_prepare_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, B, Hq, Hkv, N, Np, signs, rope_cos, rope_sin,
                       (uint8_t*)q8, (uint8_t*)k8, (uint8_t*)v8);
    return hipGetLastError();
}

// -----------------------------------------------------------------------------
// fp8 forward, d = 128, no mask. Same tiling and two-waves-per-SIMD ping-pong
// as the bf16 kernel (see attn_fwd_bf16.hip), on 32x32x64 e4m3 matrix cores:
//   GEMM0  S^T = K8 Q8^T   per 64-key tile: 2 key blocks x 2 k-steps of 64,
//          three products per step on one accumulator: value x value,
//          value(K) x residual(Q) and residual(K) x value(Q) (the residual x
//          residual term, below 2^-8 of the score, is left out); both codes
//          of a row share its tile scale, so the sum is one scaled score.
//          The K rows of block kb are read in the order
//              pi(m) = 32 ((m >> 2) & 1) + 16 kb + 4 (m >> 3) + (m & 3)
//          so that accumulator register r of half-wave h holds key
//          32 h + 16 kb + r: every lane then owns 32 consecutive keys.
//   GEMM1  O^T = V8^T P8^T  one 64-key instruction per 32 output columns; the
//          32 consecutive keys of a lane are exactly the B operand, and V^T
//          rows give the A operand with contiguous keys.
// Scales: S = s_q s_k (q8 . k8) -- folded into the per-tile score multiplier.
// P is stored as e4m3(p 2^4 s_v(t) / s_vmax), the factor folded into the exp2
// bias; the running sum uses the unscaled p; the epilogue multiplies by
// s_vmax / 2^4. The exponent reference moves only when the row max grows by
// more than 2^4, so p 2^4 s_v / s_vmax stays below 448.
struct Fp8Tile {
    static constexpr int KROW = 128;                 // bytes per key row (d = 128)
    static constexpr int VROW = 64;                  // bytes per V^T row (64 keys)
    static constexpr int KBYTES = BN * KROW;         // 8 KiB
    static constexpr int VBYTES = 128 * VROW;        // 8 KiB
    static __device__ __forceinline__ int swz_k(int r) { return ((r >> 1) ^ (r >> 3)) & 7; }
    static __device__ __forceinline__ int swz_v(int r) { return (r >> 2) & 3; }
};

template <bool RAGGED>
__global__ __launch_bounds__(512) void fwd_fp8_kernel(FwdParams p) {
    using T = Fp8Tile;
    constexpr int NW = 8, BM = NW * 32, D = 128;
#ifdef ATTN_SINGLE_STAGE
    // debug build: one tile in flight, each copy waited for as soon as it is
    // issued; the arithmetic is unchanged, so the results must be equal bit for bit
    constexpr int PF = 1;
#else
    constexpr int PF = 2;
#endif
    constexpr int NKB = PF + 1, NVB = PF + 2;
    constexpr float kTau = kFp8PShift;   // lazy-rescale threshold (log2 units)
    constexpr int KBUF = 2 * T::KBYTES;  // key tile: value codes, then residual codes
    constexpr int LOADS_PER_TILE = 3;    // copies per wave and tile: K value, K residual, V
    // The epilogue stages each wave's 32 output rows (8 KiB) in a slot of this
    // space no wave reads any more: at least 9 slots, one of which may still
    // hold the last value tile.
    constexpr int kTileSpace = NKB * KBUF + NVB * T::VBYTES;
    constexpr int kSlot = 32 * D * 2;
    static_assert(KBUF % kSlot == 0 && T::VBYTES == kSlot, "output staging slots");
    __shared__ __attribute__((aligned(1024))) char tiles_lds[kTileSpace > 9 * kSlot ? kTileSpace : 9 * kSlot];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool group_b = wave >= NW / 2;
    const int l32 = lane & 31, hh = lane >> 5;
    const int wid = blockIdx.x;
    int qt = p.n_qt - 1 - wid / p.n_bh;
    int bh = wid % p.n_bh;
    // With xgrp > 0 each XCD (workgroup w runs on XCD w % 8) takes its heads
    // xgrp at a time, all query tiles of those heads before the next ones, so
    // the tiles in flight on one XCD read the same K / V codes from its L2.
    if (p.xgrp > 0) {
        const int x = wid % 8, k = wid / 8, per = p.xgrp * p.n_qt, r = k % per;
        qt = p.n_qt - 1 - r / p.xgrp;
        bh = x + 8 * ((k / per) * p.xgrp + r % p.xgrp);
    }
    const int b = bh / p.Hq, h = bh % p.Hq, g = h / p.group;
    const int N = p.Nk, Np = p.npad, ntile = Np / kFp8Tile;
    const int q0 = qt * BM;
    const size_t bhq = (size_t)b * p.Hq + h, bhk = (size_t)b * p.Hkv + g;
    // packed buffers: value codes, residual codes (Q, K), then the tile scales
    const size_t qplane = (size_t)p.B * p.Hq * Np * D, kplane = (size_t)p.B * p.Hkv * Np * D;
    const uint8_t* Q8 = (const uint8_t*)p.q + bhq * Np * D;
    const uint8_t* K8 = (const uint8_t*)p.k + bhk * Np * D;
    const uint8_t* K8r = K8 + kplane;
    const uint8_t* V8 = (const uint8_t*)p.v + bhk * D * Np;
    const float* qsc = (const float*)((const uint8_t*)p.q + 2 * qplane) + bhq * ntile;
    const float* ksc = (const float*)((const uint8_t*)p.k + 2 * kplane) + bhk * ntile;
    const float* vsc = (const float*)((const uint8_t*)p.v + 2 * kplane) + bhk * ntile;

    const int wq0 = q0 + wave * 32;
    const bool wave_active = wq0 < N;
    const int row = wq0 + l32;
    const int n_tiles = (N + BN - 1) / BN;

    // largest V scale of the head (wave reduction over its tiles)
    float svmax = 0.f;
    for (int i = lane; i < ntile; i += 64) svmax = fmaxf(svmax, vsc[i]);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) svmax = fmaxf(svmax, __shfl_xor(svmax, s));
    const float log2_svmax = __builtin_amdgcn_logf(svmax);
    const float sq = qsc[min(wq0, Np - 1) / kFp8Tile];
    const float c_q = sq * p.scale_log2;

    // Q fragments (value and residual codes): lane holds row l32, bytes
    // 64 s + 32 hh .. + 31
    i32x8 qf[2], qr2[2];
    {
        const uint8_t* qr = Q8 + (size_t)min(row, Np - 1) * D + 32 * hh;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            qf[s] = *(const i32x8*)(qr + 64 * s);
            qr2[s] = *(const i32x8*)(qr + qplane + 64 * s);
        }
    }
    // Retire every compiler-visible global load before the loop: the tile
    // copies are inline asm the compiler does not count, so a pending load
    // would get in-loop vmcnt waits that also drain the prefetches.
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    // per-tile scales, read in the loop through the scalar cache
    const ATTN_CONST float* ksc_s = (const ATTN_CONST float*)ksc;
    const ATTN_CONST float* vsc_s = (const ATTN_CONST float*)vsc;

    f32x16 o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = f32x16{};
    float m = kFp8NoMax, l = 0.f;
    // Matrix operands written by vector code: set here, pinned in their
    // register files, followed by wait states before the first product.
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        pin_a(qf[s]);
        pin_a(qr2[s]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) pin_a(o[t]);
    mfma_guard();

    ATTN_LDS char* lds = (ATTN_LDS char*)tiles_lds;
    auto kbuf = [&](int i) __attribute__((always_inline)) { return lds + (i % NKB) * KBUF; };
    auto vbuf = [&](int i) __attribute__((always_inline)) {
        return lds + NKB * KBUF + (i % NVB) * T::VBYTES;
    };
    // Lane-constant fragment offsets. K: block kb, lane row pi(l32) (+16 kb),
    // 16-byte chunks 4 s + 2 hh + {0, 1}. V^T: row 32 t + l32 (the swizzle
    // does not depend on t), 16-byte chunks 2 hh + {0, 1}.
    const int krow = 32 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);
    int kofs[2][2][2], vofs[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int r = krow + 16 * kb, sw = T::swz_k(r);
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) kofs[kb][st][hf] = r * T::KROW + (((4 * st + 2 * hh + hf) ^ sw) << 4);
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) vofs[hf] = l32 * T::VROW + (((2 * hh + hf) ^ T::swz_v(l32)) << 4);
    auto at = [](int addr, int imm) __attribute__((always_inline)) {
        return (const ATTN_LDS char*)(uintptr_t)addr + imm;
    };

    // tile copies: one 16-byte slot per lane per tile, for K and for V^T
    const int s_slot = wave * 64 + lane;                      // 0..511
    const int ck_row = s_slot >> 3, ck_pc = s_slot & 7;
    const unsigned ck_off = ck_row * T::KROW + ((ck_pc ^ T::swz_k(ck_row)) << 4);
    const int cv_row = s_slot >> 2, cv_pc = s_slot & 3;
    const unsigned cv_off = cv_row * Np + ((cv_pc ^ T::swz_v(cv_row)) << 4);
    auto tile_k = [&](int i) __attribute__((always_inline)) {
        dma16s(K8 + (size_t)i * BN * D, ck_off, lds_addr(kbuf(i)) + wave * 1024);
        dma16s(K8r + (size_t)i * BN * D, ck_off, lds_addr(kbuf(i)) + T::KBYTES + wave * 1024);
    };
    auto tile_v = [&](int i) __attribute__((always_inline)) {
        dma16s(V8 + (size_t)i * BN, cv_off, lds_addr(vbuf(i)) + wave * 1024);
    };

    f32x16 sacc[2];
    auto gemm0 = [&](const ATTN_LDS char* kl) __attribute__((always_inline)) {
        const int sb = __builtin_amdgcn_readfirstlane((int)lds_addr(kl));
        int ka[2][2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    ka[kb][st][hf] = sb + kofs[kb][st][hf];
                    pin(ka[kb][st][hf]);
                }
        i32x8 kf[4], kr[4];   // value and residual fragments, i = (kb, st)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const i32x4 lo = *(const ATTN_LDS i32x4*)at(ka[i >> 1][i & 1][0], 0);
            const i32x4 hi = *(const ATTN_LDS i32x4*)at(ka[i >> 1][i & 1][1], 0);
            kf[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const i32x4 lo = *(const ATTN_LDS i32x4*)at(ka[i >> 1][i & 1][0], T::KBYTES);
            const i32x4 hi = *(const ATTN_LDS i32x4*)at(ka[i >> 1][i & 1][1], T::KBYTES);
            kr[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if ((i & 1) == 0) mfma_fp8_va0(sacc[i >> 1], kf[i], qf[0]);
            else mfma_fp8_va(sacc[i >> 1], kf[i], qf[1]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) mfma_fp8_va(sacc[i >> 1], kf[i], qr2[i & 1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) mfma_fp8_va(sacc[i >> 1], kr[i], qf[i & 1]);
        mfma_guard();   // the scores may be read right after
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) pin(sacc[kb]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            keep(kf[i]);
            keep(kr[i]);
        }
    };

    i32x8 pf = {};
    float rescale_by = 1.f;
    bool rescale_any = false;
    auto softmax = [&](int it) __attribute__((always_inline)) {
        const int tsc = (it * BN) / kFp8Tile;
        const float c = c_q * ksc_s[tsc];                        // score multiplier, exp2 units
        const float bias = kFp8PShift + __builtin_amdgcn_logf(vsc_s[tsc]) - log2_svmax;
        const int jl_hi = RAGGED ? N - 1 - it * BN : BN;         // last valid key in the tile
        if (RAGGED && jl_hi < BN - 1) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int jl = 32 * hh + 16 * kb + r;
                    sacc[kb][r] = jl <= jl_hi ? sacc[kb][r] : -INFINITY;
                }
        }
        float a0 = max3(sacc[0][0], sacc[0][1], sacc[0][2]), a1 = max3(sacc[1][0], sacc[1][1], sacc[1][2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) {
            a0 = max3(a0, sacc[0][r], sacc[0][r + 1]);
            a1 = max3(a1, sacc[1][r], sacc[1][r + 1]);
        }
        const float mx = xhalf_max(max3(a0, sacc[0][15], max2(a1, sacc[1][15]))) * c;
        const float mn = max2(m, mx);
        const bool need = mn > m + kTau;
        const float alpha = need ? fast_exp2(m - mn) : 1.f;
        m = need ? mn : m;
        const float mb = m - bias;
        float ls0, ls1, ls2, ls3;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 4) {
                const float p0 = fast_exp2(__builtin_fmaf(sacc[kb][r], c, -mb));
                const float p1 = fast_exp2(__builtin_fmaf(sacc[kb][r + 1], c, -mb));
                const float p2 = fast_exp2(__builtin_fmaf(sacc[kb][r + 2], c, -mb));
                const float p3 = fast_exp2(__builtin_fmaf(sacc[kb][r + 3], c, -mb));
                if (kb == 0 && r == 0) {
                    ls0 = p0; ls1 = p1; ls2 = p2; ls3 = p3;
                } else {
                    ls0 += p0; ls1 += p1; ls2 += p2; ls3 += p3;
                }
                // both halves of the word are written: the old contents only
                // name the register
                const int w = 4 * kb + (r >> 2);
                const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pf[w], false);
                pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, pk, true);
            }
        pin(pf);   // P is complete here; GEMM1 reads it after wait states
        l = l * alpha + ((ls0 + ls1) + (ls2 + ls3)) * fast_exp2(-bias);
        // take the sums here, while the other wave of the SIMD is in its matrix
        // phase (left alone, the compiler sinks them into this wave's own)
        pin(l);
        rescale_by = alpha;
        rescale_any = __builtin_amdgcn_ballot_w64(need) != 0;
        if (__builtin_expect(rescale_any, 0)) {   // rare: the reference max moved
            mfma_guard();
#pragma unroll
            for (int t = 0; t < 4; ++t) {
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

    auto gemm1 = [&](const ATTN_LDS char* vl) __attribute__((always_inline)) {
        const int sb = __builtin_amdgcn_readfirstlane((int)lds_addr(vl));
        int va[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            va[hf] = sb + vofs[hf];
            pin(va[hf]);
        }
        i32x8 vf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const i32x4 lo = *(const ATTN_LDS i32x4*)at(va[0], 32 * t * T::VROW);
            const i32x4 hi = *(const ATTN_LDS i32x4*)at(va[1], 32 * t * T::VROW);
            vf[t] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) mfma_fp8_a(o[t], vf[t], pf);
#pragma unroll
        for (int t = 0; t < 4; ++t) keep(vf[t]);
        keep(pf);
    };

    // Barrier i (i >= 1) is passed by group B at the top of iteration i - 1
    // and by group A between its softmax and GEMM1 of tile i - 1, so that one
    // wave's products overlap the other's softmax on each SIMD; the buffer
    // reuse argument is the bf16 kernel's. In the loop each wave issues its
    // copies of tile i + PF at the end of the interval (after its GEMM0), not
    // right after the barrier where all waves would queue up together.
    auto copies = [&](int i) __attribute__((always_inline)) {
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
        // tile i must have landed; with PF = 2 the copies of tile i + 1 may stay in flight
        if (PF >= 2 && i + 1 < n_tiles) __builtin_amdgcn_s_waitcnt(0x0070 | LOADS_PER_TILE);
        else __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (copy) copies(i);
    };
    auto body = [&](int it, bool next) __attribute__((always_inline)) {
        if (group_b) barrier_and_copy(it + 1, false);
        softmax(it);
        if (!group_b) barrier_and_copy(it + 1, false);
        operand_guard();   // P was written by vector code just before
        pin(pf);
        gemm1(vbuf(it));
        if (next) gemm0(kbuf(it + 1));
        copies(it + 1);
    };

    if (n_tiles > 0) {
        tile_k(0);
        tile_v(0);
        if (PF >= 2 && n_tiles > 1) {
            tile_k(1);
            tile_v(1);
        }
        barrier_and_copy(0);
    }
    if (wave_active) {
        if (n_tiles > 0) {
            gemm0(kbuf(0));
            int it = 0;
            for (; it < n_tiles - 1; ++it) body(it, true);
            body(it, false);
        }
    } else {
        for (int it = 0; it < n_tiles; ++it) barrier_and_copy(it + 1);   // copies and barriers only
    }

    if (!wave_active) return;
    mfma_guard();
#pragma unroll
    for (int t = 0; t < 4; ++t) pin_a(o[t]);
    const float lt = xhalf_sum(l);
    const float inv = lt > 0.f ? svmax / (exp2f(kFp8PShift) * lt) : 0.f;
    // Output through LDS so that each store writes whole contiguous rows (a
    // lane holds 4 of every 8 d values of its row; the wave's 32 rows are one
    // contiguous block of O). 8 KiB slots: the key buffers first, then the
    // value buffers; after the last barrier only the last tile's value buffer
    // is still read, and the wave skips its slot.
    int slot = wave;
    if (n_tiles > 0 && slot >= NKB * KBUF / kSlot + (n_tiles - 1) % NVB) ++slot;
    ATTN_LDS char* stage = (ATTN_LDS char*)tiles_lds + slot * kSlot;
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[t][4 * gq + e] * inv);
            // d = 32 t + 8 gq + 4 hh + e: 16-byte chunk 4 t + gq of row l32,
            // XOR-swizzled by the row so the 32 rows spread over the banks
            const int ch = (4 * t + gq) ^ (l32 & 15);
            *(ATTN_LDS bf16x4*)(stage + l32 * (2 * D) + ch * 16 + 8 * hh) = w;
        }
    asm volatile("" ::: "memory");
    {
        __bf16* O = (__bf16*)p.o + (bhq * N + wq0) * D;
        const int rr = lane >> 4, cc = lane & 15;   // 4 rows of 16 chunks per instruction
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int r = 4 * k + rr;
            const bf16x8 x = *(const ATTN_LDS bf16x8*)(stage + r * (2 * D) + ((cc ^ (r & 15)) * 16));
            if (wq0 + r < N) *(bf16x8*)(O + (size_t)r * D + cc * 8) = x;
        }
    }
    if (row < N && p.lse && hh == 0)
        p.lse[bhq * N + row] = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
}

template __global__ void fwd_fp8_kernel<false>(FwdParams);
template __global__ void fwd_fp8_kernel<true>(FwdParams);

hipError_t launch_fwd_fp8(const FwdParams& p0, int d, hipStream_t st) {
    if (d != 128) return hipErrorNotSupported;
    FwdParams p = p0;
    p.n_qt = (p.Nq + 255) / 256;
    p.n_bh = p.B * p.Hq;
    // Head groups per XCD: as many heads as fill its 32 resident workgroups
    // (at least one), when the heads split evenly over the 8 XCDs and groups.
    p.xgrp = 0;
    if (p.n_bh % 8 == 0) {
        int g = max(1, 32 / p.n_qt);
        while (g > 1 && (p.n_bh / 8) % g) --g;
        p.xgrp = g;
    }
    if (p.Nk % BN) hipLaunchKernelGGL(fwd_fp8_kernel<true>, dim3(p.n_qt * p.n_bh), dim3(512), 0, st, p);
    else hipLaunchKernelGGL(fwd_fp8_kernel<false>, dim3(p.n_qt * p.n_bh), dim3(512), 0, st, p);
    return hipGetLastError();
}

}  // namespace attn
