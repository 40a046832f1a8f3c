// fp32 inputs: the fused forward on the fp32 matrix cores (32x32x2), one wave
// per 32 query rows, K / V tiles staged through LDS with plain loads. Same
// tiling, online softmax and masks as the bf16 kernel; no operand is ever
// rounded below fp32.
#include "fwd_common.h"

namespace attn {

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
