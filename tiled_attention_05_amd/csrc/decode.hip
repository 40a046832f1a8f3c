// One-token decode over a paged key/value cache, split over the keys.
//
// "Les kernels d'attention rapide et la fusion d'operateurs accelerent les
// modeles d'IA", section "Attention de type FlashAttention et attention
// paginee": the cache is stored in fixed-size blocks and a block table maps
// each logical position to its physical block; the attention kernel
// translates every position through the table. The keys of a sequence are
// split into ranges processed independently; each range returns its
// normalised output and its log-sum-exp, and the exact merge is
// LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
//
// Work: one wave per (sequence, key/value head, split). The G = Hq / Hkv query
// heads of the group play the role of the query rows of the prefill kernel
// (padded to 32): S^T = K Q^T on 32x32x16 bf16 products (a lane owns one head
// and 16 of the 32 keys of a chunk), the same online softmax, O^T += V^T P^T
// with V read transposed from LDS. K fragments are gathered straight into
// registers through the table; V rows are gathered into a per-wave LDS tile by
// direct global->LDS copies (per-lane addresses). The next chunk's loads are in
// flight while the current chunk is computed. Decode reads every key once:
// the kernel is bound by HBM, not by the padded products.
#include <climits>

#include <mutex>

#include "fwd_common.h"

namespace attn {

struct DecodeParams {
    const __bf16* q;         // [B][Hq][128]
    const __bf16* kc;        // [num_blocks][Hkv][16][128]
    const __bf16* vc;
    const int32_t* table;    // [B][max_blocks]
    const int32_t* lens;     // [B]
    __bf16* o;               // [B][Hq][128]
    float* lse;              // [B][Hq] or null
    float* part;             // splits > 1: [B][Hq][splits][128] outputs, then [B][Hq][splits] LSEs
    const int32_t* order;    // [B] sequences longest first, or null for the plain order
    int B, Hq, Hkv, G, max_blocks, splits;
    float scale_log2;
};

constexpr int kPage = 16, kDD = 128, kCh = 32;   // page size, head dim, keys per chunk
constexpr float kDecNoMax = -1e30f;              // initial reference: finite, below any score
constexpr int kOrderMax = 4096;                  // sequences the launch-order kernel ranks

// Launch order of the sequences, longest cached length first (ties: lower
// index first), so that the waves of the longest sequences start first and
// the grid does not end on a few long waves. One workgroup: the lengths are
// staged in LDS and every sequence counts the sequences ahead of it; the order
// is strict and total, so the ranks are a permutation of 0 .. B - 1.
__global__ __launch_bounds__(1024) void decode_order_kernel(const int32_t* lens, int32_t* order, int B) {
    __shared__ int len_lds[kOrderMax];
    for (int j = threadIdx.x; j < B; j += blockDim.x) len_lds[j] = lens[j];
    __syncthreads();
    for (int j = threadIdx.x; j < B; j += blockDim.x) {
        const int lj = len_lds[j];
        int rank = 0;
        for (int c = 0; c < B; ++c) {
            const int lc = len_lds[c];
            rank += (lc > lj || (lc == lj && c < j)) ? 1 : 0;
        }
        order[rank] = j;
    }
}

__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
    using T = Tile<kDD>;
    constexpr int RB = T::ROW_BYTES;   // 256
    __shared__ __attribute__((aligned(1024))) char vt_lds[4][2][kCh * RB];   // per wave, double-buffered

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wid = blockIdx.x * 4 + wave;
    if (wid >= p.B * p.Hkv * p.splits) return;   // whole waves; the kernel has no barrier
    const int split = wid % p.splits;
    const int kvh = (wid / p.splits) % p.Hkv;
    const int slot = wid / (p.splits * p.Hkv);
    // (clamped: a sequence index outside 0 .. B - 1 can never be addressed)
    const int b = p.order ? min(max(p.order[slot], 0), p.B - 1) : slot;
    const int l32 = lane & 31, hh = lane >> 5;
    // cached length, clamped to what the table row can address (a longer
    // length would walk past the row into the next sequence's entries)
    const int L = min(max(p.lens[b], 0), p.max_blocks * kPage);
    const int nch = (L + kCh - 1) / kCh;
    const int cps = (nch + p.splits - 1) / p.splits;
    const int c0 = min(split * cps, nch), c1 = min(c0 + cps, nch);
    const int32_t* table = p.table + (size_t)b * p.max_blocks;
    const size_t head_off = (size_t)kvh * kPage * kDD;
    const size_t block_elems = (size_t)p.Hkv * kPage * kDD;

    // Q fragments (B operand): lane holds head kvh G + l32 (zero beyond G), dims 16 s + 8 hh + 0..7
    const bool qv = l32 < p.G;
    const int h = kvh * p.G + (qv ? l32 : 0);
    bf16x8 qf[8];
    {
        const __bf16* qr = p.q + ((size_t)b * p.Hq + h) * kDD + 8 * hh;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = qv ? *(const bf16x8*)(qr + 16 * s) : bf16x8{};
    }
    // The 32 keys of chunk c lie in pages 2 c and 2 c + 1 (keys past the end
    // are clamped to the last one, whose page is one of the two). Both table
    // entries are read once per chunk through the scalar cache (wave-uniform
    // index): a vector load of the table would have to be waited for with a
    // vmcnt that also drains every copy already in flight.
    const int last_page = (L - 1) / kPage;
    auto pages = [&](int c, int& pg0, int& pg1) __attribute__((always_inline)) {
        const ATTN_CONST int32_t* t = (const ATTN_CONST int32_t*)table;
        pg0 = t[2 * c];
        pg1 = t[min(2 * c + 1, last_page)];
    };
    // row of key `key` of chunk c (clamped into the sequence) in a cache
    auto row_of = [&](const __bf16* cache, int c, int pg0, int pg1, int key) __attribute__((always_inline)) {
        const int kk = min(key, L - 1);
        const int pg = (kk / kPage == 2 * c) ? pg0 : pg1;
        return cache + (size_t)pg * block_elems + head_off + (size_t)(kk % kPage) * kDD;
    };
    // V transposed reads (as the prefill kernel, one 32-key block): lane L of a
    // 16-lane group addresses row 4 hh + L / 4 (+ 16 u, + 8 for the high half),
    // columns 32 t + 16 cg + 4 (L % 4)
    int vofs[4];
    {
        const int Ln = lane & 15, cg = (lane >> 4) & 1;
        const int r = 4 * hh + (Ln >> 2);
        const int col = 16 * cg + 4 * (Ln & 3);
        const int v0 = r * RB + ((((col * 2) >> 4) ^ T::swz_v(r)) << 4) + ((col * 2) & 15);
#pragma unroll
        for (int t = 0; t < 4; ++t) vofs[t] = v0 ^ (64 * t);
    }

    bf16x8 kf[8];
    auto load_k = [&](int c, int pg0, int pg1) __attribute__((always_inline)) {
        const __bf16* kr = row_of(p.kc, c, pg0, pg1, c * kCh + l32) + 8 * hh;
#pragma unroll
        for (int s = 0; s < 8; ++s) kf[s] = *(const bf16x8*)(kr + 16 * s);
    };
    // V tile of chunk c into buffer c & 1: slot i 64 + lane = (row, 16-byte chunk), swizzled like the prefill tile
    auto load_v = [&](int c, int pg0, int pg1) __attribute__((always_inline)) {
        const unsigned base = lds_addr((ATTN_LDS char*)vt_lds[wave][c & 1]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int slot = i * 64 + lane, r = slot >> 4, pc = slot & 15;
            const __bf16* src = row_of(p.vc, c, pg0, pg1, c * kCh + r) + 8 * (pc ^ T::swz_v(r));
            dma16(src, base + i * 1024);
        }
    };

    f32x16 o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = f32x16{};
    float m = kDecNoMax, l = 0.f;

    if (c0 < c1) {
        int pg0, pg1;
        pages(c0, pg0, pg1);
        load_k(c0, pg0, pg1);
        load_v(c0, pg0, pg1);
    }
    for (int c = c0; c < c1; ++c) {
        // this chunk's K registers and V tile have landed; then the next chunk's loads go out
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        f32x16 s = f32x16{};
#pragma unroll
        for (int st = 0; st < 8; ++st) s = mfma_bf16(kf[st], qf[st], s);
        if (c + 1 < c1) {
            int pg0, pg1;
            pages(c + 1, pg0, pg1);
            load_k(c + 1, pg0, pg1);
            load_v(c + 1, pg0, pg1);
        }
        const int kv0 = c * kCh;
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 8 * (r >> 2) + 4 * hh + (r & 3);
            s[r] = key < L ? s[r] * p.scale_log2 : -INFINITY;
            mx = fmaxf(mx, s[r]);
        }
        mx = xhalf_max(mx);
        const float mn = fmaxf(m, mx);
        const float alpha = fast_exp2(m - mn);
        m = mn;
        float ls = 0.f;
        bf16x8 pf[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pr = fast_exp2(s[r] - m);
            ls += pr;
            pf[r >> 3][r & 7] = (__bf16)pr;
        }
        l = l * alpha + ls;
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] *= alpha;
        const ATTN_LDS char* vb = (const ATTN_LDS char*)vt_lds[wave][c & 1];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const ATTN_LDS char* a = vb + vofs[t] + 16 * u * RB;
                const bf16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4*)a);
                const bf16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((ATTN_LDS bf16x4*)(a + 8 * RB));
                o[t] = mfma_bf16(__builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7), pf[u], o[t]);
            }
        // the next iteration refills the other buffer only after its own wait,
        // by which time these reads have returned
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }

    const float lt = xhalf_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    if (!qv) return;
    const size_t bh = (size_t)b * p.Hq + h;
    if (p.splits == 1) {
        __bf16* orow = p.o + bh * kDD + 4 * hh;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                bf16x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[t][4 * gq + e] * inv);
                *(bf16x4*)(orow + 32 * t + 8 * gq) = w;
            }
        if (p.lse && hh == 0) p.lse[bh] = lse_v;
    } else {
        float* po = p.part + (bh * p.splits + split) * kDD + 4 * hh;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                f32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = o[t][4 * gq + e] * inv;
                *(f32x4*)(po + 32 * t + 8 * gq) = w;
            }
        if (hh == 0) p.part[(size_t)p.B * p.Hq * p.splits * kDD + bh * p.splits + split] = lse_v;
    }
}

// Exact merge of the splits: one workgroup per (sequence, head), thread = dim.
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeParams p) {
    const size_t bh = blockIdx.x;
    const int d = threadIdx.x;
    const float* ls = p.part + (size_t)p.B * p.Hq * p.splits * kDD + bh * p.splits;
    float mx = -INFINITY;
    for (int s = 0; s < p.splits; ++s) mx = fmaxf(mx, ls[s]);
    float acc = 0.f, den = 0.f;
    if (mx > -INFINITY) {
        for (int s = 0; s < p.splits; ++s) {
            const float w = __expf(ls[s] - mx);   // 0 for an empty split (LSE = -inf)
            den += w;
            acc += w * p.part[(bh * p.splits + s) * kDD + d];
        }
    }
    p.o[bh * kDD + d] = (__bf16)(den > 0.f ? acc / den : 0.f);
    if (p.lse && d == 0) p.lse[bh] = den > 0.f ? mx + __logf(den) : -INFINITY;
}

hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int32_t* table, const int32_t* lens,
                         void* o, float* lse, int B, int Hq, int Hkv, int max_blocks, float scale, int splits,
                         float* workspace, hipStream_t st) {
    DecodeParams p{};
    p.q = (const __bf16*)q;
    p.kc = (const __bf16*)kc;
    p.vc = (const __bf16*)vc;
    p.table = table;
    p.lens = lens;
    p.o = (__bf16*)o;
    p.lse = lse;
    p.part = workspace;
    p.order = nullptr;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.max_blocks = max_blocks; p.splits = splits;
    p.scale_log2 = scale * kLog2e;
    const long long waves = (long long)B * Hkv * splits;
    if (splits > 1 && B <= kOrderMax) {
        // the order lives after the split outputs and LSEs in the workspace
        int32_t* order = (int32_t*)(workspace + (size_t)B * Hq * splits * (kDD + 1));
        hipLaunchKernelGGL(decode_order_kernel, dim3(1), dim3(1024), 0, st, lens, order, B);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        p.order = order;
    }
    hipLaunchKernelGGL(decode_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)(B * Hq)), dim3(128), 0, st, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Workspace without allocation: a fixed device array holding the split
// outputs, LSEs and launch order of attn_decode_paged_noalloc. Every GPU the
// library runs on keeps its own copy until the process ends. In host code the
// array's name is not a device address: the address is looked up once per
// device (with that device current) and only that pointer is handed to the
// kernels. Calls on one GPU share the array, so calls that overlap in time on
// one GPU (concurrent streams) race; every entry a call reads is written
// earlier in the same call, so nothing needs clearing between calls.
constexpr size_t kDecodeScratchFloats = size_t(4) << 20;   // 16 MiB
static __device__ __align__(256) float scratch[kDecodeScratchFloats];

size_t decode_scratch_floats() { return kDecodeScratchFloats; }

static float* scratch_ptr_for_current_device(hipError_t& err) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static float* ptrs[kMaxDevices] = {};
    int dev = 0;
    err = hipGetDevice(&dev);
    if (err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* ptr = nullptr;
        err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return nullptr;
        ptrs[dev] = (float*)ptr;
    }
    return ptrs[dev];
}

hipError_t launch_decode_noalloc(const void* q, const void* kc, const void* vc, const int32_t* table,
                                 const int32_t* lens, void* o, float* lse, int B, int Hq, int Hkv, int max_blocks,
                                 float scale, int splits, hipStream_t st) {
    float* ws = nullptr;
    if (splits > 1) {
        hipError_t e;
        ws = scratch_ptr_for_current_device(e);
        if (!ws) return e;
    }
    return launch_decode(q, kc, vc, table, lens, o, lse, B, Hq, Hkv, max_blocks, scale, splits, ws, st);
}

}  // namespace attn
