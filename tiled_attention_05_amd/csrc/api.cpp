// C ABI of the fused attention forward: argument validation (before any HIP
// call), kernel-instance dispatch and error mapping. The operations and their
// sources are documented in include/attn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/attn.h"
#include "fwd_params.h"

namespace attn {
hipError_t launch_fwd_bf16(const FwdParams& p, int d, hipStream_t st);
hipError_t launch_fwd_f32(const FwdParams& p, int d, hipStream_t st);
hipError_t launch_fwd_fp8(const FwdParams& p, int d, hipStream_t st);
hipError_t launch_fp8_prepare(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int N,
                              int d, const int8_t* signs, const float* rope_cos, const float* rope_sin, void* q8,
                              void* k8, void* v8, hipStream_t st);
hipError_t launch_block_mask(int B, int Nq, int Nk, int mask, int window, const int32_t* doc, int bm,
                             int bn, void* out, hipStream_t st);
hipError_t launch_fwd_plan(int B, int Nq, int Nk, int mask, int window, const int32_t* doc, int8_t* kinds,
                           hipStream_t st);
hipError_t launch_seq_ids(const int32_t* cu, int num_seqs, int total, int32_t* ids, hipStream_t st);
hipError_t launch_varlen_tiles(const int32_t* cu, int n_seq, int bm, int32_t* items, int n_list, hipStream_t st);
constexpr int kVarlenMaxSeqs = 4096, kVarlenMaxTiles = 4096;   // as in varlen.hip
hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int32_t* table, const int32_t* lens,
                         void* o, float* lse, int B, int Hq, int Hkv, int max_blocks, float scale, int splits,
                         float* workspace, hipStream_t st);
hipError_t launch_decode_noalloc(const void* q, const void* kc, const void* vc, const int32_t* table,
                                 const int32_t* lens, void* o, float* lse, int B, int Hq, int Hkv, int max_blocks,
                                 float scale, int splits, hipStream_t st);
size_t decode_scratch_floats();
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, float* workspace, int B, int Hq, int Hkv, int N, float scale,
                      int causal, hipStream_t st);
}  // namespace attn

namespace {

constexpr int kKnownMask = ATTN_MASK_CAUSAL | ATTN_MASK_WINDOW | ATTN_MASK_DOC;
constexpr int kFp8Tile = 128;
constexpr long long kMaxElems = (1LL << 40);

bool env_flag(const char* name) {
    const char* e = std::getenv(name);
    return e && e[0] && e[0] != '0';
}

bool log_enabled() {
    static const bool on = env_flag("ATTN_LOG");
    return on;
}

// ATTN_CHECK=1: debug-only synchronous checks of preconditions on device data
// (document ids non-decreasing, sequence offsets monotone). They copy the data
// to the host and synchronise the stream, so they must not be enabled under
// graph capture.
bool check_enabled() {
    static const bool on = env_flag("ATTN_CHECK");
    return on;
}

// Copies n int32 values from the device (stream-ordered, then waits).
int fetch_i32(const int32_t* dev, size_t n, void* stream, std::vector<int32_t>& host) {
    host.resize(n);
    hipStream_t st = (hipStream_t)stream;
    if (hipMemcpyAsync(host.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return ATTN_ERR_HIP;
    return ATTN_OK;
}

// Tile counts of the bf16 / fp32 forward's schedule (blocks of 32 query rows,
// one per wave, by 64-key tiles), the same rules as the kernels' range and
// full-tile functions: a tile outside the rows' contiguous key range is
// empty (skipped), one whose pairs are all allowed is full, the rest partial.
struct PlanCounts {
    long long empty = 0, partial = 0, full = 0;
};
PlanCounts plan_counts(int B, int Nq, int Nk, int mask, int W, const std::vector<int32_t>* docs) {
    constexpr int RB = 32, BN = 64;
    PlanCounts c;
    const int off = Nk - Nq, n_kt = (Nk + BN - 1) / BN;
    for (int b = 0; b < B; ++b) {
        const int32_t* d = docs ? docs->data() + (size_t)b * Nk : nullptr;
        for (int r0 = 0; r0 < Nq; r0 += RB) {
            const int r1 = std::min(r0 + RB, Nq) - 1;
            int lo = 0, hi = Nk, dq0 = 0, dq1 = 0;
            if (mask & ATTN_MASK_CAUSAL) hi = std::min(hi, r1 + off + 1);
            if (mask & ATTN_MASK_WINDOW) lo = std::max(lo, r0 + off - W + 1);
            if (d) {
                dq0 = d[r0];
                dq1 = d[r1];
                lo = std::max(lo, (int)(std::lower_bound(d, d + Nk, dq0) - d));
                hi = std::min(hi, (int)(std::upper_bound(d, d + Nk, dq1) - d));
            }
            const int t0 = hi > lo ? lo / BN : 0, t1 = hi > lo ? (hi + BN - 1) / BN : 0;
            c.empty += n_kt - (t1 - t0);
            for (int kt = t0; kt < t1; ++kt) {
                const int j0 = kt * BN, j1 = std::min(j0 + BN, Nk) - 1;
                bool full = j0 + BN <= Nk;
                if (mask & ATTN_MASK_CAUSAL) full &= j1 <= r0 + off;
                if (mask & ATTN_MASK_WINDOW) full &= (r1 + off) - j0 < W;
                if (d) full &= d[j0] == d[j1] && dq0 == dq1 && d[j0] == dq0;
                (full ? c.full : c.partial) += 1;
            }
        }
    }
    return c;
}

// Mask / size checks shared by attn_fwd and the block-mask builder.
int check_mask(int Nq, int Nk, int mask_kind, int window, const int32_t* doc_ids) {
    if (mask_kind & ~kKnownMask) return ATTN_ERR_INVALID_ARG;
    if ((mask_kind & ATTN_MASK_WINDOW) && window < 1) return ATTN_ERR_INVALID_ARG;
    if ((mask_kind & ATTN_MASK_DOC) && doc_ids == nullptr) return ATTN_ERR_INVALID_ARG;
    if ((mask_kind & ATTN_MASK_WINDOW) && !(mask_kind & ATTN_MASK_CAUSAL)) return ATTN_ERR_UNSUPPORTED;
    if ((mask_kind & ATTN_MASK_DOC) && Nq != Nk) return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return ATTN_OK;
    if (e == hipErrorNotSupported) return ATTN_ERR_UNSUPPORTED;
    if (log_enabled()) std::fprintf(stderr, "[attn] HIP error: %s\n", hipGetErrorString(e));
    return ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_INVALID_ARG: return "invalid argument";
        case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
        case ATTN_ERR_HIP: return "HIP runtime or launch error";
        default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// Every check of attn_fwd, with no HIP call.
int fwd_check(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Nq, int Nk,
              int d, float scale, int mask_kind, int window, const int32_t* doc_ids, float softcap,
              const float* alibi_slopes, int dtype) {
    if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1) return ATTN_ERR_INVALID_ARG;
    if (Hq % Hkv) return ATTN_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
    if (!std::isfinite(softcap) || softcap < 0.f) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return ATTN_ERR_INVALID_ARG;
    if ((long long)B * Hq * Nq * d > kMaxElems || (long long)B * Hkv * Nk * d > kMaxElems)
        return ATTN_ERR_INVALID_ARG;
    if (const int r = check_mask(Nq, Nk, mask_kind, window, doc_ids)) return r;
    if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (dtype == ATTN_FP8_E4M3 &&
        (d != 128 || Nq != Nk || mask_kind != 0 || softcap != 0.f || alibi_slopes != nullptr))
        return ATTN_ERR_UNSUPPORTED;
    return ATTN_OK;
}

int fwd_launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
               int Nq, int Nk, int d, float scale, int mask_kind, int window, const int32_t* doc_ids,
               float softcap, const float* alibi_slopes, int dtype, void* stream) {
    attn::FwdParams p{};
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
    p.doc = (mask_kind & ATTN_MASK_DOC) ? doc_ids : nullptr;
    p.slopes = alibi_slopes;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.Nq = Nq; p.Nk = Nk;
    p.group = Hq / Hkv;
    p.mask = mask_kind;
    p.window = (mask_kind & ATTN_MASK_WINDOW) ? window : 0;
    p.scale = scale;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.softcap = softcap;
    p.npad = (Nk + kFp8Tile - 1) / kFp8Tile * kFp8Tile;
    hipStream_t st = (hipStream_t)stream;
    std::vector<int32_t> docs;
    if ((check_enabled() || log_enabled()) && (mask_kind & ATTN_MASK_DOC)) {
        if (fetch_i32(doc_ids, (size_t)B * Nk, stream, docs)) return ATTN_ERR_HIP;
        if (check_enabled())
            for (int b = 0; b < B; ++b)
                for (int j = 1; j < Nk; ++j)
                    if (docs[(size_t)b * Nk + j] < docs[(size_t)b * Nk + j - 1]) {
                        if (log_enabled())
                            std::fprintf(stderr, "[attn] ATTN_CHECK: doc_ids[%d] decreases at %d\n", b, j);
                        return ATTN_ERR_INVALID_ARG;
                    }
    }
    if (log_enabled()) {
        const int n_qt = (Nq + 255) / 256;
        std::fprintf(stderr, "[attn] fwd dtype=%d B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d mask=%d window=%d "
                             "softcap=%g alibi=%d grid=%lld x 512 threads\n",
                     dtype, B, Hq, Hkv, Nq, Nk, d, mask_kind, p.window, softcap, alibi_slopes != nullptr,
                     (long long)n_qt * B * Hq);
        const PlanCounts c = plan_counts(B, Nq, Nk, mask_kind, p.window, docs.empty() ? nullptr : &docs);
        const long long tot = c.empty + c.partial + c.full;
        std::fprintf(stderr, "[attn] tiles per query head (32 rows x 64 keys): empty=%lld partial=%lld full=%lld "
                             "skip=%.4f\n",
                     c.empty, c.partial, c.full, tot ? (double)c.empty / tot : 0.0);
    }
    hipError_t e;
    if (dtype == ATTN_BF16) e = attn::launch_fwd_bf16(p, d, st);
    else if (dtype == ATTN_F32) e = attn::launch_fwd_f32(p, d, st);
    else e = attn::launch_fwd_fp8(p, d, st);
    return hip_status(e);
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
             int Nq, int Nk, int d, float scale, int mask_kind, int window, const int32_t* doc_ids,
             float softcap, const float* alibi_slopes, int dtype, void* stream) {
    if (const int r = fwd_check(q, k, v, o, B, Hq, Hkv, Nq, Nk, d, scale, mask_kind, window, doc_ids, softcap,
                                alibi_slopes, dtype))
        return r;
    return fwd_launch(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, mask_kind, window, doc_ids, softcap,
                      alibi_slopes, dtype, stream);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens, int num_seqs, int total, int Hq, int Hkv, int d, float scale,
                    int mask_kind, int window, float softcap, const float* alibi_slopes, int32_t* workspace,
                    int dtype, void* stream) {
    if (!cu_seqlens || !workspace || num_seqs < 1 || total < 1) return ATTN_ERR_INVALID_ARG;
    if (mask_kind & ~(ATTN_MASK_CAUSAL | ATTN_MASK_WINDOW)) return ATTN_ERR_INVALID_ARG;
    if (dtype == ATTN_FP8_E4M3) return ATTN_ERR_UNSUPPORTED;
    const int mask = mask_kind | ATTN_MASK_DOC;
    if (const int r = fwd_check(q, k, v, o, 1, Hq, Hkv, total, total, d, scale, mask, window, workspace,
                                softcap, alibi_slopes, dtype))
        return r;
    if (check_enabled()) {   // offsets: 0 first, non-decreasing, total last
        std::vector<int32_t> cu;
        if (fetch_i32(cu_seqlens, (size_t)num_seqs + 1, stream, cu)) return ATTN_ERR_HIP;
        bool ok = cu[0] == 0 && cu[num_seqs] == total;
        for (int s2 = 1; s2 <= num_seqs; ++s2) ok &= cu[s2] >= cu[s2 - 1];
        if (!ok) return ATTN_ERR_INVALID_ARG;
    }
    // bf16: each sequence tiled on its own (256-row query tiles that never
    // straddle two sequences), when the tile list fits the workspace; else
    // (and for fp32) the document mask over the concatenation.
    constexpr int kBM = 256;
    const long long n_list = (total + kBM - 1) / kBM + (long long)num_seqs;
    const bool per_seq = dtype == ATTN_BF16 && num_seqs <= attn::kVarlenMaxSeqs &&
                         (total + kBM - 1) / kBM <= attn::kVarlenMaxTiles && n_list <= total;
    if (log_enabled())
        std::fprintf(stderr, "[attn] fwd_varlen num_seqs=%d total=%d tiling=%s\n", num_seqs, total,
                     per_seq ? "per-sequence" : "document-mask");
    if (per_seq) {
        if (const int r = hip_status(attn::launch_varlen_tiles(cu_seqlens, num_seqs, kBM, workspace, (int)n_list,
                                                               (hipStream_t)stream)))
            return r;
        attn::FwdParams p{};
        p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
        p.slopes = alibi_slopes;
        p.B = 1; p.Hq = Hq; p.Hkv = Hkv; p.Nq = total; p.Nk = total;
        p.group = Hq / Hkv;
        p.mask = mask_kind;
        p.window = (mask_kind & ATTN_MASK_WINDOW) ? window : 0;
        p.scale = scale;
        p.scale_log2 = scale * 1.4426950408889634f;
        p.softcap = softcap;
        p.items = workspace; p.cu = cu_seqlens; p.n_seq = num_seqs; p.n_list = (int)n_list;
        return hip_status(attn::launch_fwd_bf16(p, d, (hipStream_t)stream));
    }
    if (const int r = hip_status(attn::launch_seq_ids(cu_seqlens, num_seqs, total, workspace, (hipStream_t)stream)))
        return r;
    return fwd_launch(q, k, v, o, lse, 1, Hq, Hkv, total, total, d, scale, mask, window, workspace, softcap,
                      alibi_slopes, dtype, stream);
}

size_t attn_fp8_buffer_bytes(int B, int H, int N, int d) {
    if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
    const size_t np = (size_t)(N + kFp8Tile - 1) / kFp8Tile * kFp8Tile;
    const size_t plane = (size_t)B * H * np * d;   // value codes, then residual codes
    return 2 * plane + (size_t)B * H * (np / kFp8Tile) * sizeof(float);
}

int attn_fp8_prepare(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int N, int d,
                     const int8_t* signs, void* q8, void* k8, void* v8, void* stream) {
    if (!q || !k || !v || !q8 || !k8 || !v8) return ATTN_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || d < 1 || Hq % Hkv) return ATTN_ERR_INVALID_ARG;
    if ((long long)B * Hq * N * d > kMaxElems) return ATTN_ERR_INVALID_ARG;
    if (d != 128) return ATTN_ERR_UNSUPPORTED;
    return hip_status(attn::launch_fp8_prepare(q, k, v, B, Hq, Hkv, N, d, signs, nullptr, nullptr, q8, k8, v8,
                                               (hipStream_t)stream));
}

int attn_fp8_prepare_rope(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int N, int d,
                          const int8_t* signs, const float* rope_cos, const float* rope_sin, void* q8, void* k8,
                          void* v8, void* stream) {
    if (!rope_cos || !rope_sin) return ATTN_ERR_INVALID_ARG;
    if (!q || !k || !v || !q8 || !k8 || !v8) return ATTN_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || d < 1 || Hq % Hkv) return ATTN_ERR_INVALID_ARG;
    if ((long long)B * Hq * N * d > kMaxElems) return ATTN_ERR_INVALID_ARG;
    if (d != 128) return ATTN_ERR_UNSUPPORTED;
    return hip_status(attn::launch_fp8_prepare(q, k, v, B, Hq, Hkv, N, d, signs, rope_cos, rope_sin, q8, k8, v8,
                                               (hipStream_t)stream));
}

size_t attn_block_mask_bytes(int B, int Nq, int Nk, int block_m, int block_n) {
    if (B < 1 || Nq < 1 || Nk < 1 || block_m < 1 || block_n < 1 || block_m > 4096 || block_n > 4096)
        return 0;
    const size_t nq = (size_t)(Nq + block_m - 1) / block_m, nk = (size_t)(Nk + block_n - 1) / block_n;
    const size_t kinds = ((size_t)B * nq * nk + 15) / 16 * 16;
    return kinds + (size_t)B * nq * 3 * sizeof(int32_t) + sizeof(int32_t);
}

int attn_block_mask_build(int B, int Nq, int Nk, int mask_kind, int window, const int32_t* doc_ids,
                          int block_m, int block_n, void* out, void* stream) {
    if (!out) return ATTN_ERR_INVALID_ARG;
    if (B < 1 || Nq < 1 || Nk < 1) return ATTN_ERR_INVALID_ARG;
    if (block_m < 1 || block_n < 1 || block_m > 4096 || block_n > 4096) return ATTN_ERR_INVALID_ARG;
    if (const int r = check_mask(Nq, Nk, mask_kind, window, doc_ids)) return r;
    return hip_status(attn::launch_block_mask(B, Nq, Nk, mask_kind,
                                              (mask_kind & ATTN_MASK_WINDOW) ? window : 0,
                                              (mask_kind & ATTN_MASK_DOC) ? doc_ids : nullptr, block_m,
                                              block_n, out, (hipStream_t)stream));
}

size_t attn_fwd_tile_kinds_bytes(int B, int Nq, int Nk) {
    if (B < 1 || Nq < 1 || Nk < 1) return 0;
    return (size_t)B * ((Nq + 31) / 32) * ((Nk + 63) / 64);
}

int attn_fwd_tile_kinds(int B, int Nq, int Nk, int mask_kind, int window, const int32_t* doc_ids, int8_t* out,
                        void* stream) {
    if (!out || B < 1 || Nq < 1 || Nk < 1) return ATTN_ERR_INVALID_ARG;
    if (const int r = check_mask(Nq, Nk, mask_kind, window, doc_ids)) return r;
    return hip_status(attn::launch_fwd_plan(B, Nq, Nk, mask_kind, (mask_kind & ATTN_MASK_WINDOW) ? window : 0,
                                            (mask_kind & ATTN_MASK_DOC) ? doc_ids : nullptr, out,
                                            (hipStream_t)stream));
}

size_t attn_decode_workspace_floats(int B, int Hq, int d, int num_splits) {
    if (B < 1 || Hq < 1 || d < 1 || num_splits < 1) return 0;
    if (num_splits == 1) return 0;
    // split outputs and LSEs, then one 32-bit word per sequence (launch order)
    return (size_t)B * Hq * num_splits * (d + 1) + (size_t)B;
}

}  // extern "C"

namespace {

// Every check of attn_decode_paged except the workspace, with no HIP call
// other than ATTN_CHECK's length copy.
int decode_check(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                 const int32_t* seq_lens, const void* o, int B, int Hq, int Hkv, int d, int block_size,
                 int max_blocks, float scale, int num_splits, int dtype, void* stream) {
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o) return ATTN_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || d < 1 || block_size < 1 || max_blocks < 1) return ATTN_ERR_INVALID_ARG;
    if (Hq % Hkv || !std::isfinite(scale) || num_splits < 1 || num_splits > 256) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return ATTN_ERR_INVALID_ARG;
    if ((long long)B * Hq * num_splits > (1LL << 31) / 256) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_BF16 || d != 128 || block_size != 16 || Hq / Hkv > 32) return ATTN_ERR_UNSUPPORTED;
    if (check_enabled()) {   // cached lengths within the table's capacity
        std::vector<int32_t> lens;
        if (fetch_i32(seq_lens, (size_t)B, stream, lens)) return ATTN_ERR_HIP;
        for (int b = 0; b < B; ++b)
            if (lens[b] < 0 || (long long)lens[b] > (long long)max_blocks * block_size) return ATTN_ERR_INVALID_ARG;
    }
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                      const int32_t* seq_lens, void* o, float* lse, int B, int Hq, int Hkv, int d, int block_size,
                      int max_blocks, float scale, int num_splits, float* workspace, int dtype, void* stream) {
    if (const int r = decode_check(q, k_cache, v_cache, block_table, seq_lens, o, B, Hq, Hkv, d, block_size,
                                   max_blocks, scale, num_splits, dtype, stream))
        return r;
    if (num_splits > 1 && !workspace) return ATTN_ERR_INVALID_ARG;
    if (log_enabled())
        std::fprintf(stderr, "[attn] decode_paged B=%d Hq=%d Hkv=%d max_blocks=%d splits=%d\n", B, Hq, Hkv,
                     max_blocks, num_splits);
    return hip_status(attn::launch_decode(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, Hq, Hkv,
                                          max_blocks, scale, num_splits, workspace, (hipStream_t)stream));
}

int attn_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, void* o, float* lse, int B, int Hq, int Hkv, int d,
                              int block_size, int max_blocks, float scale, int num_splits, int dtype, void* stream) {
    if (const int r = decode_check(q, k_cache, v_cache, block_table, seq_lens, o, B, Hq, Hkv, d, block_size,
                                   max_blocks, scale, num_splits, dtype, stream))
        return r;
    const size_t need = attn_decode_workspace_floats(B, Hq, d, num_splits);
    if (need > attn::decode_scratch_floats()) {
        if (log_enabled())
            std::fprintf(stderr, "[attn] decode_paged_noalloc: %zu workspace floats needed, the fixed scratch "
                                 "holds %zu\n", need, attn::decode_scratch_floats());
        return ATTN_ERR_INVALID_ARG;
    }
    if (log_enabled())
        std::fprintf(stderr, "[attn] decode_paged_noalloc B=%d Hq=%d Hkv=%d max_blocks=%d splits=%d\n", B, Hq, Hkv,
                     max_blocks, num_splits);
    return hip_status(attn::launch_decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, Hq, Hkv,
                                                  max_blocks, scale, num_splits, (hipStream_t)stream));
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, float* workspace, int B, int Hq, int Hkv, int N, int d, float scale,
             int mask_kind, int dtype, void* stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return ATTN_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || d < 1 || Hq % Hkv) return ATTN_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return ATTN_ERR_INVALID_ARG;
    if (mask_kind & ~kKnownMask) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return ATTN_ERR_INVALID_ARG;
    if ((long long)B * Hq * N * d > kMaxElems) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_BF16 || d != 128 || (mask_kind & ~ATTN_MASK_CAUSAL)) return ATTN_ERR_UNSUPPORTED;
    if (log_enabled())
        std::fprintf(stderr, "[attn] bwd B=%d Hq=%d Hkv=%d N=%d mask=%d\n", B, Hq, Hkv, N, mask_kind);
    return hip_status(attn::launch_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, Hq, Hkv, N, scale,
                                       mask_kind & ATTN_MASK_CAUSAL, (hipStream_t)stream));
}

}  // extern "C"
