// C ABI of the fused attention forward: argument validation (before any HIP
// call), kernel-instance dispatch and error mapping. The operations and their
// sources are documented in include/attn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

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
hipError_t launch_seq_ids(const int32_t* cu, int num_seqs, int total, int32_t* ids, hipStream_t st);
hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int32_t* table, const int32_t* lens,
                         void* o, float* lse, int B, int Hq, int Hkv, int max_blocks, float scale, int splits,
                         float* workspace, hipStream_t st);
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, float* workspace, int B, int Hq, int Hkv, int N, float scale,
                      int causal, hipStream_t st);
}  // namespace attn

namespace {

constexpr int kKnownMask = ATTN_MASK_CAUSAL | ATTN_MASK_WINDOW | ATTN_MASK_DOC;
constexpr int kFp8Tile = 128;
constexpr long long kMaxElems = (1LL << 40);

bool log_enabled() {
    static const bool on = [] {
        const char* e = std::getenv("ATTN_LOG");
        return e && e[0] && e[0] != '0';
    }();
    return on;
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
    if (log_enabled())
        std::fprintf(stderr, "[attn] fwd dtype=%d B=%d Hq=%d Hkv=%d Nq=%d Nk=%d d=%d mask=%d window=%d "
                             "softcap=%g alibi=%d\n",
                     dtype, B, Hq, Hkv, Nq, Nk, d, mask_kind, p.window, softcap, alibi_slopes != nullptr);
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
    if (log_enabled())
        std::fprintf(stderr, "[attn] fwd_varlen num_seqs=%d total=%d\n", num_seqs, total);
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

size_t attn_decode_workspace_floats(int B, int Hq, int d, int num_splits) {
    if (B < 1 || Hq < 1 || d < 1 || num_splits < 1) return 0;
    if (num_splits == 1) return 0;
    // split outputs and LSEs, then one 32-bit word per sequence (launch order)
    return (size_t)B * Hq * num_splits * (d + 1) + (size_t)B;
}

int attn_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                      const int32_t* seq_lens, void* o, float* lse, int B, int Hq, int Hkv, int d, int block_size,
                      int max_blocks, float scale, int num_splits, float* workspace, int dtype, void* stream) {
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o) return ATTN_ERR_INVALID_ARG;
    if (B < 1 || Hq < 1 || Hkv < 1 || d < 1 || block_size < 1 || max_blocks < 1) return ATTN_ERR_INVALID_ARG;
    if (Hq % Hkv || !std::isfinite(scale) || num_splits < 1 || num_splits > 256) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_F32 && dtype != ATTN_BF16 && dtype != ATTN_FP8_E4M3) return ATTN_ERR_INVALID_ARG;
    if (num_splits > 1 && !workspace) return ATTN_ERR_INVALID_ARG;
    if ((long long)B * Hq * num_splits > (1LL << 31) / 256) return ATTN_ERR_INVALID_ARG;
    if (dtype != ATTN_BF16 || d != 128 || block_size != 16 || Hq / Hkv > 32) return ATTN_ERR_UNSUPPORTED;
    if (log_enabled())
        std::fprintf(stderr, "[attn] decode_paged B=%d Hq=%d Hkv=%d max_blocks=%d splits=%d\n", B, Hq, Hkv,
                     max_blocks, num_splits);
    return hip_status(attn::launch_decode(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, Hq, Hkv,
                                          max_blocks, scale, num_splits, workspace, (hipStream_t)stream));
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
