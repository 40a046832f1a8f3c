// Host-only driver of the C ABI's validation code (csrc/api.cpp), built with
// g++ under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_abi_sanitize.py. The kernel launchers are replaced by stubs that
// count their calls, so no GPU and no HIP kernel is involved: every invalid
// call must return its status without reaching a launcher, every valid call
// must reach exactly one, and the host-side tile counting of ATTN_LOG runs on
// a range of shapes.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "../include/attn.h"

namespace attn {
struct FwdParams;
static int launches = 0;
hipError_t launch_fwd_bf16(const FwdParams&, int, hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_fwd_f32(const FwdParams&, int, hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_fwd_fp8(const FwdParams&, int, hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_fp8_prepare(const void*, const void*, const void*, int, int, int, int, int, const int8_t*,
                              const float*, const float*, void*, void*, void*, hipStream_t) {
    ++launches;
    return hipSuccess;
}
hipError_t launch_block_mask(int, int, int, int, int, const int32_t*, int, int, void*, hipStream_t) {
    ++launches;
    return hipSuccess;
}
hipError_t launch_fwd_plan(int, int, int, int, int, const int32_t*, int8_t*, hipStream_t) {
    ++launches;
    return hipSuccess;
}
hipError_t launch_seq_ids(const int32_t*, int, int, int32_t*, hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_varlen_tiles(const int32_t*, int, int, int32_t*, int, hipStream_t) { ++launches; return hipSuccess; }
hipError_t launch_decode(const void*, const void*, const void*, const int32_t*, const int32_t*, void*, float*, int,
                         int, int, int, float, int, float*, hipStream_t) {
    ++launches;
    return hipSuccess;
}
hipError_t launch_decode_noalloc(const void*, const void*, const void*, const int32_t*, const int32_t*, void*,
                                 float*, int, int, int, int, float, int, hipStream_t) {
    ++launches;
    return hipSuccess;
}
size_t decode_scratch_floats() { return size_t(4) << 20; }
hipError_t launch_bwd(const void*, const void*, const void*, const void*, const void*, const float*, void*, void*,
                      void*, float*, int, int, int, int, float, int, hipStream_t) {
    ++launches;
    return hipSuccess;
}
}  // namespace attn

static int failures = 0;
#define EXPECT(call, want, n_launch)                                                                   \
    do {                                                                                               \
        const int before = attn::launches;                                                             \
        const int got = (call);                                                                        \
        if (got != (want) || attn::launches - before != (n_launch)) {                                  \
            std::fprintf(stderr, "line %d: %s -> %d (want %d), launches %d (want %d)\n", __LINE__, #call, \
                         got, (int)(want), attn::launches - before, (int)(n_launch));                  \
            ++failures;                                                                                \
        }                                                                                              \
    } while (0)

int main() {
    char buf[64];
    void* P = buf;   // never dereferenced: the launchers are stubs
    const int32_t* D = (const int32_t*)buf;
    const float nan = std::nanf("");
    // attn_fwd: valid calls reach one launcher
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1, 2, 2, 16, 16, 128, 0.1f, 0, 0, nullptr, 0.f, nullptr, ATTN_BF16, nullptr),
           ATTN_OK, 1);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 2, 8, 2, 1000, 1000, 64, 0.1f, ATTN_MASK_CAUSAL | ATTN_MASK_WINDOW, 33,
                    nullptr, 5.f, (const float*)P, ATTN_F32, nullptr),
           ATTN_OK, 1);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1, 2, 2, 300, 300, 128, 0.1f, 0, 0, nullptr, 0.f, nullptr, ATTN_FP8_E4M3,
                    nullptr),
           ATTN_OK, 1);
    // invalid arguments: no launch
    EXPECT(attn_fwd(nullptr, P, P, P, nullptr, 1, 2, 2, 16, 16, 128, 0.1f, 0, 0, nullptr, 0.f, nullptr, 1, nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 0, 2, 2, 16, 16, 128, 0.1f, 0, 0, nullptr, 0.f, nullptr, 1, nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1, 3, 2, 16, 16, 128, 0.1f, 0, 0, nullptr, 0.f, nullptr, 1, nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1, 2, 2, 16, 16, 128, nan, 0, 0, nullptr, 0.f, nullptr, 1, nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1, 2, 2, 16, 16, 128, 0.1f, 0, 0, nullptr, -1.f, nullptr, 1, nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1, 2, 2, 16, 16, 128, 0.1f, 8, 0, nullptr, 0.f, nullptr, 1, nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1, 2, 2, 16, 16, 128, 0.1f, ATTN_MASK_DOC, 0, nullptr, 0.f, nullptr, 1,
                    nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1, 2, 2, 16, 16, 128, 0.1f, 0, 0, nullptr, 0.f, nullptr, 7, nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1 << 20, 1 << 10, 1 << 10, 1 << 10, 1 << 10, 128, 0.1f, 0, 0, nullptr,
                    0.f, nullptr, 1, nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    // unsupported: no launch
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1, 2, 2, 16, 16, 96, 0.1f, 0, 0, nullptr, 0.f, nullptr, 1, nullptr),
           ATTN_ERR_UNSUPPORTED, 0);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1, 2, 2, 16, 16, 128, 0.1f, ATTN_MASK_WINDOW, 4, nullptr, 0.f, nullptr, 1,
                    nullptr),
           ATTN_ERR_UNSUPPORTED, 0);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1, 2, 2, 16, 20, 128, 0.1f, ATTN_MASK_DOC, 0, D, 0.f, nullptr, 1, nullptr),
           ATTN_ERR_UNSUPPORTED, 0);
    EXPECT(attn_fwd(P, P, P, P, nullptr, 1, 2, 2, 16, 16, 128, 0.1f, ATTN_MASK_CAUSAL, 0, nullptr, 0.f, nullptr,
                    ATTN_FP8_E4M3, nullptr),
           ATTN_ERR_UNSUPPORTED, 0);
    // varlen, prepare, block mask, plan, decode, backward
    // bf16 varlen: the tile list, then the forward; fp32 varlen: the sequence
    // index, then the document-mask forward -- with ATTN_LOG that forward
    // copies the document ids to the host, which with no device fails, after
    // the sequence-index launch, as ATTN_ERR_HIP
    const char* lg = std::getenv("ATTN_LOG");
    const bool log = lg && lg[0] && lg[0] != '0';
    EXPECT(attn_fwd_varlen(P, P, P, P, nullptr, D, 3, 100, 4, 2, 128, 0.1f, ATTN_MASK_CAUSAL, 0, 0.f, nullptr,
                           (int32_t*)P, ATTN_BF16, nullptr),
           ATTN_OK, 2);
    EXPECT(attn_fwd_varlen(P, P, P, P, nullptr, D, 3, 100, 4, 2, 64, 0.1f, ATTN_MASK_CAUSAL, 0, 0.f, nullptr,
                           (int32_t*)P, ATTN_F32, nullptr),
           log ? ATTN_ERR_HIP : ATTN_OK, log ? 1 : 2);
    EXPECT(attn_fwd_varlen(P, P, P, P, nullptr, D, 0, 100, 4, 2, 128, 0.1f, 0, 0, 0.f, nullptr, (int32_t*)P, 1,
                           nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_fp8_prepare(P, P, P, 1, 2, 2, 16, 128, nullptr, P, P, P, nullptr), ATTN_OK, 1);
    EXPECT(attn_fp8_prepare(P, P, P, 1, 2, 2, 16, 64, nullptr, P, P, P, nullptr), ATTN_ERR_UNSUPPORTED, 0);
    EXPECT(attn_fp8_prepare_rope(P, P, P, 1, 2, 2, 16, 128, nullptr, nullptr, (const float*)P, P, P, P, nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_block_mask_build(2, 100, 90, ATTN_MASK_CAUSAL, 0, nullptr, 32, 64, P, nullptr), ATTN_OK, 1);
    EXPECT(attn_block_mask_build(2, 100, 90, ATTN_MASK_CAUSAL, 0, nullptr, 0, 64, P, nullptr), ATTN_ERR_INVALID_ARG,
           0);
    EXPECT(attn_fwd_tile_kinds(2, 100, 90, ATTN_MASK_CAUSAL, 0, nullptr, (int8_t*)P, nullptr), ATTN_OK, 1);
    EXPECT(attn_fwd_tile_kinds(2, 100, 90, ATTN_MASK_DOC, 0, nullptr, (int8_t*)P, nullptr), ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_decode_paged(P, P, P, D, D, P, nullptr, 4, 8, 2, 128, 16, 10, 0.1f, 4, (float*)P, ATTN_BF16,
                             nullptr),
           ATTN_OK, 1);
    EXPECT(attn_decode_paged(P, P, P, D, D, P, nullptr, 4, 8, 2, 128, 16, 10, 0.1f, 4, nullptr, ATTN_BF16, nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_decode_paged(P, P, P, D, D, P, nullptr, 4, 8, 2, 128, 8, 10, 0.1f, 1, nullptr, ATTN_BF16, nullptr),
           ATTN_ERR_UNSUPPORTED, 0);
    EXPECT(attn_decode_paged_noalloc(P, P, P, D, D, P, nullptr, 64, 32, 8, 128, 16, 512, 0.1f, 8, ATTN_BF16,
                                     nullptr),
           ATTN_OK, 1);
    // 256 x 64 heads x 16 splits x 129 floats: beyond the fixed scratch
    EXPECT(attn_decode_paged_noalloc(P, P, P, D, D, P, nullptr, 256, 64, 8, 128, 16, 512, 0.1f, 16, ATTN_BF16,
                                     nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_decode_paged_noalloc(nullptr, P, P, D, D, P, nullptr, 4, 8, 2, 128, 16, 10, 0.1f, 4, ATTN_BF16,
                                     nullptr),
           ATTN_ERR_INVALID_ARG, 0);
    EXPECT(attn_bwd(P, P, P, P, P, (const float*)P, P, P, P, (float*)P, 1, 2, 2, 16, 128, 0.1f, ATTN_MASK_CAUSAL,
                    ATTN_BF16, nullptr),
           ATTN_OK, 1);
    EXPECT(attn_bwd(P, P, P, P, P, (const float*)P, P, P, P, (float*)P, 1, 2, 2, 16, 128, 0.1f, ATTN_MASK_WINDOW,
                    ATTN_BF16, nullptr),
           ATTN_ERR_UNSUPPORTED, 0);
    // size helpers never overflow or accept bad sizes
    if (attn_fp8_buffer_bytes(0, 1, 1, 128) != 0 || attn_block_mask_bytes(1, 1, 1, 0, 1) != 0 ||
        attn_fwd_tile_kinds_bytes(1, 0, 1) != 0 || attn_decode_workspace_floats(1, 1, 128, 0) != 0) {
        std::fprintf(stderr, "size helper accepted a bad size\n");
        ++failures;
    }
    std::printf("abi host check: %d failures, %d launches\n", failures, attn::launches);
    return failures ? 1 : 0;
}
