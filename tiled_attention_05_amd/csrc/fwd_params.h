// Kernel argument block of the fused forward (host and device share it).
#pragma once
#include <stdint.h>

namespace attn {

enum : int { kMaskCausal = 1, kMaskWindow = 2, kMaskDoc = 4 };

struct FwdParams {
    const void* q;          // [B][Hq][Nq][d]   (fp8: packed buffer, rows padded to 128)
    const void* k;          // [B][Hkv][Nk][d]  (fp8: packed buffer)
    const void* v;          // [B][Hkv][Nk][d]  (fp8: packed, transposed [d][Np])
    void* o;                // [B][Hq][Nq][d]
    float* lse;             // [B][Hq][Nq] or nullptr
    const int32_t* doc;     // [B][Nk] or nullptr
    const float* slopes;    // [Hq] or nullptr
    int B, Hq, Hkv, Nq, Nk;
    int group;              // Hq / Hkv
    int mask;               // kMask* flags
    int window;
    float scale;            // multiplier of q . k
    float scale_log2;       // scale * log2(e)
    float softcap;          // > 0 when soft-capping
    int n_qt;               // query tiles per (b, h)
    int n_bh;               // B * Hq
    int npad;               // fp8: token count padded to the scale tile
    int xgrp;               // bf16: heads per XCD in one dispatch group, 0 = plain order
    // bf16 packed variable-length batch tiled per sequence (B = 1, Nq = Nk =
    // the packed length, tensors [H][total][d]): items[k] is the first packed
    // row of the k-th heaviest query tile (-1: list padding), cu the sequence
    // offsets [n_seq + 1]; nullptr otherwise
    const int32_t* items;
    const int32_t* cu;
    int n_seq;
    int n_list;             // entries of items
};

}  // namespace attn
