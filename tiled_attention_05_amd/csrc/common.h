// Shared device helpers for the gfx950 attention kernels: vector types, LDS
// address-space casts, the direct global->LDS load, the raw workgroup barrier,
// cross-half wave exchange and MFMA wrappers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define ATTN_LDS __attribute__((address_space(3)))

// Read-only global memory reached through the scalar cache: a wave-uniform
// load from it is an s_load (counted by lgkmcnt, not vmcnt).
#define ATTN_CONST __attribute__((address_space(4)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Asynchronous 16-byte copy global -> LDS. The LDS destination of lane i is
// lds_wave_base + 16 * i (the base must be wave-uniform): a wave moves 1 KiB.
__device__ __forceinline__ void load_lds16(const void* src, ATTN_LDS void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, lds_wave_base, 16, 0, 0);
}

// 4-byte variant: a wave moves 256 bytes (used for per-tile document ids).
__device__ __forceinline__ void load_lds4(const void* src, ATTN_LDS void* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(src, lds_wave_base, 4, 0, 0);
}

// Same copies issued from inline assembly: the compiler then does not know
// that they write LDS, so it does not insert a wait for them before unrelated
// LDS reads; the caller waits explicitly (wait_all_and_barrier) before reading
// the destination. lds_wave_base is a wave-uniform LDS byte address (M0).
__device__ __forceinline__ void dma16(const void* src, unsigned lds_wave_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(lds_wave_base), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* src, unsigned lds_wave_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                 :: "s"(lds_wave_base), "v"(src) : "memory", "m0");
}
// Scalar-base forms: address = sbase (wave-uniform, SGPR pair) + voff (per lane).
__device__ __forceinline__ void dma16s(const void* sbase, unsigned voff, unsigned lds_wave_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds_wave_base), "v"(voff), "s"(sbase) : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const void* sbase, unsigned voff, unsigned lds_wave_base) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(lds_wave_base), "v"(voff), "s"(sbase) : "memory", "m0");
}
__device__ __forceinline__ unsigned lds_addr(const ATTN_LDS void* p) {
    return (unsigned)(uintptr_t)p;
}

// Wait until this wave's global loads (including global->LDS copies) have all
// landed and its LDS reads have returned, then barrier the workgroup. The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void wait_all_and_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Value held by lane l ^ 32 combined with this lane's: op(x[l], x[l ^ 32]).
__device__ __forceinline__ float xhalf_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    float m;
    asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
    return m;
}
__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product issued as inline assembly with the register file of each
// operand fixed: "v" keeps a value in VGPRs (read by vector code), "a" in
// AGPRs (touched only by the matrix core). The compiler does not see these as
// matrix instructions, so the caller keeps every vector access to their
// registers away from them: results are read (and AGPRs read or written by
// vector code) at least mfma_guard() after the instruction, operands written
// by vector code are written well before it, and source registers stay
// allocated (keep) for a few instructions after it.
__device__ __forceinline__ void mfma_bf16_va(f32x16& c, bf16x8 a, bf16x8 b) {   // c += a b, b in AGPRs
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_bf16_va0(f32x16& c, bf16x8 a, bf16x8 b) {  // c = a b, b in AGPRs
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_bf16_a(f32x16& c, bf16x8 a, bf16x8 b) {    // c += a b, c in AGPRs
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// e4m3 x e4m3 -> f32 32x32x64 products in the same form (unscaled encoding).
__device__ __forceinline__ void mfma_fp8_va(f32x16& c, i32x8 a, i32x8 b) {    // c += a b, b in AGPRs
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_fp8_va0(f32x16& c, i32x8 a, i32x8 b) {   // c = a b, b in AGPRs
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_fp8_a(f32x16& c, i32x8 a, i32x8 b) {     // c += a b, c in AGPRs
    asm volatile("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// 32 wait states: more than a 32x32x16 bf16 or 32x32x64 e4m3 product needs
// before its result may be read by vector code or its AGPRs accessed with
// v_accvgpr_read / write. The guard orders only against other volatile asm:
// plain register reads may still be scheduled above it, so every value read
// after a guard is re-pinned (pin / pin_a) right after it, which makes its
// readers depend on a statement that follows the wait states.
__device__ __forceinline__ void mfma_guard() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}
// 4 wait states: more than the two instructions that must separate a vector
// write of a register from a matrix instruction reading it as its A or B
// operand (the reverse direction, a result read by vector code, takes
// mfma_guard()). Values written before it are re-pinned after it, as there.
__device__ __forceinline__ void operand_guard() {
    asm volatile("s_nop 3" ::: "memory");
}
// Pins a value at this point of the instruction stream (an empty volatile
// statement that reads and rewrites it), so work placed around it stays there.
template <typename T>
__device__ __forceinline__ void pin(T& x) {
    asm volatile("" : "+v"(x));
}
template <typename T>
__device__ __forceinline__ void pin_a(T& x) {   // same for a value in AGPRs
    asm volatile("" : "+a"(x));
}
// Keeps a value (and its registers) allocated up to this point.
template <typename T>
__device__ __forceinline__ void keep(const T& x) {
    asm volatile("" :: "v"(x));
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// OCP e4m3 x e4m3 -> f32, 32x32x64 (block scales fixed at 2^0).
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// max(a, b, c) in one instruction (hardware max semantics).
__device__ __forceinline__ float max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// max(a, b) in one instruction (no operand canonicalization).
// max(|a|, |b|, |c|) through the instruction's absolute-value modifiers
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float max2(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// First index j in [0, n) with a[j] >= x (a non-decreasing), n if none.
__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

// First index j in [0, n) with a[j] > x, n if none.
__device__ __forceinline__ int upper_bound_i32(const int32_t* a, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (a[mid] <= x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

}  // namespace attn
