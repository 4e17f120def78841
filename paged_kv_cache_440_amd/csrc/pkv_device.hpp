// Device helpers for the gfx950 kernels: 16-byte vector types, element
// conversions, fp32-accumulating dot products and cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Storage tags: the element type only matters for width and conversion.
struct F32 { static constexpr int bytes = 4; };
struct F16 { static constexpr int bytes = 2; };
struct BF16 { static constexpr int bytes = 2; };

__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }

// -- the two 16-bit values packed in a dword, widened to fp32 (exact) -------
__device__ __forceinline__ float lo_to_f32(F16, uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float hi_to_f32(F16, uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
__device__ __forceinline__ float lo_to_f32(BF16, uint32_t w) { return u2f(w << 16); }
__device__ __forceinline__ float hi_to_f32(BF16, uint32_t w) { return u2f(w & 0xffff0000u); }

// -- dot product of one 16-byte piece of q and of k, fp32 accumulation ------
// fp16 / bf16: v_dot2 (two exact products added into an fp32 accumulator).
// The packed pairs are taken BY VALUE before the bit cast: a bit cast applied
// directly to a vector-subscript lvalue (q[i]) was compiled as element 0.
__device__ __forceinline__ f16x2 as_f16x2(uint32_t x) { return __builtin_bit_cast(f16x2, x); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t x) { return __builtin_bit_cast(bf16x2, x); }

__device__ __forceinline__ float dot16(F16, const u32x4& q, const u32x4& k) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_fdot2(as_f16x2(q[i]), as_f16x2(k[i]), acc, false);
    return acc;
}
__device__ __forceinline__ float dot16(BF16, const u32x4& q, const u32x4& k) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q[i]), as_bf16x2(k[i]), acc, false);
    return acc;
}
__device__ __forceinline__ float dot16(F32, const u32x4& q, const u32x4& k) {
    float acc = u2f(q[0]) * u2f(k[0]);
    acc = __builtin_fmaf(u2f(q[1]), u2f(k[1]), acc);
    acc = __builtin_fmaf(u2f(q[2]), u2f(k[2]), acc);
    acc = __builtin_fmaf(u2f(q[3]), u2f(k[3]), acc);
    return acc;
}

// -- the elements of a 16-byte piece as fp32 --------------------------------
template <typename S> struct Piece;
template <> struct Piece<F32> {
    static constexpr int n = 4;
    __device__ __forceinline__ static void widen(const u32x4& w, float (&f)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = u2f(w[i]);
    }
};
template <typename S> struct Piece16 {
    static constexpr int n = 8;
    __device__ __forceinline__ static void widen(const u32x4& w, float (&f)[8]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = lo_to_f32(S{}, w[i]);
            f[2 * i + 1] = hi_to_f32(S{}, w[i]);
        }
    }
};
template <> struct Piece<F16> : Piece16<F16> {};
template <> struct Piece<BF16> : Piece16<BF16> {};

// -- 16-byte global accesses --------------------------------------------------
__device__ __forceinline__ u32x4 load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
// Loads of K/V data. STREAM: non-temporal loads, for calls that read each
// K/V byte once (the lines take the streaming replacement policy instead of
// displacing data that is reused); otherwise ordinary cached loads, for
// batches whose sequences share blocks (a shared prompt prefix), which then
// come from cache after the first reader.
template <bool STREAM>
__device__ __forceinline__ u32x4 load16_kv(const void* p) {
    if constexpr (STREAM)
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else
        return *reinterpret_cast<const u32x4*>(p);
}
template <bool STREAM>
__device__ __forceinline__ u32x2 load8_kv(const void* p) {
    if constexpr (STREAM)
        return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    else
        return *reinterpret_cast<const u32x2*>(p);
}

// -- cross-lane reductions inside a wave64 ---------------------------------
// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowRor8 = 0x128;      // rotate right by 8 inside a 16-lane row

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return u2f(__builtin_amdgcn_mov_dpp((int)f2u(x), CTRL, 0xF, 0xF, true));
}

// Swap-based exchanges with the lane 16 (resp. 32) positions away (gfx950).
__device__ __forceinline__ void xchg16(float x, float& a, float& b) {
    auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
    a = u2f(r[0]);
    b = u2f(r[1]);
}
__device__ __forceinline__ void xchg32(float x, float& a, float& b) {
    auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    a = u2f(r[0]);
    b = u2f(r[1]);
}

// Sum over aligned groups of N consecutive lanes (N = 8, 16, 32 or 64); every
// lane of the group receives the group's sum. The order of the additions
// depends only on lane positions, so results are reproducible.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group size");
    x += dpp<kDppQuadXor1>(x);
    x += dpp<kDppQuadXor2>(x);
    x += dpp<kDppRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
    if constexpr (N >= 32) { float a, b; xchg16(x, a, b); x = a + b; }
    if constexpr (N >= 64) { float a, b; xchg32(x, a, b); x = a + b; }
    return x;
}

// Combine lanes that are STRIDE apart (the lanes sharing lane % STRIDE),
// for STRIDE = 8, 16 or 32: after the call every lane holds op over all
// 64 / STRIDE lanes of its class.
template <int STRIDE>
__device__ __forceinline__ float strided_sum(float x) {
    if constexpr (STRIDE <= 8) x += dpp<kDppRowRor8>(x);
    if constexpr (STRIDE <= 16) { float a, b; xchg16(x, a, b); x = a + b; }
    if constexpr (STRIDE <= 32) { float a, b; xchg32(x, a, b); x = a + b; }
    return x;
}
template <int STRIDE>
__device__ __forceinline__ float strided_max(float x) {
    if constexpr (STRIDE <= 8) x = __builtin_fmaxf(x, dpp<kDppRowRor8>(x));
    if constexpr (STRIDE <= 16) { float a, b; xchg16(x, a, b); x = __builtin_fmaxf(a, b); }
    if constexpr (STRIDE <= 32) { float a, b; xchg32(x, a, b); x = __builtin_fmaxf(a, b); }
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// OR `bits` into the caller's error word from every lane where `bad` holds
// (a global atomic through the vector memory path; err may be null).
__device__ __forceinline__ void report_if(int* err, bool bad, int bits) {
    if (err != nullptr && bad) atomicOr(err, bits);
}

// The same for a wave: one atomic, from the lowest lane where `bad` holds.
__device__ __forceinline__ void report_wave(int* err, bool bad, int bits) {
    if (err == nullptr) return;
    const unsigned long long any = __ballot(bad);
    if (any != 0 && (int)(threadIdx.x & 63) == __builtin_ctzll(any)) atomicOr(err, bits);
}

}  // namespace pkv
