// Pieces shared by the paged-attention walkers and schedules.
#pragma once

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {
namespace {

#ifndef PKV_ATTN_WAVES
#define PKV_ATTN_WAVES 4
#endif
constexpr int kWaves = PKV_ATTN_WAVES;          // independent waves per workgroup
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void store_out(void* out, int out_dtype, size_t idx, float v) {
    if (out_dtype == PKV_F32) {
        reinterpret_cast<float*>(out)[idx] = v;
    } else if (out_dtype == PKV_F16) {
        reinterpret_cast<_Float16*>(out)[idx] = (_Float16)v;
    } else {
        reinterpret_cast<__bf16*>(out)[idx] = (__bf16)v;
    }
}

__device__ __forceinline__ int clamp_len(const AttnParams& a, int L) {
    L = L < 0 ? 0 : L;
    return L < a.max_tokens ? L : a.max_tokens;
}

// Zero output rows of the G query heads of kv head g (padding sequences).
template <int D, int G>
__device__ __forceinline__ void write_zero_rows(const AttnParams& a, int seq, int g, int lane) {
    const size_t row0 = (size_t)seq * a.num_kv_heads * G + (size_t)g * G;
    for (int idx = lane; idx < G * D; idx += 64) store_out(a.out, a.out_dtype, row0 * D + idx, 0.f);
}

}  // namespace
}  // namespace pkv
