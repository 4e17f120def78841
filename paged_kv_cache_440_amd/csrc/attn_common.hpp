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

// Output row of column n of segment (seq, g): query token n / G, head g*G + n % G.
__device__ __forceinline__ size_t out_row(const AttnParams& a, int seq, int g, int n) {
    const int G = a.group;
    return ((size_t)seq * a.num_queries + n / G) * ((size_t)a.num_kv_heads * G) +
           (size_t)g * G + n % G;
}

// Zero the output rows of every column of segment (seq, g) (padding sequences).
template <int D>
__device__ __forceinline__ void write_zero_rows(const AttnParams& a, int seq, int g, int lane) {
    const int cols = a.num_queries * a.group;
    for (int idx = lane; idx < cols * D; idx += 64)
        store_out(a.out, a.out_dtype, out_row(a, seq, g, idx / D) * D + idx % D, 0.f);
}

}  // namespace
}  // namespace pkv
