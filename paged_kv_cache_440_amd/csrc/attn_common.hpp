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

// Eight consecutive outputs from idx (a multiple of 8; out is 16-byte
// aligned) with 16-byte stores, rounded as store_out rounds.
__device__ __forceinline__ void store_out8(void* out, int out_dtype, size_t idx, const float (&v)[8]) {
    if (out_dtype == PKV_F32) {
        f32x4* p = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + idx);
        p[0] = f32x4{v[0], v[1], v[2], v[3]};
        p[1] = f32x4{v[4], v[5], v[6], v[7]};
        return;
    }
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t lo, hi;
        if (out_dtype == PKV_F16) {
            lo = __builtin_bit_cast(uint16_t, (_Float16)v[2 * k]);
            hi = __builtin_bit_cast(uint16_t, (_Float16)v[2 * k + 1]);
        } else {
            lo = __builtin_bit_cast(uint16_t, (__bf16)v[2 * k]);
            hi = __builtin_bit_cast(uint16_t, (__bf16)v[2 * k + 1]);
        }
        w[k] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + idx) = w;
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

// Zero the output rows of columns [c0, c1) of segment (seq, g) (padding
// sequences, and queries before the start of their sequence).
template <int D>
__device__ __forceinline__ void write_zero_cols(const AttnParams& a, int seq, int g, int c0,
                                                int c1, int lane) {
    for (int idx = lane; idx < (c1 - c0) * D; idx += 64)
        store_out(a.out, a.out_dtype, out_row(a, seq, g, c0 + idx / D) * D + idx % D, 0.f);
}

// ... of every column of segment (seq, g).
template <int D>
__device__ __forceinline__ void write_zero_rows(const AttnParams& a, int seq, int g, int lane) {
    write_zero_cols<D>(a, seq, g, 0, a.num_queries * a.group, lane);
}

// Token positions the columns of 16-column tile `tile` of a segment of
// length L may see: 0 .. reach - 1, where reach - 1 is the causal limit of
// the tile's last column (new token j sits at L - nq + j and sees up to
// itself). L for a segment of at most 16 columns; 0 or less when every
// column of the tile is a query before the start of its sequence.
__device__ __forceinline__ int tile_reach(const AttnParams& a, int L, int tile) {
    const int cols = a.num_queries * a.group;
    const int last = 16 * tile + 15 < cols ? 16 * tile + 15 : cols - 1;
    return L - a.num_queries + last / a.group + 1;
}

// The same for the group of tiles_per_item tiles one work item walks together:
// the reach of its last tile.
__device__ __forceinline__ int group_reach(const AttnParams& a, int L, int group) {
    const int last = a.tiles_per_item * (group + 1) - 1;
    return tile_reach(a, L, last < a.col_tiles ? last : a.col_tiles - 1);
}

}  // namespace
}  // namespace pkv
