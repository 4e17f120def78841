// Internal interface between the C-ABI layer (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

// Everything one attention launch needs, validated by the host layer.
struct AttnParams {
    void* out;
    int out_dtype;
    float* ws_acc;                 // unnormalised partial sums, D floats per row:
                                   // [B][H][max_parts] rows (fixed partitions) or
                                   // [2 * kMaxBalancedWaves][G] rows (balanced)
    float* ws_ml;                  // per row: running max in log2 units, sum
    int* ws_info;                  // balanced: 2 ints per workgroup (segment ending
                                   // in it that began earlier, first wave holding it)
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    int max_blocks;                // row stride of block_tables
    int num_seqs;
    int num_kv_heads;
    int group;                     // query heads per kv head
    int head_dim;
    int log2_bs;
    int num_blocks;
    float scale;
    int part_tokens;               // 0: one pass per sequence
    int max_parts;                 // partitions per sequence the launch covers
    int max_tokens;                // lengths are clamped to this
    int num_items;                 // waves launched: max_parts * num_seqs * num_kv_heads;
                                   // balanced: the compute-unit count on entry to the
                                   // launcher, the persistent wave count in the kernels
    int balanced;                  // 1: balanced schedule (see attention.hip)
    int kv_stream;                 // 1: non-temporal K/V loads (PKV_KV_STREAM), 0: cached
    int stage;                     // host side: kStageBoth, kStageWalk or kStageMerge
    // sampling groups (pkv_paged_attention_decode_grouped): sequences
    // k*group_size .. (k+1)*group_size - 1 share their first shared_tokens[k]
    // tokens' blocks; shared_tokens is null for every other call
    int group_size;
    const int32_t* shared_tokens;
    int num_queries;               // new tokens per sequence (1: decode); q and out are
                                   // [B][num_queries][H][D]. A segment (seq, kv head) has
                                   // num_queries * group columns (query token, head).
    int col_tiles;                 // 16-column tiles per segment: ceil(columns / 16); more
                                   // than one only for the matrix-core walker, under the
                                   // single pass or fixed partitions
    int tiles_per_item;            // tiles one work item (a wave, or a workgroup for
                                   // chunked prefill) walks together, sharing each K/V chunk
    int dtype;                     // q / K / V element type (16/32-bit path)
    int* err;                      // error word (pkv_set_error_word), or null
    int force_vector;              // PKV_WALKER_VECTOR: grouped heads on the vector units
    // FP8 pools: K/V are E4M3 codes times a per-kv-head scale; q has q_dtype
    const float* k_scales;
    const float* v_scales;
    int q_dtype;
};

// Launches a split attention call enqueues (PKV_STAGE_WALK / PKV_STAGE_MERGE).
constexpr int kStageBoth = 0, kStageWalk = 1, kStageMerge = 2;
__host__ __device__ inline bool stage_walks(int stage) { return stage != kStageMerge; }
__host__ __device__ inline bool stage_merges(int stage) { return stage != kStageWalk; }

// Persistent waves of the balanced schedule: each walker's
// kBalancedWavesPerCU per compute unit (fewer if fewer fit), at most
// kMaxBalancedWaves (which sizes the workspace).
constexpr int kMaxBalancedWaves = 4096;

struct AppendParams {
    const void* k_new;
    const void* v_new;
    void* k_pool;
    void* v_pool;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    int max_blocks;
    int num_seqs;
    int num_kv_heads;
    int row_bytes;                 // head_dim * element bytes
    int log2_bs;
    int num_blocks;
    int num_queries;               // new tokens per sequence: k_new is [B][nq][Hkv][D]
    int* err;                      // error word (pkv_set_error_word), or null
};

// Quantising append into FP8 E4M3 pools.
struct AppendFp8Params {
    const void* k_new;
    const void* v_new;
    int new_dtype;                 // PKV_F32 / PKV_F16 / PKV_BF16
    uint8_t* k_pool;
    uint8_t* v_pool;
    const float* k_scales;         // [num_kv_heads]
    const float* v_scales;
    const int32_t* block_tables;
    const int32_t* seq_lens;
    int max_blocks;
    int num_seqs;
    int num_kv_heads;
    int head_dim;
    int log2_bs;
    int num_blocks;
    int num_queries;               // new tokens per sequence: k_new is [B][nq][Hkv][D]
    int* err;                      // error word (pkv_set_error_word), or null
};

// Block copies from one pool pair into another (the same pair for
// copy-on-write, a device and a host pool for swapping).
struct CopyParams {
    const void* src_k;
    const void* src_v;
    void* dst_k;
    void* dst_v;
    const int32_t* mapping;
    int num_pairs;
    long long block_bytes;         // num_kv_heads * block_size * row bytes
    int src_num_blocks;
    int dst_num_blocks;
    int* err;                      // error word (pkv_set_error_word), or null
};

// The error word registered for the current device (null if none).
int* error_word();

hipError_t launch_paged_attention(const AttnParams& a, hipStream_t stream);
hipError_t launch_append(const AppendParams& a, hipStream_t stream);
hipError_t launch_append_fp8(const AppendFp8Params& a, hipStream_t stream);
hipError_t launch_paged_attention_fp8(const AttnParams& a, hipStream_t stream);
hipError_t launch_paged_attention_multi(const AttnParams& a, hipStream_t stream);
hipError_t launch_paged_attention_grouped(const AttnParams& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyParams& a, hipStream_t stream);

}  // namespace pkv
