// C-ABI entry points: argument validation, then one launch (or two) on the
// caller's stream. Declarations and contracts are in include/pkv.h and
// include/pkv_swap.h.

#include <math.h>

#include <atomic>

#include "pkv_internal.hpp"
#include "pkv_swap.h"

namespace {

bool valid_dtype(int d) { return d == PKV_F32 || d == PKV_F16 || d == PKV_BF16; }
bool valid_pool_dtype(int d) { return valid_dtype(d) || d == PKV_FP8_E4M3; }
int dtype_bytes(int d) { return d == PKV_F32 ? 4 : d == PKV_FP8_E4M3 ? 1 : 2; }
bool supported_head_dim(int d) { return d == 64 || d == 128; }

// log2 of a supported block size (a power of two in [8, 256]), else -1
int block_log2(int bs) {
    for (int s = 3; s <= 8; ++s)
        if (bs == (1 << s)) return s;
    return -1;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Partition count the launch must cover, or -1 if the sizes overflow.
long long parts_for(int max_seq_len, int partition_size) {
    if (partition_size <= 0 || max_seq_len <= partition_size) return 1;
    return ((long long)max_seq_len + partition_size - 1) / partition_size;
}

size_t workspace_bytes_for(long long rows, int head_dim, long long parts) {
    if (parts <= 1) return 0;
    return (size_t)(rows * parts) * (size_t)(head_dim + 2) * sizeof(float);
}

// Room for two records of `group` rows per persistent wave (record 2w + 1 of
// a wave where a cut segment begins, 2w of the first wave of a workgroup),
// then two ints of merge information per wave (one pair per workgroup is
// used).
size_t balanced_record_rows(int group) { return (size_t)2 * pkv::kMaxBalancedWaves * group; }
size_t balanced_workspace_bytes(int group, int head_dim) {
    return balanced_record_rows(group) * (size_t)(head_dim + 2) * sizeof(float) +
           (size_t)2 * pkv::kMaxBalancedWaves * sizeof(int);
}

// Compute units of the current device, queried once per device.
int compute_units() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < 64) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return -1;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// The error word registered per device (pkv_set_error_word).
std::atomic<int*> g_error_word[64];

// The address a kernel on `device` uses for `bytes` bytes at p: p itself for
// memory of that device, the mapped address for pinned host memory. Pageable
// host memory, other devices' memory and ranges that run past the end of
// their allocation are refused (the kernel would fault on them).
int device_view(const void* p, size_t bytes, int device, const void** out) {
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();          // an unknown pointer is the caller's error
        return PKV_ERR_INVALID;
    }
    const void* dp;
    if (attr.type == hipMemoryTypeDevice) {
        if (attr.device != device) return PKV_ERR_INVALID;
        dp = p;
    } else if (attr.type == hipMemoryTypeHost) {
        if (!attr.devicePointer) return PKV_ERR_INVALID;
        dp = attr.devicePointer;
    } else {
        return PKV_ERR_INVALID;
    }
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(dp)) != hipSuccess) {
        (void)hipGetLastError();
        return PKV_ERR_INVALID;
    }
    const uintptr_t lo = reinterpret_cast<uintptr_t>(base), at = reinterpret_cast<uintptr_t>(dp);
    if (at < lo || at - lo > size || bytes > size - (at - lo)) return PKV_ERR_INVALID;
    *out = dp;
    return PKV_OK;
}

// Validation and parameter setup shared by the attention entry points
// (everything but the element types). Returns a pkv_status; on PKV_OK with
// num_seqs > 0, `a` is ready but for dtype / q_dtype / scales.
int prepare_attention(pkv::AttnParams& a, void* out, int out_dtype, const void* q,
                      const void* k_pool, const void* v_pool, const int32_t* block_tables,
                      int max_blocks_per_seq, const int32_t* seq_lens, int max_seq_len,
                      int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, float scale, int partition_size,
                      void* workspace, size_t workspace_bytes, int kv_policy,
                      int num_queries = 1) {
    const int stage_bits = kv_policy & (PKV_STAGE_WALK | PKV_STAGE_MERGE);
    kv_policy &= ~(PKV_STAGE_WALK | PKV_STAGE_MERGE);
    if (stage_bits == (PKV_STAGE_WALK | PKV_STAGE_MERGE)) return PKV_ERR_INVALID;
    if (kv_policy != PKV_KV_STREAM && kv_policy != PKV_KV_REUSE) return PKV_ERR_INVALID;
    a.stage = stage_bits == PKV_STAGE_WALK ? pkv::kStageWalk
            : stage_bits == PKV_STAGE_MERGE ? pkv::kStageMerge : pkv::kStageBoth;
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
        block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_seq_len < 0 ||
        partition_size < PKV_PARTITION_BALANCED || !valid_dtype(out_dtype) || !isfinite(scale))
        return PKV_ERR_INVALID;
    if (num_heads % num_kv_heads != 0) return PKV_ERR_INVALID;
    if (partition_size > 0 && partition_size % 64 != 0) return PKV_ERR_INVALID;
    const int group = num_heads / num_kv_heads;
    if (!supported_head_dim(head_dim) || block_log2(block_size) < 0 ||
        !(group == 1 || group == 2 || group == 4 || group == 8))
        return PKV_ERR_UNSUPPORTED;
    if ((long long)max_seq_len > (long long)max_blocks_per_seq * block_size)
        return PKV_ERR_INVALID;
    a.group = group;
    a.num_queries = num_queries;
    if (num_seqs == 0) return PKV_OK;
    if (!out || !q || !k_pool || !v_pool || !block_tables || !seq_lens) return PKV_ERR_INVALID;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
        return PKV_ERR_INVALID;
    if ((long long)num_seqs * max_blocks_per_seq > INT32_MAX) return PKV_ERR_INVALID;
    if ((long long)num_seqs * num_queries * num_heads * head_dim > INT32_MAX) return PKV_ERR_INVALID;
    const int cols = group * num_queries;       // output rows per (sequence, kv head)
    // more than 16 columns (chunked prefill) run as 16-column tiles; there the
    // balanced schedule is a single pass per tile: the tiles fill the GPU, and
    // a partial record per query token would cost more than it evens out
    const int tiles = (cols + 15) / 16;
    const bool balanced = partition_size == PKV_PARTITION_BALANCED && tiles == 1;
    const long long parts = partition_size == PKV_PARTITION_BALANCED
                                ? 1 : parts_for(max_seq_len, partition_size);
    long long items = parts * num_seqs * num_kv_heads * tiles;
    if (items > INT32_MAX - 64) return PKV_ERR_INVALID;
    const size_t need =
        balanced ? balanced_workspace_bytes(cols, head_dim)
                 : workspace_bytes_for((long long)num_seqs * num_kv_heads * cols, head_dim, parts);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return PKV_ERR_WORKSPACE;
    if (balanced) {
        // the launch turns this into the persistent wave count
        const int cus = compute_units();
        if (cus <= 0) return PKV_ERR_HIP;
        items = cus;
    }
    const size_t rows = balanced ? balanced_record_rows(cols)
                                 : need / ((size_t)(head_dim + 2) * sizeof(float));

    a.out = out;
    a.out_dtype = out_dtype;
    a.ws_acc = reinterpret_cast<float*>(workspace);
    a.ws_ml = need ? a.ws_acc + rows * head_dim : nullptr;
    a.ws_info = balanced ? reinterpret_cast<int*>(a.ws_ml + 2 * rows) : nullptr;
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.log2_bs = block_log2(block_size);
    a.num_blocks = num_blocks;
    a.scale = scale;
    a.part_tokens = (!balanced && parts > 1) ? partition_size : 0;
    a.col_tiles = tiles;
    a.tiles_per_item = 1;
    a.max_parts = (int)parts;
    a.max_tokens = max_seq_len;
    a.num_items = (int)items;
    a.balanced = balanced ? 1 : 0;
    a.kv_stream = kv_policy == PKV_KV_STREAM ? 1 : 0;
    a.err = pkv::error_word();
    return PKV_OK;
}

}  // namespace

int* pkv::error_word() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    return g_error_word[dev].load(std::memory_order_acquire);
}

extern "C" {

const char* pkv_status_string(int status) {
    switch (status) {
        case PKV_OK: return "ok";
        case PKV_ERR_INVALID: return "invalid argument";
        case PKV_ERR_UNSUPPORTED: return "unsupported head_dim, block_size, head grouping or dtype";
        case PKV_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case PKV_ERR_HIP: return "HIP runtime error at launch";
        case PKV_ERR_NO_BLOCKS: return "no free block in the pool";
        case PKV_ERR_SCRATCH:
            return "the call needs more split-K scratch than the library's static buffer holds";
        default: return "unknown status";
    }
}

int pkv_set_error_word(int32_t* error_word) {
    if ((reinterpret_cast<uintptr_t>(error_word) & 3u) != 0) return PKV_ERR_INVALID;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return PKV_ERR_HIP;
    g_error_word[dev].store(reinterpret_cast<int*>(error_word), std::memory_order_release);
    return PKV_OK;
}

int pkv_kv_cache_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                        const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* seq_lens, int num_seqs, int num_kv_heads, int head_dim,
                        int block_size, int num_blocks, pkv_dtype dtype, void* stream) {
    if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0 || max_blocks_per_seq <= 0 || !valid_pool_dtype(dtype))
        return PKV_ERR_INVALID;
    if (dtype == PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;   // see pkv_kv_cache_append_fp8
    if (!supported_head_dim(head_dim) || block_log2(block_size) < 0) return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PKV_OK;
    if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !seq_lens)
        return PKV_ERR_INVALID;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
        return PKV_ERR_INVALID;
    if ((long long)num_seqs * max_blocks_per_seq > INT32_MAX) return PKV_ERR_INVALID;
    pkv::AppendParams a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.row_bytes = head_dim * dtype_bytes(dtype);
    a.log2_bs = block_log2(block_size);
    a.num_blocks = num_blocks;
    a.num_queries = 1;
    a.err = pkv::error_word();
    return pkv::launch_append(a, (hipStream_t)stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_kv_cache_append_multi(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* seq_lens, int num_seqs, int num_queries,
                              int num_kv_heads, int head_dim, int block_size, int num_blocks,
                              pkv_dtype dtype, void* stream) {
    if (num_queries <= 0 || num_seqs < 0) return PKV_ERR_INVALID;
    if ((long long)num_seqs * num_queries > INT32_MAX) return PKV_ERR_INVALID;
    // the scalar checks of the single-token append (no sequences: nothing enqueued)
    const int st = pkv_kv_cache_append(k_new, v_new, k_pool, v_pool, block_tables,
                                       max_blocks_per_seq, seq_lens, 0, num_kv_heads, head_dim,
                                       block_size, num_blocks, dtype, nullptr);
    if (st != PKV_OK || num_seqs == 0) return st;
    if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !seq_lens)
        return PKV_ERR_INVALID;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
        return PKV_ERR_INVALID;
    if ((long long)num_seqs * max_blocks_per_seq > INT32_MAX) return PKV_ERR_INVALID;
    pkv::AppendParams a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.row_bytes = head_dim * dtype_bytes(dtype);
    a.log2_bs = block_log2(block_size);
    a.num_blocks = num_blocks;
    a.num_queries = num_queries;
    a.err = pkv::error_word();
    return pkv::launch_append(a, (hipStream_t)stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_kv_cache_append_fp8(const void* k_new, const void* v_new, pkv_dtype new_dtype,
                            void* k_pool, void* v_pool, const float* k_scales,
                            const float* v_scales, const int32_t* block_tables,
                            int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs,
                            int num_kv_heads, int head_dim, int block_size, int num_blocks,
                            void* stream) {
    return pkv_kv_cache_append_multi_fp8(k_new, v_new, new_dtype, k_pool, v_pool, k_scales,
                                         v_scales, block_tables, max_blocks_per_seq, seq_lens,
                                         num_seqs, 1, num_kv_heads, head_dim, block_size,
                                         num_blocks, stream);
}

int pkv_kv_cache_append_multi_fp8(const void* k_new, const void* v_new, pkv_dtype new_dtype,
                                  void* k_pool, void* v_pool, const float* k_scales,
                                  const float* v_scales, const int32_t* block_tables,
                                  int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs,
                                  int num_queries, int num_kv_heads, int head_dim,
                                  int block_size, int num_blocks, void* stream) {
    if (num_queries <= 0 || (long long)num_seqs * num_queries > INT32_MAX) return PKV_ERR_INVALID;
    if (num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0 || max_blocks_per_seq <= 0 || !valid_dtype(new_dtype))
        return PKV_ERR_INVALID;
    if (head_dim != 128 || block_log2(block_size) < 0) return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PKV_OK;
    if (!k_new || !v_new || !k_pool || !v_pool || !k_scales || !v_scales || !block_tables ||
        !seq_lens)
        return PKV_ERR_INVALID;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
        return PKV_ERR_INVALID;
    if ((long long)num_seqs * max_blocks_per_seq > INT32_MAX) return PKV_ERR_INVALID;
    pkv::AppendFp8Params a{};
    a.k_new = k_new;
    a.v_new = v_new;
    a.new_dtype = new_dtype;
    a.k_pool = reinterpret_cast<uint8_t*>(k_pool);
    a.v_pool = reinterpret_cast<uint8_t*>(v_pool);
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.max_blocks = max_blocks_per_seq;
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.head_dim = head_dim;
    a.log2_bs = block_log2(block_size);
    a.num_blocks = num_blocks;
    a.num_queries = num_queries;
    a.err = pkv::error_word();
    return pkv::launch_append_fp8(a, (hipStream_t)stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_mapping, int num_pairs,
                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                    pkv_dtype dtype, void* stream) {
    if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        num_blocks <= 0 || !valid_pool_dtype(dtype))
        return PKV_ERR_INVALID;
    if (!supported_head_dim(head_dim) || block_log2(block_size) < 0) return PKV_ERR_UNSUPPORTED;
    if (num_pairs == 0) return PKV_OK;
    if (!k_pool || !v_pool || !block_mapping) return PKV_ERR_INVALID;
    if (!aligned16(k_pool) || !aligned16(v_pool)) return PKV_ERR_INVALID;
    const long long block_bytes = (long long)num_kv_heads * block_size * head_dim * dtype_bytes(dtype);
    const long long chunks = (block_bytes / 16 + 1023) / 1024;
    if (chunks * num_pairs * 2 > INT32_MAX) return PKV_ERR_INVALID;
    pkv::CopyParams a{};
    a.src_k = a.dst_k = k_pool;
    a.src_v = a.dst_v = v_pool;
    a.mapping = block_mapping;
    a.num_pairs = num_pairs;
    a.block_bytes = block_bytes;
    a.src_num_blocks = a.dst_num_blocks = num_blocks;
    a.err = pkv::error_word();
    return pkv::launch_copy_blocks(a, (hipStream_t)stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_swap_blocks(const void* src_k, const void* src_v, int src_num_blocks, void* dst_k,
                    void* dst_v, int dst_num_blocks, const int32_t* block_mapping, int num_pairs,
                    int num_kv_heads, int head_dim, int block_size, pkv_dtype dtype,
                    void* stream) {
    if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        src_num_blocks <= 0 || dst_num_blocks <= 0 || !valid_pool_dtype(dtype))
        return PKV_ERR_INVALID;
    if (!supported_head_dim(head_dim) || block_log2(block_size) < 0) return PKV_ERR_UNSUPPORTED;
    if (num_pairs == 0) return PKV_OK;
    if (!src_k || !src_v || !dst_k || !dst_v || !block_mapping) return PKV_ERR_INVALID;
    if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v))
        return PKV_ERR_INVALID;
    const long long block_bytes = (long long)num_kv_heads * block_size * head_dim * dtype_bytes(dtype);
    const long long chunks = (block_bytes / 16 + 1023) / 1024;
    if (chunks * num_pairs * 2 > INT32_MAX) return PKV_ERR_INVALID;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return PKV_ERR_HIP;
    pkv::CopyParams a{};
    const void* p[5];
    const void* want[5] = {src_k, src_v, dst_k, dst_v, block_mapping};
    const size_t bytes[5] = {(size_t)(src_num_blocks * block_bytes),
                             (size_t)(src_num_blocks * block_bytes),
                             (size_t)(dst_num_blocks * block_bytes),
                             (size_t)(dst_num_blocks * block_bytes),
                             (size_t)num_pairs * 2 * sizeof(int32_t)};
    for (int i = 0; i < 5; ++i) {
        const int st = device_view(want[i], bytes[i], device, &p[i]);
        if (st != PKV_OK) return st;
    }
    a.src_k = p[0];
    a.src_v = p[1];
    a.dst_k = const_cast<void*>(p[2]);
    a.dst_v = const_cast<void*>(p[3]);
    a.mapping = static_cast<const int32_t*>(p[4]);
    a.num_pairs = num_pairs;
    a.block_bytes = block_bytes;
    a.src_num_blocks = src_num_blocks;
    a.dst_num_blocks = dst_num_blocks;
    a.err = pkv::error_word();
    return pkv::launch_copy_blocks(a, (hipStream_t)stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

size_t pkv_paged_attention_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                          int head_dim, int max_seq_len, int partition_size) {
    if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
        head_dim <= 0 || max_seq_len < 0 || partition_size < PKV_PARTITION_BALANCED)
        return 0;
    if (partition_size == PKV_PARTITION_BALANCED) {
        // more than 16 columns per kv head: a single pass per 16-column tile
        const int cols = num_heads / num_kv_heads;
        return num_seqs > 0 && cols <= 16 ? balanced_workspace_bytes(cols, head_dim) : 0;
    }
    return workspace_bytes_for((long long)num_seqs * num_heads, head_dim,
                               parts_for(max_seq_len, partition_size));
}

int pkv_paged_attention_decode(void* out, pkv_dtype out_dtype, const void* q,
                               const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* seq_lens, int max_seq_len, int num_seqs,
                               int num_heads, int num_kv_heads, int head_dim, int block_size,
                               int num_blocks, float scale, int partition_size, void* workspace,
                               size_t workspace_bytes, pkv_dtype dtype, int kv_policy,
                               void* stream) {
    if (!valid_pool_dtype(dtype)) return PKV_ERR_INVALID;
    if (dtype == PKV_FP8_E4M3) return PKV_ERR_UNSUPPORTED;   // see pkv_paged_attention_decode_fp8
    if (kv_policy & ~(PKV_KV_REUSE | PKV_STAGE_WALK | PKV_STAGE_MERGE | PKV_WALKER_VECTOR))
        return PKV_ERR_INVALID;
    const bool force_vector = (kv_policy & PKV_WALKER_VECTOR) != 0;
    kv_policy &= ~PKV_WALKER_VECTOR;
    if (force_vector && (kv_policy & PKV_KV_REUSE)) return PKV_ERR_UNSUPPORTED;
    pkv::AttnParams a{};
    const int st = prepare_attention(a, out, out_dtype, q, k_pool, v_pool, block_tables,
                                     max_blocks_per_seq, seq_lens, max_seq_len, num_seqs, num_heads,
                                     num_kv_heads, head_dim, block_size, num_blocks, scale,
                                     partition_size, workspace, workspace_bytes, kv_policy);
    if (st != PKV_OK || num_seqs == 0) return st;
    a.dtype = dtype;
    a.q_dtype = dtype;
    a.force_vector = force_vector ? 1 : 0;
    return pkv::launch_paged_attention(a, (hipStream_t)stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_paged_attention_multi(void* out, pkv_dtype out_dtype, const void* q,
                              const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* seq_lens, int max_seq_len, int num_seqs,
                              int num_queries, int num_heads, int num_kv_heads, int head_dim,
                              int block_size, int num_blocks, float scale, int partition_size,
                              void* workspace, size_t workspace_bytes, pkv_dtype dtype,
                              int kv_policy, void* stream) {
    if (!valid_pool_dtype(dtype) || num_queries <= 0) return PKV_ERR_INVALID;
    pkv::AttnParams a{};
    const int st = prepare_attention(a, out, out_dtype, q, k_pool, v_pool, block_tables,
                                     max_blocks_per_seq, seq_lens, max_seq_len, num_seqs, num_heads,
                                     num_kv_heads, head_dim, block_size, num_blocks, scale,
                                     partition_size, workspace, workspace_bytes, kv_policy,
                                     num_queries);
    if (st != PKV_OK) return st;
    if ((dtype != PKV_F16 && dtype != PKV_BF16) || head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PKV_OK;
    a.dtype = dtype;
    a.q_dtype = dtype;
    return pkv::launch_paged_attention_multi(a, (hipStream_t)stream) == hipSuccess ? PKV_OK
                                                                                   : PKV_ERR_HIP;
}

int pkv_paged_attention_decode_grouped(void* out, pkv_dtype out_dtype, const void* q,
                                       const void* k_pool, const void* v_pool,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* seq_lens, int max_seq_len, int num_seqs,
                                       int num_heads, int num_kv_heads, int head_dim,
                                       int block_size, int num_blocks, float scale,
                                       int partition_size, int group_size,
                                       const int32_t* shared_tokens, void* workspace,
                                       size_t workspace_bytes, pkv_dtype dtype, int kv_policy,
                                       void* stream) {
    if (!valid_pool_dtype(dtype) || group_size <= 0 || partition_size <= 0) return PKV_ERR_INVALID;
    pkv::AttnParams a{};
    const int st = prepare_attention(a, out, out_dtype, q, k_pool, v_pool, block_tables,
                                     max_blocks_per_seq, seq_lens, max_seq_len, num_seqs, num_heads,
                                     num_kv_heads, head_dim, block_size, num_blocks, scale,
                                     partition_size, workspace, workspace_bytes, kv_policy);
    if (st != PKV_OK) return st;
    if ((dtype != PKV_F16 && dtype != PKV_BF16) || head_dim != 128 ||
        (long long)group_size * a.group > 16)
        return PKV_ERR_UNSUPPORTED;
    if (num_seqs % group_size != 0) return PKV_ERR_INVALID;
    if (num_seqs == 0) return PKV_OK;
    if (!shared_tokens) return PKV_ERR_INVALID;
    a.dtype = dtype;
    a.q_dtype = dtype;
    a.group_size = group_size;
    a.shared_tokens = shared_tokens;
    return pkv::launch_paged_attention_grouped(a, (hipStream_t)stream) == hipSuccess ? PKV_OK
                                                                                     : PKV_ERR_HIP;
}

int pkv_paged_attention_multi_fp8(void* out, pkv_dtype out_dtype, const void* q,
                                  pkv_dtype q_dtype, const void* k_pool, const void* v_pool,
                                  const float* k_scales, const float* v_scales,
                                  const int32_t* block_tables, int max_blocks_per_seq,
                                  const int32_t* seq_lens, int max_seq_len, int num_seqs,
                                  int num_queries, int num_heads, int num_kv_heads, int head_dim,
                                  int block_size, int num_blocks, float scale,
                                  int partition_size, void* workspace, size_t workspace_bytes,
                                  int kv_policy, void* stream) {
    if (!valid_dtype(q_dtype) || num_queries <= 0) return PKV_ERR_INVALID;
    pkv::AttnParams a{};
    const int st = prepare_attention(a, out, out_dtype, q, k_pool, v_pool, block_tables,
                                     max_blocks_per_seq, seq_lens, max_seq_len, num_seqs, num_heads,
                                     num_kv_heads, head_dim, block_size, num_blocks, scale,
                                     partition_size, workspace, workspace_bytes, kv_policy,
                                     num_queries);
    if (st != PKV_OK) return st;
    if (q_dtype == PKV_F32 || head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PKV_OK;
    if (!k_scales || !v_scales) return PKV_ERR_INVALID;
    a.dtype = PKV_FP8_E4M3;
    a.q_dtype = q_dtype;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    return pkv::launch_paged_attention_multi(a, (hipStream_t)stream) == hipSuccess ? PKV_OK
                                                                                   : PKV_ERR_HIP;
}

int pkv_paged_attention_decode_grouped_fp8(void* out, pkv_dtype out_dtype, const void* q,
                                           pkv_dtype q_dtype, const void* k_pool,
                                           const void* v_pool, const float* k_scales,
                                           const float* v_scales, const int32_t* block_tables,
                                           int max_blocks_per_seq, const int32_t* seq_lens,
                                           int max_seq_len, int num_seqs, int num_heads,
                                           int num_kv_heads, int head_dim, int block_size,
                                           int num_blocks, float scale, int partition_size,
                                           int group_size, const int32_t* shared_tokens,
                                           void* workspace, size_t workspace_bytes, int kv_policy,
                                           void* stream) {
    if (!valid_dtype(q_dtype) || group_size <= 0 || partition_size <= 0) return PKV_ERR_INVALID;
    pkv::AttnParams a{};
    const int st = prepare_attention(a, out, out_dtype, q, k_pool, v_pool, block_tables,
                                     max_blocks_per_seq, seq_lens, max_seq_len, num_seqs, num_heads,
                                     num_kv_heads, head_dim, block_size, num_blocks, scale,
                                     partition_size, workspace, workspace_bytes, kv_policy);
    if (st != PKV_OK) return st;
    if (q_dtype == PKV_F32 || head_dim != 128 || (long long)group_size * a.group > 16)
        return PKV_ERR_UNSUPPORTED;
    if (num_seqs % group_size != 0) return PKV_ERR_INVALID;
    if (num_seqs == 0) return PKV_OK;
    if (!shared_tokens || !k_scales || !v_scales) return PKV_ERR_INVALID;
    a.dtype = PKV_FP8_E4M3;
    a.q_dtype = q_dtype;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    a.group_size = group_size;
    a.shared_tokens = shared_tokens;
    return pkv::launch_paged_attention_grouped(a, (hipStream_t)stream) == hipSuccess ? PKV_OK
                                                                                     : PKV_ERR_HIP;
}

int pkv_paged_attention_decode_fp8(void* out, pkv_dtype out_dtype, const void* q,
                                   pkv_dtype q_dtype, const void* k_pool, const void* v_pool,
                                   const float* k_scales, const float* v_scales,
                                   const int32_t* block_tables, int max_blocks_per_seq,
                                   const int32_t* seq_lens, int max_seq_len, int num_seqs,
                                   int num_heads, int num_kv_heads, int head_dim, int block_size,
                                   int num_blocks, float scale, int partition_size,
                                   void* workspace, size_t workspace_bytes, int kv_policy,
                                   void* stream) {
    if (!valid_dtype(q_dtype)) return PKV_ERR_INVALID;
    pkv::AttnParams a{};
    const int st = prepare_attention(a, out, out_dtype, q, k_pool, v_pool, block_tables,
                                     max_blocks_per_seq, seq_lens, max_seq_len, num_seqs, num_heads,
                                     num_kv_heads, head_dim, block_size, num_blocks, scale,
                                     partition_size, workspace, workspace_bytes, kv_policy);
    if (st != PKV_OK) return st;
    if (head_dim != 128) return PKV_ERR_UNSUPPORTED;
    if (q_dtype == PKV_F32 && a.group > 1) return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PKV_OK;
    if (!k_scales || !v_scales) return PKV_ERR_INVALID;
    a.dtype = PKV_FP8_E4M3;
    a.q_dtype = q_dtype;
    a.k_scales = k_scales;
    a.v_scales = v_scales;
    return pkv::launch_paged_attention_fp8(a, (hipStream_t)stream) == hipSuccess ? PKV_OK
                                                                                 : PKV_ERR_HIP;
}

}  // extern "C"
