// Allocation-free decode attention: the split-K records live in a static
// device array of the library, one copy per device, instead of a workspace
// the caller allocates. For callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops). Declared in
// include/pkv.h (pkv_paged_attention_decode_noalloc).
//
// Nothing in the records needs to start at zero: the walk writes every
// record and every merge-information word the merge then reads (the
// balanced schedule writes its per-wave word even for waves with no work),
// so the array is never cleared and keeps the last call's contents.

#include <atomic>
#include <mutex>

#include "pkv_internal.hpp"

namespace {

// PKV_NOALLOC_SCRATCH_BYTES (40 MiB): the balanced schedule's records for
// up to 8 query heads per kv head at head_dim 128 (2 * 4096 waves * 8 rows *
// 130 floats = 34.1 MB), or fixed partitions up to the same size.
constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// This device's address of `scratch`: looked up once per device, with that
// device current, and kept. In host code `scratch` names a host-side
// stand-in, so only this address may reach a kernel.
int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_HIP;
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (ptr == nullptr) {
            if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess ||
                ptr == nullptr) {
                (void)hipGetLastError();
                return PKV_ERR_HIP;
            }
            g_scratch_ptr[dev].store(ptr, std::memory_order_release);
        }
    }
    *out = ptr;
    return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_paged_attention_decode_noalloc(void* out, pkv_dtype out_dtype, const void* q,
                                       const void* k_pool, const void* v_pool,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* seq_lens, int max_seq_len, int num_seqs,
                                       int num_heads, int num_kv_heads, int head_dim,
                                       int block_size, int num_blocks, float scale,
                                       int partition_size, pkv_dtype dtype, int kv_policy,
                                       void* stream) {
    const size_t need = pkv_paged_attention_workspace_size(num_seqs, num_heads, num_kv_heads,
                                                           head_dim, max_seq_len, partition_size);
    if (need > kScratchBytes) return PKV_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0 && num_seqs > 0) {
        const int st = scratch_address(&ws);
        if (st != PKV_OK) return st;
    }
    return pkv_paged_attention_decode(out, out_dtype, q, k_pool, v_pool, block_tables,
                                      max_blocks_per_seq, seq_lens, max_seq_len, num_seqs,
                                      num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                      scale, partition_size, ws, need, dtype, kv_policy, stream);
}

}  // extern "C"
