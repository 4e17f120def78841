/*
 * pkv_swap.h - moving KV blocks between a device pool and a pool in pinned
 * host memory.
 *
 * When device memory runs short, the blocks of preempted sequences can be
 * moved to CPU memory and brought back later instead of recomputing their
 * KV cache (supersilo.blog vLLM/PagedAttention summary, section "적용 범위와
 * 관련 연구": swapping to CPU memory and recomputation are the two recovery
 * paths, chosen by comparing the cost of fetching the data back with the
 * cost of recomputing it). The host block manager (pkv_block_manager.h) plans
 * which blocks go where; pkv_swap_blocks moves the bytes.
 *
 * Memory.  Unlike pkv.h, the pools and the mapping given here may each be
 * either device memory of the current HIP device (hipMalloc) or pinned host
 * memory (hipHostMalloc, or torch's pin_memory). The kernel reads and writes
 * host memory directly over the host link: one launch moves every pair.
 * Pageable host memory (plain malloc, numpy) is rejected with
 * PKV_ERR_INVALID before anything is enqueued, since the device cannot reach
 * it. The library allocates nothing.
 * Streams.  As in pkv.h: work is enqueued on `stream` and the call returns.
 * Host memory written by a swap is complete once the stream has reached the
 * end of the call (synchronise the stream or an event before reading it on
 * the host); host memory a swap reads must not change until then.
 */
#ifndef PKV_SWAP_H
#define PKV_SWAP_H

#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy whole blocks, K and V, from one pool into another of the same block
 * geometry.
 *
 * src_k, src_v   [src_num_blocks][num_kv_heads][block_size][head_dim] (read)
 * dst_k, dst_v   [dst_num_blocks][num_kv_heads][block_size][head_dim] (written)
 * block_mapping  int32 [num_pairs][2] = (source block, destination block)
 *
 * For each pair, block dst of dst_k (and dst_v) becomes a bit-exact image of
 * block src of src_k (src_v): all heads, all slots. Swapping a sequence out
 * is a call with the device pool as source and the host pool as
 * destination; swapping it in is the reverse. Destinations must be distinct
 * (pairs run concurrently), and the source and destination pools must not
 * overlap. Pairs with an id outside [0, src_num_blocks) or
 * [0, dst_num_blocks) are skipped. Any pool element type of pkv.h (FP8 pools
 * included: their scales are per kv head, so they do not move with a block).
 *
 * Returns PKV_ERR_INVALID for bad sizes, a pointer the device cannot reach
 * (pageable host memory, another device's memory), a buffer shorter than its
 * stated size, or pools not 16-byte aligned; PKV_ERR_UNSUPPORTED for a
 * head_dim or block_size pkv.h does not support; PKV_ERR_HIP if the runtime
 * rejects a query or the launch. num_pairs == 0 enqueues nothing.
 */
PKV_API int pkv_swap_blocks(const void* src_k, const void* src_v, int src_num_blocks,
                            void* dst_k, void* dst_v, int dst_num_blocks,
                            const int32_t* block_mapping, int num_pairs, int num_kv_heads,
                            int head_dim, int block_size, pkv_dtype dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_SWAP_H */
