/*
 * pkv_probe.h - measurement kernels that sit beside the paged KV cache
 * library (libpkv.so). They compute nothing of attention: they give the
 * memory-system reference points the attention kernel is judged against.
 *
 *   pkv_probe_read   streams a buffer once with 16-byte non-temporal loads
 *                    (the flavour the attention kernels use for K/V): the practical
 *                    HBM read ceiling for a kernel that only reads.
 *   pkv_probe_copy   copies a buffer with 16-byte loads (non-temporal, as
 *                    above) and plain stores: a
 *                    transfer of known size, used to scale hardware traffic
 *                    counters (bytes fetched / written per dispatch) into
 *                    bytes.
 *   pkv_probe_gather reads exactly the K/V rows a decode launch reads --
 *                    every valid token of every (sequence, kv head), through
 *                    the block tables, tile by tile -- with the same
 *                    non-temporal 16-byte loads and the same equal split of
 *                    32-token units over persistent waves, and computes
 *                    nothing: the read ceiling of the paged access pattern
 *                    itself (scattered bs x row-byte tiles, [summary]
 *                    section "커널 비용과 블록 크기" on block size and access).
 *   pkv_probe_gather_mfma  the same rows, split the same way, read with the
 *                    matrix-core walker's own load shapes (K as 16-row
 *                    operand tiles, 64 bytes of each row per wave load; V as
 *                    4-row pieces): the ceiling of that walker's access pattern.
 *
 * Conventions are those of pkv.h: device pointers owned by the caller, work
 * enqueued on `stream` (a hipStream_t, NULL = null stream), a pkv_status
 * returned, nothing allocated.
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes of `src` (16-byte aligned; bytes a positive multiple of
 * 16) once, in 16-byte pieces, and write one 32-bit value per workgroup into
 * `sink` (the XOR of what that workgroup read, so that no load can be
 * elided). `sink` must hold pkv_probe_read_sink_words(bytes) uint32 values.
 */
PKV_API int pkv_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Number of uint32 values pkv_probe_read writes to `sink` (0 if bytes is invalid). */
PKV_API size_t pkv_probe_read_sink_words(size_t bytes);

/*
 * Copy `bytes` bytes (a positive multiple of 16) from `src` to `dst`
 * (16-byte aligned, not overlapping) with 16-byte loads and stores.
 */
PKV_API int pkv_probe_copy(void* dst, const void* src, size_t bytes, void* stream);

/*
 * Read every K and V row that decode attention over these tables reads:
 * tokens 0 .. seq_lens[i]-1 of every kv head of every sequence, row t of
 * sequence i and head g at slot t % block_size of block
 * block_tables[i][t / block_size] (entries outside [0, num_blocks) are
 * clamped), in pools laid out as in pkv.h with rows of row_bytes bytes
 * (128 or 256: head_dim times the element size). `waves` persistent waves
 * each take an equal share of the 32-token units of all (sequence, kv head)
 * pairs; each round a wave issues loads_per_round (2, 4 or 8) wave-wide
 * 16-byte loads of K and as many of V. One uint32 per wave goes to sink
 * (`waves` words), the XOR of what it read. Lengths must not exceed
 * max_blocks_per_seq * block_size.
 */
PKV_API int pkv_probe_gather(const void* k_pool, const void* v_pool, const int32_t* block_tables,
                             int max_blocks_per_seq, const int32_t* seq_lens, int num_seqs,
                             int num_kv_heads, int row_bytes, int block_size, int num_blocks,
                             int waves, int loads_per_round, uint32_t* sink, void* stream);

/*
 * Read the same rows as pkv_probe_gather (same tables, lengths, pools and
 * split of 32-token units over `waves` persistent waves), a 32-token chunk
 * at a time with the load shapes of the matrix-core walker: for K, two
 * 16-token tiles, each wave load giving lane (n, q) (n = lane % 16,
 * q = lane / 16) the 16 bytes at byte 64 s + 16 q of the tile's row n
 * (row_bytes / 64 loads per tile); for V, eight wave loads giving lane
 * (n, q) bytes (row_bytes / 16) n .. + row_bytes / 16 - 1 of token
 * 16 h + 4 q + j of the chunk (h < 2, j < 4). chunks_per_round (1 or 2)
 * chunks are requested before any is used. As in the walker, lanes whose
 * row is at or past a range's end re-read the range's last row. sink gets
 * one uint32 per wave (`waves` words): the XOR of words 0 and 3 of every
 * 16-byte piece of the K rows and words 1 and 2 of every 16-byte piece of
 * the V rows in range (each once), the same fold as pkv_probe_gather.
 */
PKV_API int pkv_probe_gather_mfma(const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, int max_blocks_per_seq,
                                  const int32_t* seq_lens, int num_seqs, int num_kv_heads,
                                  int row_bytes, int block_size, int num_blocks, int waves,
                                  int chunks_per_round, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
