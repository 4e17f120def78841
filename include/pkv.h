/*
 * pkv.h - paged KV cache decode on AMD MI355X (gfx950): C ABI.
 *
 * Three operations over a KV cache cut into fixed-size blocks, each sequence
 * finding its blocks through a block table (supersilo.blog vLLM/PagedAttention
 * summary, section "PagedAttention의 설계" -- cited below as [summary];
 * hjr-study-book "Day 3: KV 캐시와 Continuous Batching", section 4.2):
 *   pkv_kv_cache_append        store the new token's K/V in the slot its table names
 *   pkv_copy_blocks            copy whole blocks (the copy behind copy-on-write sharing)
 *   pkv_paged_attention_decode single-query attention over each sequence's
 *                              blocks, one softmax over all valid tokens
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.  Every pointer argument is a DEVICE pointer to memory the caller
 *   allocated on the current HIP device and keeps alive until the enqueued work
 *   has finished. The library allocates and frees nothing.
 * Streams. `stream` is a hipStream_t (NULL = the null stream). Each call only
 *   enqueues kernels on it and returns; results are visible to later work on
 *   the same stream. Calls on different streams that touch the same pool
 *   buffers race (the caller orders them).
 * Layouts (row-major, no padding):
 *   k_pool, v_pool   [num_blocks][num_kv_heads][block_size][head_dim]
 *   block_tables     int32 [num_seqs][max_blocks_per_seq]: logical block b of
 *                    sequence i lives in physical block block_tables[i][b]
 *   seq_lens         int32 [num_seqs]: number of valid tokens of each sequence
 *                    INCLUDING the token appended this step (0 = padding row)
 *   q, out           [num_seqs][num_heads][head_dim]
 *   k_new, v_new     [num_seqs][num_kv_heads][head_dim]
 *   block_mapping    int32 [num_pairs][2] = (source block, destination block)
 * Alignment.  q, out, k_pool, v_pool, k_new and v_new must be 16-byte
 *   aligned (the kernels move them 16 bytes at a time); PKV_ERR_INVALID
 *   otherwise.
 * Element types.  pkv_dtype. In pkv_kv_cache_append and
 *   pkv_paged_attention_decode all of q, k_new, v_new, k_pool, v_pool share
 *   one of F32, F16, BF16. PKV_FP8_E4M3 is a pool storage type: pools of
 *   8-bit codes with one float scale per kv head for K and for V, written by
 *   pkv_kv_cache_append_fp8 and read by pkv_paged_attention_decode_fp8;
 *   pkv_copy_blocks copies any pool type (scales are per head, not per
 *   block, so a block copy needs nothing else).
 * Supported shapes.  head_dim 64 or 128 (128 for FP8 pools); block_size a
 *   power of two in [8, 256]; num_heads / num_kv_heads in {1, 2, 4, 8}.
 * Device-resident values (table entries, seq_lens, block_mapping) are the
 *   caller's contract and are not read by the host. The kernels never access
 *   memory outside the buffers described above: a table entry outside
 *   [0, num_blocks) is clamped into range by attention (its result is then
 *   meaningless) and skipped by append and copy; a length above
 *   max_blocks_per_seq * block_size (or above max_seq_len, for attention) is
 *   clamped to it. Each of these events can be reported through an error
 *   word (pkv_set_error_word, below).
 * Errors.  Every entry point returns a pkv_status. Host-checkable problems
 *   return a negative status before anything is enqueued; PKV_ERR_HIP means the
 *   HIP runtime rejected a launch. No C++ exception crosses this interface.
 * Threads.  Calls are reentrant. The only global state is per device: a
 *   cache of the compute-unit count, filled on first use, and the registered
 *   error word; both are thread-safe.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define PKV_API __attribute__((visibility("default")))
#else
#define PKV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_FP8_E4M3 = 3 } pkv_dtype;

typedef enum {
    PKV_OK = 0,
    PKV_ERR_INVALID = -1,     /* null pointer, negative size, inconsistent arguments */
    PKV_ERR_UNSUPPORTED = -2, /* head_dim / block_size / head grouping / dtype not built */
    PKV_ERR_WORKSPACE = -3,   /* split-K workspace missing, misaligned or too small */
    PKV_ERR_HIP = -4,         /* the HIP runtime reported an error when launching */
    PKV_ERR_NO_BLOCKS = -5,   /* block manager: the pool has no free block */
    PKV_ERR_SCRATCH = -6      /* the call needs more scratch than the static buffer holds */
} pkv_status;

/*
 * Store each sequence's new token ([summary] section "자기회귀 생성과 KV 캐시":
 * a decode step appends the new token's K/V after the cached ones; Day 3
 * section 1 lists the same step per token).
 *
 * For every sequence i with L = seq_lens[i] > 0, the token goes to position
 * L-1: slot (L-1) % block_size of physical block
 * block_tables[i][(L-1) / block_size], for all num_kv_heads heads, K into
 * k_pool and V into v_pool. The copy is bit-exact; nothing else in the pools
 * is written. Rows with L <= 0, or whose target block id is outside
 * [0, num_blocks), or whose logical block is >= max_blocks_per_seq, are skipped.
 */
PKV_API int pkv_kv_cache_append(const void* k_new, const void* v_new,
                        void* k_pool, void* v_pool,
                        const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* seq_lens,
                        int num_seqs, int num_kv_heads, int head_dim, int block_size,
                        int num_blocks, pkv_dtype dtype, void* stream);

/*
 * Copy whole blocks, K and V ([summary] section "블록 공유" and blog.aqudi.me
 * "벤치마크가 다가 아니야! vLLM으로 보는 LLM 추론 최적화" section 3: a block
 * shared by several sequences is copied only when one of them must write to
 * it, i.e. copy-on-write).
 *
 * For each pair (src, dst) of block_mapping, block dst of k_pool (and of
 * v_pool) becomes a bit-exact image of block src: all num_kv_heads heads,
 * all block_size slots. Destinations must be distinct and must not be sources
 * in the same call (the pairs run concurrently). Pairs with an id outside
 * [0, num_blocks) are skipped. num_pairs == 0 enqueues nothing.
 */
PKV_API int pkv_copy_blocks(void* k_pool, void* v_pool,
                    const int32_t* block_mapping, int num_pairs,
                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                    pkv_dtype dtype, void* stream);

/* partition_size value that selects the balanced schedule (see below). */
#define PKV_PARTITION_BALANCED (-1)

/*
 * kv_policy of the attention entry points: how K/V are read. It changes
 * speed only, never a result bit.
 *   PKV_KV_STREAM  every block is read by one sequence of the batch: K/V are
 *                  read with non-temporal loads, which stream through the
 *                  caches without displacing reused data (the fast choice
 *                  when no block is shared);
 *   PKV_KV_REUSE   blocks may be shared by several sequences of the batch (a
 *                  common prompt prefix, parallel sampling; [summary] section
 *                  "블록 공유"): ordinary cached loads, so that a shared
 *                  block read by one sequence is found in cache by the
 *                  others (pair it with fixed partitions, which run
 *                  neighbouring sequences side by side).
 */
#define PKV_KV_STREAM 0
#define PKV_KV_REUSE 1

/*
 * Launch stages, OR-ed into kv_policy of any attention entry point. Under a
 * split schedule (fixed partitions or PKV_PARTITION_BALANCED) a call is two
 * launches: the walk over the K/V blocks, which writes the rows of segments
 * it finishes and leaves partial results of split segments in the
 * workspace, and the log-sum-exp merge of those partial results, which
 * writes the remaining rows. By default one call enqueues both.
 *   PKV_STAGE_WALK   enqueue only the walk;
 *   PKV_STAGE_MERGE  enqueue only the merge. Call it after a PKV_STAGE_WALK
 *                    call with the same arguments and the same workspace,
 *                    untouched in between, on the same stream; out is
 *                    complete after it. Under a single pass there is
 *                    nothing to merge and it enqueues nothing.
 * Setting both is PKV_ERR_INVALID. For callers that place other work, or
 * timing events, between the two launches; results are identical bits.
 */
#define PKV_STAGE_WALK 0x10
#define PKV_STAGE_MERGE 0x20

/*
 * PKV_WALKER_VECTOR, OR-ed into kv_policy of pkv_paged_attention_decode (and
 * only there): run 4 or 8 query heads per kv head (16-bit K/V, head_dim 128)
 * on the vector units instead of the matrix cores. For measurement: it shows
 * what the matrix cores buy on grouped-query layers. Results agree with the
 * default within the same tolerance, not bit for bit. Streaming policy only
 * (PKV_ERR_UNSUPPORTED with PKV_KV_REUSE); no effect where the vector walker
 * is the default already.
 */
#define PKV_WALKER_VECTOR 0x40

/*
 * Bytes of workspace pkv_paged_attention_decode needs for the given sizes and
 * partition_size (0 when it needs none: partition_size == 0, or every
 * sequence fits one partition). Returns 0 for invalid sizes as well. For
 * PKV_PARTITION_BALANCED the size depends only on head_dim and the head
 * grouping: 2 * 4096 * (num_heads / num_kv_heads) * (head_dim + 2) * 4 bytes
 * of partial records plus 2 * 4096 * 4 bytes of merge information, and 0
 * when num_heads / num_kv_heads exceeds 16 (more than 16 columns per kv head
 * run the balanced schedule as a single pass).
 */
PKV_API size_t pkv_paged_attention_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                          int head_dim, int max_seq_len, int partition_size);

/*
 * Single-query decode attention through block tables ([summary] sections
 * "자기회귀 생성과 KV 캐시" and "PagedAttention의 설계").
 *
 * For each sequence i (L = seq_lens[i]) and query head h, with kv head
 * g = h / (num_heads / num_kv_heads):
 *   out[i][h] = sum_{t < L} softmax_t(scale * q[i][h] . K_i[t][g]) * V_i[t][g]
 * where K_i[t], V_i[t] are read from slot t % block_size of physical block
 * block_tables[i][t / block_size]. The softmax is one normalisation over all
 * L tokens, not a per-block one. Rows with L == 0 are written as zeros.
 * Slots at or past L are never used (they may hold any bits, NaN included).
 *
 * out_dtype selects the output element type (PKV_F32 keeps the fp32
 * accumulation; F16/BF16 round to nearest even). Arithmetic is fp32
 * regardless of the input type.
 *
 * max_seq_len must bound every seq_lens entry (it sizes the launch) and must
 * not exceed max_blocks_per_seq * block_size.
 *
 * partition_size selects how the tokens are split over the GPU's waves; the
 * result is the same attention up to floating-point summation order:
 *   0                       one pass per (sequence, kv head);
 *   a positive multiple of 64
 *                           each sequence is cut into partitions of that many
 *                           tokens, handled independently and merged by a
 *                           log-sum-exp reduce. Under PKV_KV_REUSE, the
 *                           sequences next to each other in the batch are
 *                           processed side by side, so blocks they share
 *                           (parallel sampling) are read once from HBM and
 *                           then from cache;
 *   PKV_PARTITION_BALANCED  a fixed set of persistent waves (4 or 8 per
 *                           compute unit, depending on the kernel, or as
 *                           many as fit when the (sequence, kv head) pairs
 *                           outnumber twice that; at most 4096) each takes
 *                           an equal share of
 *                           all tokens of the batch, whatever the lengths;
 *                           pieces of a sequence split between waves are
 *                           merged by a log-sum-exp reduce (in LDS among
 *                           the waves of a workgroup, through the workspace
 *                           and the merge launch across workgroups). The
 *                           split points
 *                           depend on the lengths of the whole batch, so a
 *                           row's rounding can change when other rows change
 *                           (under 0 or fixed partitions it cannot: a row's
 *                           bits depend on its own sequence only).
 * When a split is possible, `workspace` (16-byte aligned, at least
 * pkv_paged_attention_workspace_size(...) bytes, contents ignored and
 * overwritten) holds the partial results. Work enqueued on `stream` by
 * different calls must not share a workspace unless ordered by the stream.
 *
 * A PKV_STAGE_MERGE call is the exception: it reads the workspace its
 * PKV_STAGE_WALK call left.
 *
 * kv_policy is PKV_KV_STREAM or PKV_KV_REUSE, optionally with one stage
 * flag (see above; PKV_ERR_INVALID otherwise).
 */
PKV_API int pkv_paged_attention_decode(void* out, pkv_dtype out_dtype,
                               const void* q,
                               const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* seq_lens, int max_seq_len,
                               int num_seqs, int num_heads, int num_kv_heads,
                               int head_dim, int block_size, int num_blocks,
                               float scale, int partition_size,
                               void* workspace, size_t workspace_bytes,
                               pkv_dtype dtype, int kv_policy, void* stream);

/*
 * pkv_paged_attention_decode without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. The split-K records go to a
 * static device array of the library instead, PKV_NOALLOC_SCRATCH_BYTES
 * bytes, one copy per device, held from the library's first use on that
 * device until the process ends. Arguments, results (the same bits) and
 * errors are those of pkv_paged_attention_decode, plus PKV_ERR_SCRATCH,
 * before anything is enqueued, when pkv_paged_attention_workspace_size(...)
 * for these arguments exceeds PKV_NOALLOC_SCRATCH_BYTES (the balanced
 * schedule fits for up to 8 query heads per kv head at head_dim 128). The
 * call allocates nothing; its first call on a device looks up that
 * device's copy of the array. Every call on a device shares its copy, which
 * keeps the last call's contents: calls that can overlap on one device
 * (different streams, or different host threads) race and give wrong
 * results; so does any such call between a PKV_STAGE_WALK call and its
 * PKV_STAGE_MERGE call.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)40 << 20)
PKV_API int pkv_paged_attention_decode_noalloc(void* out, pkv_dtype out_dtype, const void* q,
                               const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* seq_lens, int max_seq_len,
                               int num_seqs, int num_heads, int num_kv_heads,
                               int head_dim, int block_size, int num_blocks,
                               float scale, int partition_size,
                               pkv_dtype dtype, int kv_policy, void* stream);

/*
 * Decode attention for parallel sampling ([summary] section "블록 공유": the
 * samples of one prompt share the prompt's blocks, by reference). The batch
 * is cut into groups of group_size consecutive sequences (num_seqs must be a
 * multiple of group_size); shared_tokens (device int32 [num_seqs /
 * group_size]) gives, per group, how many leading tokens every sequence of
 * the group reads from the same physical blocks (the caller's contract: a
 * block manager knows it; pkv_bm_shared_prefix computes it). The result is
 * that of pkv_paged_attention_decode with the same arguments, up to
 * floating-point summation order.
 *
 * partition_size must be a positive multiple of 64 (fixed partitions). A
 * partition lying inside the tokens its group shares (for a sequence of
 * length L: ending at or before min(shared_tokens, L - 1)) is computed once
 * for the whole group on the matrix cores, the group's queries forming the
 * columns, so its blocks are read from HBM once instead of once per sample;
 * every other partition is computed per sequence. F16 / BF16 K/V and q,
 * head_dim 128, group_size * (num_heads / num_kv_heads) <= 16
 * (PKV_ERR_UNSUPPORTED otherwise). The workspace is sized as for
 * pkv_paged_attention_decode with the same partition_size. shared_tokens = 0
 * everywhere gives exactly the bits of pkv_paged_attention_decode.
 */
PKV_API int pkv_paged_attention_decode_grouped(void* out, pkv_dtype out_dtype, const void* q,
                               const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* seq_lens, int max_seq_len,
                               int num_seqs, int num_heads, int num_kv_heads,
                               int head_dim, int block_size, int num_blocks,
                               float scale, int partition_size,
                               int group_size, const int32_t* shared_tokens,
                               void* workspace, size_t workspace_bytes,
                               pkv_dtype dtype, int kv_policy, void* stream);

/*
 * Several new tokens per sequence (blog.aqudi.me "벤치마크가 다가 아니야!
 * vLLM으로 보는 LLM 추론 최적화", section 4: chunked prefill feeds a long
 * prompt in pieces between decode steps; speculative decoding checks several
 * proposed tokens in one pass of the large model). Sequence i of (new) length
 * L holds its num_queries (nq) new tokens at positions L-nq .. L-1.
 *
 * pkv_kv_cache_append_multi: k_new, v_new [num_seqs][nq][num_kv_heads]
 * [head_dim]; new token j goes to position L-nq+j (skipped when negative),
 * bit-exact, as pkv_kv_cache_append does for one token. nq = 1 is that call.
 *
 * pkv_paged_attention_multi: q and out [num_seqs][nq][num_heads][head_dim];
 * new token j (position p = L-nq+j) attends causally to positions 0 .. p:
 *   out[i][j][h] = sum_{t <= p} softmax_t(scale * q[i][j][h] . K_i[t][g]) V_i[t][g]
 * (a token with p < 0 gets a zero row). F16 / BF16 K/V and q, head_dim 128
 * (PKV_ERR_UNSUPPORTED otherwise). The nq * (num_heads / num_kv_heads)
 * (query token, head) columns of a (sequence, kv head) run on the matrix
 * cores 16 at a time; each group of 16 reads the cache only up to the causal
 * limit of its last column, so a long prefill chunk costs its causal work,
 * not nq times the history. partition_size, kv_policy and the workspace work
 * as in pkv_paged_attention_decode, except that with more than 16 columns
 * PKV_PARTITION_BALANCED runs as a single pass over each group of 16 columns
 * (the groups fill the GPU; no workspace). Size the workspace with
 * pkv_paged_attention_workspace_size(num_seqs, num_heads * nq, num_kv_heads,
 * head_dim, max_seq_len, partition_size).
 */
PKV_API int pkv_kv_cache_append_multi(const void* k_new, const void* v_new,
                              void* k_pool, void* v_pool,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* seq_lens, int num_seqs, int num_queries,
                              int num_kv_heads, int head_dim, int block_size,
                              int num_blocks, pkv_dtype dtype, void* stream);

PKV_API int pkv_paged_attention_multi(void* out, pkv_dtype out_dtype, const void* q,
                              const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, int max_blocks_per_seq,
                              const int32_t* seq_lens, int max_seq_len,
                              int num_seqs, int num_queries, int num_heads, int num_kv_heads,
                              int head_dim, int block_size, int num_blocks,
                              float scale, int partition_size,
                              void* workspace, size_t workspace_bytes,
                              pkv_dtype dtype, int kv_policy, void* stream);

/*
 * FP8 KV cache (blog.aqudi.me "벤치마크가 다가 아니야! vLLM으로 보는 LLM 추론
 * 최적화", section 4: lowering the precision of the KV cache saves memory
 * and bandwidth). Storage is OCP FP8 E4M3: a code s eeee mmm stands for
 * (-1)^s 2^(e-7) (1 + m/8), or (-1)^s 2^-6 m/8 when e = 0; s 1111 111 is
 * NaN; the largest finite magnitude is 448. A stored code c of kv head g
 * means value(c) * k_scales[g] in k_pool (v_scales[g] in v_pool).
 *
 * pkv_kv_cache_append_fp8: as pkv_kv_cache_append, but k_new / v_new
 * ([num_seqs][num_kv_heads][head_dim], new_dtype F32, F16 or BF16) are
 * quantised into the uint8 pools: each element x of head g becomes the
 * E4M3 code nearest to float32(x) / k_scales[g] (IEEE float32 division;
 * ties to the even code; magnitudes beyond 448 saturate to 448; NaN stays
 * NaN). k_scales / v_scales are device float arrays [num_kv_heads], read by
 * the kernel. head_dim must be 128.
 */
PKV_API int pkv_kv_cache_append_fp8(const void* k_new, const void* v_new, pkv_dtype new_dtype,
                            void* k_pool, void* v_pool,
                            const float* k_scales, const float* v_scales,
                            const int32_t* block_tables, int max_blocks_per_seq,
                            const int32_t* seq_lens,
                            int num_seqs, int num_kv_heads, int head_dim, int block_size,
                            int num_blocks, void* stream);

/*
 * pkv_paged_attention_decode_fp8: as pkv_paged_attention_decode, over uint8
 * E4M3 pools with per-head scales: K_i[t][g] = value(code) * k_scales[g],
 * V_i[t][g] = value(code) * v_scales[g]. q has q_dtype (F32, F16 or BF16);
 * arithmetic is fp32 as in the 16-bit path. head_dim must be 128; with more
 * than one query head per kv head q must be F16 or BF16. The workspace is sized by
 * pkv_paged_attention_workspace_size exactly as for the 16-bit path; kv_policy
 * is as there.
 */
PKV_API int pkv_paged_attention_decode_fp8(void* out, pkv_dtype out_dtype,
                               const void* q, pkv_dtype q_dtype,
                               const void* k_pool, const void* v_pool,
                               const float* k_scales, const float* v_scales,
                               const int32_t* block_tables, int max_blocks_per_seq,
                               const int32_t* seq_lens, int max_seq_len,
                               int num_seqs, int num_heads, int num_kv_heads,
                               int head_dim, int block_size, int num_blocks,
                               float scale, int partition_size,
                               void* workspace, size_t workspace_bytes, int kv_policy,
                               void* stream);

/*
 * Error word: reports of device-resident values outside the contract above.
 * The block table is the paged kernel's extra indirection ([summary] section
 * "PagedAttention의 설계"; section "커널 비용과 블록 크기" counts the table
 * lookups as its added cost), so a corrupted entry is a likely failure, and
 * the kernels' clamps keep it from faulting but not from giving wrong numbers.
 *
 * pkv_set_error_word registers, for the CURRENT device, a caller-owned
 * device int32 (4-byte aligned) into which every later call's kernels on
 * that device OR these bits:
 *   PKV_ERRBIT_TABLE   attention met a table entry of a valid logical block
 *                      (block < ceil(L / block_size)) outside [0, num_blocks);
 *                      it read a clamped block instead, so that row's output
 *                      is meaningless
 *   PKV_ERRBIT_LENGTH  attention met a length below 0 or above max_seq_len
 *                      and clamped it
 *   PKV_ERRBIT_APPEND  an append skipped a new token whose logical block is
 *                      at or past max_blocks_per_seq or whose table entry is
 *                      outside [0, num_blocks)
 *   PKV_ERRBIT_COPY    a block copy or swap skipped a pair with an id outside
 *                      its pool
 * Bits are set with device atomics from the kernels and never cleared by the
 * library: the caller zeroes the word, runs its calls, synchronises and reads
 * it. NULL (the default) switches the reports off. Calls already enqueued
 * keep the word they were enqueued with, so the word must stay allocated
 * until they finish. Calls on one device share its word. Returns
 * PKV_ERR_INVALID for a misaligned pointer, PKV_ERR_HIP if there is no
 * current device.
 */
#define PKV_ERRBIT_TABLE 0x1
#define PKV_ERRBIT_LENGTH 0x2
#define PKV_ERRBIT_APPEND 0x4
#define PKV_ERRBIT_COPY 0x8
PKV_API int pkv_set_error_word(int32_t* error_word);

/*
 * The multi-query and sampling-group calls over FP8 pools (blog.aqudi.me
 * section 4 names both a lower-precision KV cache and the several-token
 * passes of chunked prefill and speculative decoding; [summary] section
 * "블록 공유" the samples sharing a prompt's blocks).
 *
 * pkv_kv_cache_append_multi_fp8: pkv_kv_cache_append_multi into uint8 E4M3
 * pools, each new token quantised as pkv_kv_cache_append_fp8 quantises its
 * one token; k_new / v_new are [num_seqs][num_queries][num_kv_heads][128] of
 * new_dtype. num_queries = 1 is pkv_kv_cache_append_fp8.
 *
 * pkv_paged_attention_multi_fp8: pkv_paged_attention_multi over E4M3 pools
 * with per-head scales (values as in pkv_paged_attention_decode_fp8); q is
 * F16 or BF16 and sets the type the matrix cores compute in (the codes widen
 * to it exactly). Same shapes, column groups, schedules, workspace and
 * errors as pkv_paged_attention_multi.
 *
 * pkv_paged_attention_decode_grouped_fp8: pkv_paged_attention_decode_grouped
 * over E4M3 pools, q F16 or BF16: partitions inside a group's shared tokens
 * are read once per group on the matrix cores; every other partition per
 * sequence (the FP8 decode walker). Same arguments, limits, workspace and
 * errors as pkv_paged_attention_decode_grouped.
 */
PKV_API int pkv_kv_cache_append_multi_fp8(const void* k_new, const void* v_new,
                                          pkv_dtype new_dtype, void* k_pool, void* v_pool,
                                          const float* k_scales, const float* v_scales,
                                          const int32_t* block_tables, int max_blocks_per_seq,
                                          const int32_t* seq_lens, int num_seqs,
                                          int num_queries, int num_kv_heads, int head_dim,
                                          int block_size, int num_blocks, void* stream);

PKV_API int pkv_paged_attention_multi_fp8(void* out, pkv_dtype out_dtype,
                                          const void* q, pkv_dtype q_dtype,
                                          const void* k_pool, const void* v_pool,
                                          const float* k_scales, const float* v_scales,
                                          const int32_t* block_tables, int max_blocks_per_seq,
                                          const int32_t* seq_lens, int max_seq_len,
                                          int num_seqs, int num_queries, int num_heads,
                                          int num_kv_heads, int head_dim, int block_size,
                                          int num_blocks, float scale, int partition_size,
                                          void* workspace, size_t workspace_bytes,
                                          int kv_policy, void* stream);

PKV_API int pkv_paged_attention_decode_grouped_fp8(void* out, pkv_dtype out_dtype,
                                          const void* q, pkv_dtype q_dtype,
                                          const void* k_pool, const void* v_pool,
                                          const float* k_scales, const float* v_scales,
                                          const int32_t* block_tables, int max_blocks_per_seq,
                                          const int32_t* seq_lens, int max_seq_len,
                                          int num_seqs, int num_heads, int num_kv_heads,
                                          int head_dim, int block_size, int num_blocks,
                                          float scale, int partition_size, int group_size,
                                          const int32_t* shared_tokens,
                                          void* workspace, size_t workspace_bytes,
                                          int kv_policy, void* stream);

/* Static, NUL-terminated description of a pkv_status value. */
PKV_API const char* pkv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
