"""Plain, slow, float64 CPU oracle for PagedAttention decode.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the bench's
CPU-baseline leg, never by the product path. It shares no code, header, table
or helper with the HIP library.

Sources are three web pages, cited by title and section:

  [summary] supersilo.blog, summary of the vLLM / PagedAttention paper
            (writing/llm/2026/01/04/vllm).
  [meetup]  blog.aqudi.me, "벤치마크가 다가 아니야! vLLM으로 보는 LLM 추론 최적화".
  [day3]    hjr-study-book, "[LLM 추론 최적화] Day 3: KV 캐시와 Continuous Batching".

What each function computes, in the pages' terms:

* Attention for one decode step ([summary] §"자기회귀 생성과 KV 캐시"): the new
  query of a sequence scores every valid key, past and current, as q.k / sqrt(d_k);
  the scores are softmax-normalised over those positions and weight the values.
* Paging ([summary] §"PagedAttention의 설계"; [day3] §4.2): the cache of a sequence
  is cut into fixed-size blocks; a per-sequence block table sends logical block b
  to a physical block that need not be adjacent to the others. The kernel reads
  K/V through the table in logical order and the softmax is taken once over all
  valid tokens, not per block. So the paged result is, by definition, the dense
  result over the logically ordered history: the oracle gathers that history
  through the table and runs dense attention on it.
* Append ([summary] §"자기회귀 생성과 KV 캐시"; [day3] §1): a decode step stores
  the new token's K/V after the cached ones.
* Block copy ([summary] §"블록 공유"; [meetup] §3): shared blocks are copied only
  when one holder must modify them (copy-on-write); the copy is a plain block
  image copy.

Readings where the pages are silent (each is listed in the design notes):
* seq_lens counts the new token: a sequence of length L attends over positions
  0..L-1 and the appended token sits at position L-1.
* A sequence of length 0 is a padding row: nothing is appended and its output
  row is zero.
* Grouped-query attention: query head h uses KV head h // (H / H_kv).
* Pool layout [num_blocks][H_kv][block_size][head_dim] (a layout choice; the
  pages give none).
"""

import numpy as np


def block_and_slot(position, block_size):
    """Logical block index and slot of a token position.

    [day3] §4.2 with 16-token blocks: a 37-token sequence spans logical
    blocks 0, 1, 2 and the third block holds 5 tokens, so token t lies in
    logical block t // block_size at offset t % block_size.
    """
    return position // block_size, position % block_size


def gather_sequence(pool, table_row, n_tokens, block_size):
    """The logically ordered history of one sequence, read through its table.

    pool: [num_blocks][H_kv][block_size][D]; table_row: logical -> physical
    block ids. Returns [n_tokens][H_kv][D]. ([summary] §"PagedAttention의 설계":
    K/V are fetched through the block table in logical order.)
    """
    out = np.empty((n_tokens, pool.shape[1], pool.shape[3]), dtype=pool.dtype)
    for t in range(n_tokens):
        logical, slot = block_and_slot(t, block_size)
        physical = int(table_row[logical])
        out[t] = pool[physical, :, slot, :]
    return out


def dense_decode_attention(q, k, v, scale):
    """Dense single-query attention of one sequence, in float64.

    q: [H][D] (the new token's queries), k, v: [L][H_kv][D] (the full
    contiguous history including the new token). Returns [H][D].

    [summary] §"자기회귀 생성과 KV 캐시": scores are q.k_j * scale over every
    valid position j, normalised by one softmax over all of them, and the
    output is the score-weighted sum of the values. Query head h reads KV
    head h // (H / H_kv).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    num_heads, head_dim = q.shape
    seq_len, num_kv_heads, _ = k.shape
    group = num_heads // num_kv_heads
    out = np.zeros((num_heads, head_dim), dtype=np.float64)
    if seq_len == 0:
        return out
    for h in range(num_heads):
        g = h // group
        scores = scale * (k[:, g, :] @ q[h])          # [L]
        weights = np.exp(scores - scores.max())       # softmax numerator, shifted
        out[h] = (weights @ v[:, g, :]) / weights.sum()
    return out


def paged_decode_attention(q, k_pool, v_pool, block_tables, seq_lens,
                           block_size, scale):
    """Decode attention for a batch whose KV history sits in a paged pool.

    q: [B][H][D]; k_pool, v_pool: [num_blocks][H_kv][block_size][D];
    block_tables: [B][max_blocks]; seq_lens: [B] (new token included).
    Returns float64 [B][H][D]. Each row is the dense attention over that
    sequence's history gathered through its table; rows with length 0 are zero.
    """
    batch, num_heads, head_dim = q.shape
    out = np.zeros((batch, num_heads, head_dim), dtype=np.float64)
    for i in range(batch):
        n = int(seq_lens[i])
        if n <= 0:
            continue
        k = gather_sequence(k_pool, block_tables[i], n, block_size)
        v = gather_sequence(v_pool, block_tables[i], n, block_size)
        out[i] = dense_decode_attention(q[i], k, v, scale)
    return out


def pool_after_append(k_pool, v_pool, k_new, v_new, block_tables, seq_lens,
                      block_size):
    """The pools after each sequence stores its new token's K/V.

    k_new, v_new: [B][H_kv][D]; seq_lens counts the new token, so it goes to
    position L-1, i.e. slot (L-1) % block_size of physical block
    table[(L-1) // block_size]. Length-0 rows store nothing. Works on raw
    (e.g. integer-viewed) arrays, so the result is bit-exact. Returns copies.
    """
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for i in range(len(seq_lens)):
        n = int(seq_lens[i])
        if n <= 0:
            continue
        logical, slot = block_and_slot(n - 1, block_size)
        physical = int(block_tables[i][logical])
        k_out[physical, :, slot, :] = k_new[i]
        v_out[physical, :, slot, :] = v_new[i]
    return k_out, v_out


def pool_after_copy(k_pool, v_pool, pairs):
    """The pools after copy-on-write block copies.

    pairs: [P][2] of (source, destination) physical block ids, applied in
    order; each copies the whole block image (all KV heads, all slots) of K
    and of V. Returns copies.
    """
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for src, dst in np.asarray(pairs).reshape(-1, 2):
        k_out[int(dst)] = k_out[int(src)]
        v_out[int(dst)] = v_out[int(src)]
    return k_out, v_out


def pool_after_swap(src_k, src_v, dst_k, dst_v, pairs):
    """The destination pools after moving blocks between two pools (a device
    pool and a host pool, in either direction): swapping preempted sequences
    to CPU memory and back (supersilo.blog vLLM/PagedAttention summary,
    section "적용 범위와 관련 연구").

    pairs: [P][2] of (source block of src, destination block of dst); each
    copies the whole block image of K and of V. The sources are not changed.
    Returns copies of the destination pools.
    """
    k_out = dst_k.copy()
    v_out = dst_v.copy()
    for src, dst in np.asarray(pairs).reshape(-1, 2):
        k_out[int(dst)] = src_k[int(src)]
        v_out[int(dst)] = src_v[int(src)]
    return k_out, v_out


def paged_multi_query_attention(q, k_pool, v_pool, block_tables, seq_lens, block_size, scale):
    """Attention of several new tokens per sequence over a paged pool.

    blog.aqudi.me ("벤치마크가 다가 아니야! vLLM으로 보는 LLM 추론 최적화",
    section 4): chunked prefill feeds a long prompt in pieces between decode
    steps, and speculative decoding has the large model check several
    proposed tokens in one pass; both attend several new tokens of a sequence
    to its cached history. q: [B][nq][H][D]; seq_lens count all nq new tokens,
    which sit at positions L-nq .. L-1, so new token j (position L-nq+j) sees
    the tokens at positions 0 .. L-nq+j -- the causal rule of the summary
    page's "자기회귀 생성과 KV 캐시" section, current position included. A
    query whose position is negative (L < nq - j) gets a zero row.
    Returns float64 [B][nq][H][D].
    """
    batch, nq, num_heads, head_dim = q.shape
    out = np.zeros((batch, nq, num_heads, head_dim), dtype=np.float64)
    for i in range(batch):
        n = int(seq_lens[i])
        for j in range(nq):
            pos = n - nq + j
            if pos < 0:
                continue
            k = gather_sequence(k_pool, block_tables[i], pos + 1, block_size)
            v = gather_sequence(v_pool, block_tables[i], pos + 1, block_size)
            out[i, j] = dense_decode_attention(q[i, j], k, v, scale)
    return out


def pool_after_append_multi(k_pool, v_pool, k_new, v_new, block_tables, seq_lens, block_size):
    """The pools after each sequence stores nq new tokens: k_new, v_new
    [B][nq][H_kv][D]; token j goes to position L-nq+j (skipped if negative).
    Raw (bit-exact) copies, like pool_after_append."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    nq = k_new.shape[1]
    for i in range(len(seq_lens)):
        n = int(seq_lens[i])
        for j in range(nq):
            pos = n - nq + j
            if pos < 0:
                continue
            logical, slot = block_and_slot(pos, block_size)
            physical = int(block_tables[i][logical])
            k_out[physical, :, slot, :] = k_new[i, j]
            v_out[physical, :, slot, :] = v_new[i, j]
    return k_out, v_out
