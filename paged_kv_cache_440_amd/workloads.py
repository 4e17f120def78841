"""Seeded synthetic decode workloads for the paged KV cache.

This module only draws inputs: sequence lengths, the assignment of physical
blocks to sequences (a seeded permutation of the pool), pool contents, the new
tokens' K/V and the queries. It computes nothing of attention, append or copy,
and imports neither the HIP binding nor the oracle; both sides consume what it
returns.

Shapes follow the pages' workloads (OPT-13B and LLaMA-13B attention layers,
parallel sampling from a shared prompt, 16-token blocks) with synthetic values:
the pages' datasets (ShareGPT, Alpaca) are replaced by seeded length
distributions of the same character.

Layout of what is returned (all host tensors, moved to the GPU by the caller):
  k_pool, v_pool : [num_blocks][num_kv_heads][block_size][head_dim]
  block_tables   : int32 [num_seqs][max_blocks], padded with -1
  seq_lens       : int32 [num_seqs], lengths including the token appended
                   this step
  k_new, v_new   : [num_seqs][num_kv_heads][head_dim]
  q              : [num_seqs][num_heads][head_dim]
Blocks that no table names are filled with NaN; every slot of a block that
some table names holds a finite draw (slots past a sequence's length hold
stale finite values).
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

_CHUNK = 1 << 22          # elements per independently seeded chunk of a pool
SEED_BASE = 4400

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Workload:
    name: str
    dtype: torch.dtype
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    num_blocks: int
    seq_lens: np.ndarray
    block_tables: np.ndarray
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    q: torch.Tensor
    copy_pairs: np.ndarray = field(default_factory=lambda: np.zeros((0, 2), np.int32))
    # Tokens that must be appended, one decode step at a time, after the
    # copies and before the step's own append: [steps][B][Hkv][D] and the
    # lengths (after each of those appends) per step, 0 = no append.
    pending_k: torch.Tensor | None = None
    pending_v: torch.Tensor | None = None
    pending_lens: np.ndarray | None = None
    info: dict = field(default_factory=dict)
    # FP8 pools: uint8 E4M3 codes; a code of kv head g means value * scale[g]
    k_scales: torch.Tensor | None = None
    v_scales: torch.Tensor | None = None
    # several new tokens per sequence: k_new, v_new [B][nq][Hkv][D] and
    # q [B][nq][H][D]; seq_lens count them, they sit at L-nq .. L-1
    num_queries: int = 1
    # several tables name the same physical blocks (a shared prompt prefix)
    shared_blocks: bool = False

    @property
    def fp8(self) -> bool:
        return self.k_scales is not None

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self) -> int:
        """Bytes of one stored K/V element (1 for FP8 pools)."""
        return self.k_pool.element_size()

    def kv_bytes(self) -> int:
        """Bytes of K and V history one decode step reads: sum_i L_i * 2*Hkv*D*eb."""
        per_token = 2 * self.num_kv_heads * self.head_dim * self.elem_bytes
        return int(self.seq_lens.astype(np.int64).sum()) * per_token

    def unique_kv_bytes(self) -> int:
        """The same over distinct (physical block, slot) pairs: what HBM must
        deliver at least once when tables share blocks (equal to kv_bytes
        when they do not)."""
        if not self.shared_blocks:
            return self.kv_bytes()
        bs = self.block_size
        slots = set()
        for i, n in enumerate(self.seq_lens):
            n = int(n)
            nb = -(-n // bs)
            for b in range(nb):
                phys = int(self.block_tables[i, b])
                used = min(bs, n - b * bs)
                slots.update((phys, s) for s in range(used))
        per_token = 2 * self.num_kv_heads * self.head_dim * self.elem_bytes
        return len(slots) * per_token


# ----------------------------------------------------------------------------
# value draws

def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw_into(out: torch.Tensor, seed_seq: np.random.SeedSequence, dist: str,
               fp8_scales: np.ndarray | None = None, row_elems: int = 1) -> None:
    """Fill a flat host tensor with seeded draws, chunk by chunk.

    Each fixed-size chunk has its own child seed, so the values do not depend
    on the number of threads. Draws are float32, rounded to the target dtype
    to nearest-even. For a uint8 (FP8) tensor, element i belongs to kv head
    (i // row_elems) % len(fp8_scales) and stores torch's float8_e4m3fn
    conversion of draw / scale of that head.
    """
    flat = out.view(-1)
    n = flat.numel()
    nchunks = (n + _CHUNK - 1) // _CHUNK
    children = seed_seq.spawn(nchunks)

    def work(c: int) -> None:
        rng = np.random.Generator(np.random.PCG64(children[c]))
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        if dist == "normal":
            x = rng.standard_normal(hi - lo, dtype=np.float32)
        elif dist == "uniform":
            x = rng.uniform(-1.0, 1.0, hi - lo).astype(np.float32)
        else:
            raise ValueError(dist)
        if fp8_scales is None:
            flat[lo:hi] = torch.from_numpy(x).to(out.dtype)
        else:
            head = (np.arange(lo, hi, dtype=np.int64) // row_elems) % len(fp8_scales)
            y = torch.from_numpy(x / fp8_scales[head])
            flat[lo:hi] = y.to(torch.float8_e4m3fn).view(torch.uint8)

    if nchunks == 1:
        work(0)
        return
    # one torch thread per worker: the conversions run inside the pool's
    # threads, and torch's own intra-op threads on top of them oversubscribe
    # the cores many times over
    prev = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(work, range(nchunks)))
    finally:
        torch.set_num_threads(prev)


def _small_draw(rng: np.random.Generator, shape, dtype, dist: str) -> torch.Tensor:
    size = int(np.prod(shape))
    if dist == "normal":
        x = rng.standard_normal(size, dtype=np.float32)
    else:
        x = rng.uniform(-1.0, 1.0, size).astype(np.float32)
    return torch.from_numpy(x).to(dtype).reshape(shape)


FP8_NAN = 0x7F


def _pool(num_blocks, num_kv_heads, block_size, head_dim, dtype, seed_seq, dist,
          used_blocks, fp8_scales=None) -> torch.Tensor:
    pool_dtype = torch.uint8 if fp8_scales is not None else dtype
    pool = torch.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=pool_dtype)
    _draw_into(pool, seed_seq, dist, fp8_scales, block_size * head_dim)
    unused = np.ones(num_blocks, dtype=bool)
    unused[np.asarray(used_blocks, dtype=np.int64)] = False
    idx = torch.from_numpy(np.nonzero(unused)[0])
    if idx.numel():
        pool[idx] = FP8_NAN if fp8_scales is not None else float("nan")
    return pool


def shared_tokens(w: Workload, group_size: int) -> np.ndarray:
    """int32 [B // group_size]: per group of group_size consecutive
    sequences, block_size times the number of leading logical blocks all of
    them map to the same physical block (read off the tables)."""
    out = np.zeros(w.num_seqs // group_size, dtype=np.int32)
    bs = w.block_size
    for k in range(len(out)):
        rows = range(k * group_size, (k + 1) * group_size)
        blocks = min(-(-int(w.seq_lens[i]) // bs) for i in rows)
        b = 0
        while b < blocks and len({int(w.block_tables[i, b]) for i in rows}) == 1:
            b += 1
        out[k] = b * bs
    return out


def fp8_head_scales(num_kv_heads: int, spread: float) -> np.ndarray:
    """Per-head scales for FP8 pools: head g gets (1 + g / Hkv) * spread / 448,
    so N(0, 1) values of magnitude up to `spread` stay within the format."""
    g = np.arange(num_kv_heads, dtype=np.float64)
    return ((1.0 + g / num_kv_heads) * spread / 448.0).astype(np.float32)


def _blocks_needed(n_tokens: int, block_size: int) -> int:
    return -(-int(n_tokens) // block_size)


# ----------------------------------------------------------------------------
# generic builder: independent sequences, each with its own blocks

def build_independent(name, seq_lens, *, dtype, num_heads, num_kv_heads, head_dim,
                      block_size, dist, seed, pool_factor=1.25, num_blocks=None,
                      scale=None, fp8_spread=None) -> Workload:
    """Sequences that share no blocks; the table rows are consecutive slices of
    a seeded permutation of the pool ids. With fp8_spread, the pools hold
    FP8 E4M3 codes under fp8_head_scales(num_kv_heads, fp8_spread); q and the
    new tokens keep `dtype`."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    ss_tables, ss_k, ss_v, ss_small = np.random.SeedSequence(seed).spawn(4)
    rng_tables = np.random.default_rng(ss_tables)
    nb = [_blocks_needed(n, block_size) for n in seq_lens]
    needed = int(sum(nb))
    if num_blocks is None:
        num_blocks = max(1, math.ceil(pool_factor * needed))
    if num_blocks < needed:
        raise ValueError(f"pool of {num_blocks} blocks < {needed} needed")
    perm = rng_tables.permutation(num_blocks).astype(np.int32)
    max_blocks = max(1, max(nb) if nb else 1)
    tables = np.full((len(seq_lens), max_blocks), -1, dtype=np.int32)
    cursor = 0
    for i, n in enumerate(nb):
        tables[i, :n] = perm[cursor:cursor + n]
        cursor += n
    used = perm[:needed]
    sc = fp8_head_scales(num_kv_heads, fp8_spread) if fp8_spread is not None else None
    k_pool = _pool(num_blocks, num_kv_heads, block_size, head_dim, dtype, ss_k, dist, used, sc)
    v_pool = _pool(num_blocks, num_kv_heads, block_size, head_dim, dtype, ss_v, dist, used, sc)
    rng = np.random.default_rng(ss_small)
    b = len(seq_lens)
    k_new = _small_draw(rng, (b, num_kv_heads, head_dim), dtype, dist)
    v_new = _small_draw(rng, (b, num_kv_heads, head_dim), dtype, dist)
    q = _small_draw(rng, (b, num_heads, head_dim), dtype, dist)
    return Workload(name=name, dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, block_size=block_size,
                    scale=(1.0 / math.sqrt(head_dim)) if scale is None else scale,
                    num_blocks=num_blocks, seq_lens=seq_lens, block_tables=tables,
                    k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new, q=q,
                    k_scales=None if sc is None else torch.from_numpy(sc.copy()),
                    v_scales=None if sc is None else torch.from_numpy(sc.copy()))


# ----------------------------------------------------------------------------
# the five workloads

def tiny_fp32(seed=SEED_BASE + 1) -> Workload:
    """4 sequences of lengths 1, 16, 17, 37; 4 heads of 64; 16-token blocks;
    a 16-block pool; uniform[-1, 1] values; scale 1/8."""
    return build_independent("tiny_fp32", [1, 16, 17, 37], dtype=torch.float32,
                             num_heads=4, num_kv_heads=4, head_dim=64, block_size=16,
                             dist="uniform", seed=seed, num_blocks=16, scale=1.0 / 8.0)


def opt13b_fp16(seed=SEED_BASE + 2, num_seqs=64, len_range=(32, 2048),
                block_size=16) -> Workload:
    """OPT-13B attention layer: 40 heads of 128, fp16, batch 64, lengths
    uniform in [32, 2048], N(0, 1) values, pool 1.25x the blocks needed."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(1)[0])
    lens = rng.integers(len_range[0], len_range[1], size=num_seqs, endpoint=True)
    return build_independent("opt13b_fp16", lens, dtype=torch.float16, num_heads=40,
                             num_kv_heads=40, head_dim=128, block_size=block_size,
                             dist="normal", seed=seed + 100_000)


def opt13b_fp8(seed=SEED_BASE + 6, num_seqs=64, len_range=(32, 2048), block_size=16) -> Workload:
    """The OPT-13B layer with an FP8 E4M3 KV cache: the same shape and length
    draw as opt13b_fp16, K/V stored as codes under per-head scales
    (magnitudes up to 8 representable), q and new tokens in fp16."""
    rng = np.random.default_rng(np.random.SeedSequence(SEED_BASE + 2).spawn(1)[0])
    lens = rng.integers(len_range[0], len_range[1], size=num_seqs, endpoint=True)
    return build_independent("opt13b_fp8", lens, dtype=torch.float16, num_heads=40,
                             num_kv_heads=40, head_dim=128, block_size=block_size,
                             dist="normal", seed=seed + 100_000, fp8_spread=8.0)


def long_gqa_fp8(seed=SEED_BASE + 7, block_size=16, num_seqs=16,
                 len_range=(16384, 32768)) -> Workload:
    """The long-context grouped-query layer (64 query heads over 8 kv heads)
    with an FP8 E4M3 KV cache; q and new tokens in bf16."""
    rng = np.random.default_rng(np.random.SeedSequence(SEED_BASE + 5).spawn(1)[0])
    lens = rng.integers(len_range[0], len_range[1], size=num_seqs, endpoint=True)
    return build_independent(f"long_gqa_fp8_bs{block_size}", lens, dtype=torch.bfloat16,
                             num_heads=64, num_kv_heads=8, head_dim=128, block_size=block_size,
                             dist="normal", seed=seed + 1000 * block_size, fp8_spread=8.0)


def opt13b_spec4_fp16(seed=SEED_BASE + 8, num_seqs=64, len_range=(32, 2048), nq=4,
                      block_size=16) -> Workload:
    """Speculative verification on the OPT-13B layer: each sequence checks
    nq = 4 proposed tokens in one pass (the cached history as in opt13b_fp16,
    plus the 4 new tokens), causal among the new tokens."""
    rng = np.random.default_rng(np.random.SeedSequence(SEED_BASE + 2).spawn(1)[0])
    lens = rng.integers(len_range[0], len_range[1], size=num_seqs, endpoint=True) + nq - 1
    w = build_independent("opt13b_spec4_fp16", lens, dtype=torch.float16, num_heads=40,
                          num_kv_heads=40, head_dim=128, block_size=block_size, dist="normal",
                          seed=seed + 100_000)
    r = np.random.default_rng(np.random.SeedSequence(seed).spawn(2)[1])
    b = w.num_seqs
    w.k_new = _small_draw(r, (b, nq, 40, 128), torch.float16, "normal")
    w.v_new = _small_draw(r, (b, nq, 40, 128), torch.float16, "normal")
    w.q = _small_draw(r, (b, nq, 40, 128), torch.float16, "normal")
    w.num_queries = nq
    return w


def opt13b_prefill256_fp16(seed=SEED_BASE + 11, num_seqs=8, cached_range=(1024, 2048),
                           chunk=256, block_size=16) -> Workload:
    """Chunked prefill on the OPT-13B layer (blog.aqudi.me section 4: a long
    prompt fed in pieces between decode steps): 8 sequences each feed a
    256-token chunk of prompt after 1024..2048 cached tokens; the chunk's
    tokens attend causally to the cache and to each other."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(1)[0])
    lens = rng.integers(cached_range[0], cached_range[1], size=num_seqs, endpoint=True) + chunk
    w = build_independent("opt13b_prefill256_fp16", lens, dtype=torch.float16, num_heads=40,
                          num_kv_heads=40, head_dim=128, block_size=block_size, dist="normal",
                          seed=seed + 100_000)
    r = np.random.default_rng(np.random.SeedSequence(seed).spawn(2)[1])
    b = w.num_seqs
    w.k_new = _small_draw(r, (b, chunk, 40, 128), torch.float16, "normal")
    w.v_new = _small_draw(r, (b, chunk, 40, 128), torch.float16, "normal")
    w.q = _small_draw(r, (b, chunk, 40, 128), torch.float16, "normal")
    w.num_queries = chunk
    return w


def opt13b_spec4_fp8(seed=SEED_BASE + 9, num_seqs=64, len_range=(32, 2048), nq=4,
                     block_size=16) -> Workload:
    """Speculative verification of 4 proposed tokens on the OPT-13B layer over
    an FP8 E4M3 KV cache (per-head scales as opt13b_fp8); q and the new tokens
    in fp16. Same lengths as opt13b_spec4_fp16."""
    rng = np.random.default_rng(np.random.SeedSequence(SEED_BASE + 2).spawn(1)[0])
    lens = rng.integers(len_range[0], len_range[1], size=num_seqs, endpoint=True) + nq - 1
    w = build_independent("opt13b_spec4_fp8", lens, dtype=torch.float16, num_heads=40,
                          num_kv_heads=40, head_dim=128, block_size=block_size, dist="normal",
                          seed=seed + 100_000, fp8_spread=8.0)
    r = np.random.default_rng(np.random.SeedSequence(seed).spawn(2)[1])
    b = w.num_seqs
    w.k_new = _small_draw(r, (b, nq, 40, 128), torch.float16, "normal")
    w.v_new = _small_draw(r, (b, nq, 40, 128), torch.float16, "normal")
    w.q = _small_draw(r, (b, nq, 40, 128), torch.float16, "normal")
    w.num_queries = nq
    return w


def llama13b_bf16(seed=SEED_BASE + 3, num_seqs=256, median=350.0, sigma=0.9,
                  max_len=4096, block_size=16) -> Workload:
    """LLaMA-13B attention layer: 40 heads of 128, bf16, batch 256, chat-like
    lengths rint(lognormal(ln 350, 0.9)) clipped to [1, 4096]."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(1)[0])
    lens = np.clip(np.rint(rng.lognormal(math.log(median), sigma, size=num_seqs)), 1, max_len)
    return build_independent("llama13b_bf16", lens.astype(np.int32), dtype=torch.bfloat16,
                             num_heads=40, num_kv_heads=40, head_dim=128,
                             block_size=block_size, dist="normal", seed=seed + 100_000)


def long_gqa_bf16(seed=SEED_BASE + 5, block_size=16, num_seqs=16,
                  len_range=(16384, 32768)) -> Workload:
    """Long-context grouped-query attention: 64 query heads over 8 KV heads
    of 128, bf16, batch 16, lengths uniform in [16384, 32768]. The lengths do
    not depend on block_size, so the block-size sweep reads the same history
    layout-for-layout."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(1)[0])
    lens = rng.integers(len_range[0], len_range[1], size=num_seqs, endpoint=True)
    return build_independent(f"long_gqa_bf16_bs{block_size}", lens, dtype=torch.bfloat16,
                             num_heads=64, num_kv_heads=8, head_dim=128,
                             block_size=block_size, dist="normal",
                             seed=seed + 1000 * block_size)


def shared_prefix_fp16(seed=SEED_BASE + 4, prefix_len=1024, num_prompts=32,
                       samples=8, max_divergent=256, block_size=16,
                       num_heads=40, head_dim=128, fp8_spread=None) -> Workload:
    """Parallel sampling: each prompt's prefix blocks are named by the tables
    of all its samples; each sample adds 0..max_divergent tokens of its own
    plus the token appended this step.

    When the prefix ends inside a block, that block is shared too, and every
    sample but the last must get a private copy before writing into it. The
    returned copy_pairs (shared block, fresh block) are those copies; the
    samples' own tokens that fall inside that block are returned as pending
    appends (to be stored after the copies, one step at a time). History
    tokens past that block are drawn directly into private blocks.

    With fp8_spread the pools hold FP8 E4M3 codes under
    fp8_head_scales(num_heads, fp8_spread) (q and new tokens stay fp16).
    """
    dtype = torch.float16
    ss_len, ss_tables, ss_k, ss_v, ss_small = np.random.SeedSequence(seed).spawn(5)
    rng_len = np.random.default_rng(ss_len)
    divergent = rng_len.integers(0, max_divergent, size=num_prompts * samples, endpoint=True)
    seq_lens = (prefix_len + divergent + 1).astype(np.int32)
    full_prefix_blocks = prefix_len // block_size
    partial = prefix_len % block_size != 0
    prefix_blocks = full_prefix_blocks + (1 if partial else 0)

    # private blocks per sample: the logical blocks past the prefix's blocks,
    # plus (partial prefix, all samples but the last) the copy of the shared one
    per_sample_private = []
    for i in range(num_prompts * samples):
        n = _blocks_needed(seq_lens[i], block_size) - prefix_blocks
        if partial and (i % samples) != samples - 1:
            n += 1
        per_sample_private.append(n)
    needed = num_prompts * prefix_blocks + sum(per_sample_private)
    num_blocks = math.ceil(1.25 * needed)
    perm = np.random.default_rng(ss_tables).permutation(num_blocks).astype(np.int32)
    max_blocks = max(_blocks_needed(n, block_size) for n in seq_lens)
    tables = np.full((num_prompts * samples, max_blocks), -1, dtype=np.int32)
    pairs = []
    cursor = 0
    for p in range(num_prompts):
        shared = perm[cursor:cursor + prefix_blocks]
        cursor += prefix_blocks
        for s in range(samples):
            i = p * samples + s
            nb = _blocks_needed(seq_lens[i], block_size)
            tables[i, :prefix_blocks] = shared
            own = perm[cursor:cursor + per_sample_private[i]]
            cursor += per_sample_private[i]
            if partial and s != samples - 1:
                tables[i, full_prefix_blocks] = own[0]
                pairs.append((int(shared[-1]), int(own[0])))
                own = own[1:]
            tables[i, prefix_blocks:nb] = own
    assert cursor == needed
    used = perm[:needed]
    sc = fp8_head_scales(num_heads, fp8_spread) if fp8_spread is not None else None
    k_pool = _pool(num_blocks, num_heads, block_size, head_dim, dtype, ss_k, "normal", used, sc)
    v_pool = _pool(num_blocks, num_heads, block_size, head_dim, dtype, ss_v, "normal", used, sc)

    rng = np.random.default_rng(ss_small)
    b = num_prompts * samples
    pending_k = pending_v = pending_lens = None
    if partial:
        # the sample's history tokens that land in the copied block
        room = block_size - prefix_len % block_size
        steps = int(min(room, int(divergent.max()) if b else 0))
        pending_lens = np.zeros((steps, b), dtype=np.int32)
        for t in range(steps):
            pending_lens[t] = np.where(divergent > t, prefix_len + t + 1, 0)
        pending_k = _small_draw(rng, (steps, b, num_heads, head_dim), dtype, "normal")
        pending_v = _small_draw(rng, (steps, b, num_heads, head_dim), dtype, "normal")
    k_new = _small_draw(rng, (b, num_heads, head_dim), dtype, "normal")
    v_new = _small_draw(rng, (b, num_heads, head_dim), dtype, "normal")
    q = _small_draw(rng, (b, num_heads, head_dim), dtype, "normal")
    name = ("shared_prefix_cow" if partial else "shared_prefix") + ("_fp8" if sc is not None
                                                                   else "_fp16")
    return Workload(name=name, dtype=dtype, num_heads=num_heads, num_kv_heads=num_heads,
                    head_dim=head_dim, block_size=block_size, scale=1.0 / math.sqrt(head_dim),
                    num_blocks=num_blocks, seq_lens=seq_lens, block_tables=tables,
                    k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new, q=q,
                    copy_pairs=np.asarray(pairs, dtype=np.int32).reshape(-1, 2),
                    pending_k=pending_k, pending_v=pending_v, pending_lens=pending_lens,
                    info={"prefix_len": prefix_len, "num_prompts": num_prompts,
                          "samples": samples, "unique_blocks": needed},
                    shared_blocks=True,
                    k_scales=None if sc is None else torch.from_numpy(sc.copy()),
                    v_scales=None if sc is None else torch.from_numpy(sc.copy()))


def shared_prefix_cow_fp16(seed=SEED_BASE + 4, **kw) -> Workload:
    """The shared-prefix workload with a 1032-token prefix: 64 full shared
    blocks plus a shared partial block that 7 of 8 samples copy."""
    kw.setdefault("prefix_len", 1032)
    return shared_prefix_fp16(seed=seed, **kw)


def shared_prefix_fp8(seed=SEED_BASE + 10, **kw) -> Workload:
    """The 32 x 8 parallel-sampling layer over an FP8 E4M3 KV cache."""
    kw.setdefault("fp8_spread", 8.0)
    return shared_prefix_fp16(seed=seed, **kw)


def shared_prefix_cow_fp8(seed=SEED_BASE + 10, **kw) -> Workload:
    """The copy-on-write variant (1032-token prefix) over an FP8 KV cache."""
    kw.setdefault("prefix_len", 1032)
    kw.setdefault("fp8_spread", 8.0)
    return shared_prefix_fp16(seed=seed, **kw)


WORKLOADS = {
    "tiny_fp32": tiny_fp32,
    "opt13b_fp16": opt13b_fp16,
    "llama13b_bf16": llama13b_bf16,
    "shared_prefix_fp16": shared_prefix_fp16,
    "shared_prefix_cow_fp16": shared_prefix_cow_fp16,
    "long_gqa_bf16": long_gqa_bf16,
    "opt13b_fp8": opt13b_fp8,
    "opt13b_spec4_fp16": opt13b_spec4_fp16,
    "long_gqa_fp8": long_gqa_fp8,
    "opt13b_spec4_fp8": opt13b_spec4_fp8,
    "opt13b_prefill256_fp16": opt13b_prefill256_fp16,
    "shared_prefix_fp8": shared_prefix_fp8,
    "shared_prefix_cow_fp8": shared_prefix_cow_fp8,
}


def make(name: str, **kw) -> Workload:
    return WORKLOADS[name](**kw)
