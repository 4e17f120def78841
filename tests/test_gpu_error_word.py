"""The error word (pkv_set_error_word): a block-table entry outside the pool,
a length above max_seq_len, an append target outside the pool and a copy
pair outside it each set their bit, while every access stays inside the
buffers (the kernels clamp or skip; nothing faults) and rows that do not
touch the bad value keep the bits of the clean call. Clean calls leave the
word at zero. The pages name the table lookup as the paged kernel's extra
step (supersilo.blog summary, "PagedAttention의 설계", "커널 비용과 블록 크기")."""

import numpy as np
import pytest
import torch

import paged_kv_cache_440_amd as pkv
from paged_kv_cache_440_amd import workloads as wl
from paged_kv_cache_440_amd._lib import PARTITION_BALANCED as BAL

from .gpu_support import Device, bits

pytestmark = pytest.mark.gpu


@pytest.fixture
def word():
    w = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.set_error_word(w)
    yield w
    torch.cuda.synchronize()
    pkv.set_error_word(None)


def read(word):
    torch.cuda.synchronize()
    v = int(word.item())
    word.zero_()
    torch.cuda.synchronize()
    return v


def attend(d, tables, lens, partition):
    w = d.w
    out = torch.empty(tuple(w.q.shape), dtype=torch.float32, device="cuda")
    if w.fp8:
        pkv.paged_attention_decode_fp8(out, d.q, d.k_pool, d.v_pool, d.k_scales, d.v_scales,
                                       tables, lens, w.max_seq_len, w.scale,
                                       partition_size=partition)
    else:
        pkv.paged_attention_decode(out, d.q, d.k_pool, d.v_pool, tables, lens, w.max_seq_len,
                                   w.scale, partition_size=partition)
    return out


CASES = {
    "vector_fp16": lambda: wl.opt13b_fp16(num_seqs=6, len_range=(40, 900)),
    "mfma_bf16_g8": lambda: wl.long_gqa_bf16(num_seqs=3, len_range=(700, 2000)),
    "fp8_vector": lambda: wl.opt13b_fp8(num_seqs=6, len_range=(40, 900)),
    "fp8_mfma_g8": lambda: wl.long_gqa_fp8(num_seqs=3, len_range=(700, 2000)),
}


@pytest.mark.parametrize("partition", [0, 64, BAL])
@pytest.mark.parametrize("case", sorted(CASES))
def test_bad_table_entry_is_reported_and_clamped(case, partition, word):
    w = CASES[case]()
    d = Device(w)
    d.copy_and_append()
    assert read(word) == 0                       # the clean append reports nothing
    clean = attend(d, d.tables, d.lens, partition)
    assert read(word) == 0
    for bad in (w.num_blocks + 5, -3):
        tables = d.tables.clone()
        tables[0, 1] = bad                       # logical block 1 of sequence 0 is valid
        out = attend(d, tables, d.lens, partition)
        assert read(word) == pkv.ERRBIT_TABLE, (case, partition, bad)
        # the other rows are the clean call's bits
        assert np.array_equal(bits(out[1:]), bits(clean[1:]))


@pytest.mark.parametrize("partition", [0, 512, BAL])
def test_length_above_max_is_reported_and_clamped(partition, word):
    w = wl.opt13b_fp16(num_seqs=5, len_range=(40, 900))
    d = Device(w)
    d.copy_and_append()
    clean = attend(d, d.tables, d.lens, partition)
    assert read(word) == 0
    lens = d.lens.clone()
    lens[2] = w.max_seq_len + 100                # clamped to max_seq_len
    out = attend(d, d.tables, lens, partition)
    assert read(word) == pkv.ERRBIT_LENGTH
    others = [i for i in range(w.num_seqs) if i != 2]
    assert np.array_equal(bits(out[others]), bits(clean[others]))
    lens[2] = -4                                 # clamped to 0: a zero row
    out = attend(d, d.tables, lens, partition)
    assert read(word) == pkv.ERRBIT_LENGTH
    assert not out[2].any()


def test_append_and_copy_targets_outside_the_pool(word):
    w = wl.opt13b_fp16(num_seqs=4, len_range=(40, 300))
    d = Device(w)
    before_k = bits(d.k_pool)
    tables = d.tables.clone()
    i = 1
    tables[i, (int(w.seq_lens[i]) - 1) // w.block_size] = w.num_blocks   # the append's target
    pkv.kv_cache_append(d.k_new, d.v_new, d.k_pool, d.v_pool, tables, d.lens)
    assert read(word) == pkv.ERRBIT_APPEND
    after_k = bits(d.k_pool)
    # the bad row wrote nothing; the others did (their slots changed)
    changed = np.argwhere((after_k != before_k).any(axis=(1, 3)))
    good = {(int(w.block_tables[s, (int(w.seq_lens[s]) - 1) // w.block_size]),
             (int(w.seq_lens[s]) - 1) % w.block_size) for s in range(4) if s != i}
    assert {(int(b), int(s)) for b, s in changed} <= good
    # a token past max_blocks_per_seq * block_size
    lens = d.lens.clone()
    lens[0] = w.block_tables.shape[1] * w.block_size + 1
    pkv.kv_cache_append(d.k_new, d.v_new, d.k_pool, d.v_pool, d.tables, lens)
    assert read(word) == pkv.ERRBIT_APPEND
    # copy pairs naming a block outside the pool are skipped and reported
    pairs = torch.tensor([[0, w.num_blocks], [-1, 2]], dtype=torch.int32, device="cuda")
    snap = bits(d.k_pool)
    pkv.copy_blocks(d.k_pool, d.v_pool, pairs)
    assert read(word) == pkv.ERRBIT_COPY
    assert np.array_equal(bits(d.k_pool), snap)
    # and a clean step reports nothing
    pkv.copy_blocks(d.k_pool, d.v_pool, torch.tensor([[0, 1]], dtype=torch.int32, device="cuda"))
    pkv.kv_cache_append(d.k_new, d.v_new, d.k_pool, d.v_pool, d.tables, d.lens)
    assert read(word) == 0


def test_no_word_registered_reports_nowhere():
    """With the reports off a bad entry still gives the clamped result (the
    bits of the run with the word registered)."""
    w = wl.opt13b_fp16(num_seqs=3, len_range=(40, 400))
    d = Device(w)
    d.copy_and_append()
    tables = d.tables.clone()
    tables[0, 0] = w.num_blocks + 1
    pkv.set_error_word(None)
    a = attend(d, tables, d.lens, BAL)
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.set_error_word(word)
    try:
        b = attend(d, tables, d.lens, BAL)
        torch.cuda.synchronize()
        assert int(word.item()) == pkv.ERRBIT_TABLE
    finally:
        pkv.set_error_word(None)
    assert np.array_equal(bits(a), bits(b))
