"""pkv_paged_attention_decode_noalloc (the split-K records in the library's
static per-device scratch, nothing allocated) against
pkv_paged_attention_decode with a caller workspace: the same bits, on two
calls in a row with the second smaller than the first, for each schedule and
both walkers. Calls go through the C ABI (ctypes) directly."""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_440_amd as pkv
from paged_kv_cache_440_amd import workloads as wl
from paged_kv_cache_440_amd._lib import DTYPE_CODES, PARTITION_BALANCED as BAL

from .gpu_support import Device, bits

pytestmark = pytest.mark.gpu


def noalloc(d, partition, out):
    """One call of pkv_paged_attention_decode_noalloc through ctypes."""
    w = d.w
    lib = pkv.library()
    nb, hkv, bs, hd = d.k_pool.shape
    st = lib.pkv_paged_attention_decode_noalloc(
        out.data_ptr(), DTYPE_CODES[out.dtype], d.q.data_ptr(), d.k_pool.data_ptr(),
        d.v_pool.data_ptr(), d.tables.data_ptr(), d.tables.shape[1], d.lens.data_ptr(),
        w.max_seq_len, w.num_seqs, w.num_heads, hkv, hd, bs, nb, ctypes.c_float(w.scale),
        partition, DTYPE_CODES[w.dtype], 0, torch.cuda.current_stream().cuda_stream)
    assert st == 0, pkv.status_string(st)


def with_workspace(d, partition):
    w = d.w
    out = torch.empty(tuple(w.q.shape), dtype=torch.float32, device="cuda")
    need = pkv.paged_attention_workspace_size(w.num_seqs, w.num_heads, w.num_kv_heads,
                                              w.head_dim, w.max_seq_len, partition)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    pkv.paged_attention_decode(out, d.q, d.k_pool, d.v_pool, d.tables, d.lens, w.max_seq_len,
                               w.scale, partition_size=partition, workspace=ws)
    return out


PAIRS = {
    # (first call, second call with a smaller input)
    "opt13b_fp16": (lambda: wl.opt13b_fp16(num_seqs=24, len_range=(32, 2048)),
                    lambda: wl.opt13b_fp16(seed=9, num_seqs=5, len_range=(32, 700))),
    "long_gqa_bf16": (lambda: wl.long_gqa_bf16(num_seqs=4, len_range=(3000, 9000)),
                      lambda: wl.long_gqa_bf16(seed=9, num_seqs=2, len_range=(600, 2000))),
}


@pytest.mark.parametrize("partition", [512, BAL])
@pytest.mark.parametrize("name", sorted(PAIRS))
def test_noalloc_matches_the_workspace_call_twice(name, partition):
    for make in PAIRS[name]:
        w = make()
        print(f"[noalloc] {name} B={w.num_seqs} max_len={w.max_seq_len} partition={partition}",
              flush=True)
        d = Device(w)
        d.copy_and_append()
        ref = with_workspace(d, partition)
        out = torch.full(tuple(w.q.shape), float("nan"), dtype=torch.float32, device="cuda")
        noalloc(d, partition, out)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any()
        assert np.array_equal(bits(out), bits(ref)), name


def test_noalloc_refuses_calls_beyond_its_scratch():
    """Fixed 64-token partitions of 256 long sequences need more records than
    the static scratch holds: refused before anything is enqueued."""
    need = pkv.paged_attention_workspace_size(256, 40, 40, 128, 4096, 64)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    lib = pkv.library()
    x = torch.empty(16, dtype=torch.uint8, device="cuda")
    st = lib.pkv_paged_attention_decode_noalloc(
        x.data_ptr(), 0, x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(), 256,
        x.data_ptr(), 4096, 256, 40, 40, 128, 16, 1000, ctypes.c_float(0.1), 64, 1, 0,
        torch.cuda.current_stream().cuda_stream)
    assert st == -6 and "static" in pkv.status_string(st)
