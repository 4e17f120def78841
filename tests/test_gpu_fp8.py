"""GPU parity of the FP8 (OCP E4M3) KV cache against the oracle.

The append's codes are compared bit for bit with the oracle's quantiser (the
same float32 division, nearest-even rounding and saturation); attention is
compared with the float64 oracle run on the dequantised pools, within the
16-bit tolerance (2e-3 max-abs): both sides read the same values, only the
arithmetic differs.
"""

import sys

import numpy as np
import pytest
import torch

from oracle import fp8_decode
from paged_kv_cache_440_amd import PARTITION_BALANCED as BAL
from paged_kv_cache_440_amd import workloads as wl
from tests.gpu_support import (Device, bits, check_error, expected_attention, expected_pools,
                               max_err,
                               poison_unwritten_slots, tol)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    sys.__stderr__.write(f"\n[gpu] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
    torch.cuda.synchronize()


def fp8_workload(lens, q_dtype, group, block_size=16, hkv=2, seed=31, poison=True):
    w = wl.build_independent("fp8", lens, dtype=q_dtype, num_heads=hkv * group,
                             num_kv_heads=hkv, head_dim=128, block_size=block_size,
                             dist="normal", seed=seed, fp8_spread=8.0)
    if poison:
        poison_unwritten_slots(w)
    return w


RAGGED = [1, 2, 3, 31, 32, 33, 63, 100, 129, 700, 1000]


@pytest.mark.parametrize("q_dtype", [torch.float16, torch.bfloat16, torch.float32])
def test_append_codes_bit_exact(q_dtype):
    """New tokens of every input type, with values that exercise saturation,
    signed zero, subnormals and exact ties (the scale of head 0 is 2^-6, so
    x / scale is exact there)."""
    w = fp8_workload(RAGGED, q_dtype, 1)
    w.k_scales[0] = 2.0 ** -6
    w.v_scales[0] = 2.0 ** -6
    special = torch.tensor([1e4, -1e4, 0.0, -0.0, 2.0 ** -16, 3 * 2.0 ** -16, 7.0,
                            (4.5 * 2 ** -6), (5.5 * 2 ** -6), 2.0 ** -15, 100.0, -3.3],
                           dtype=torch.float32).to(q_dtype)
    w.k_new[: len(special) // 2, 0, :2] = special.view(-1, 2)
    w.v_new[0, 0, : len(special)] = special
    d = Device(w)
    d.copy_and_append()
    kb, vb = expected_pools(w)
    assert np.array_equal(bits(d.k_pool), kb)
    assert np.array_equal(bits(d.v_pool), vb)


@pytest.mark.parametrize("partition", [0, 64, 512, BAL])
@pytest.mark.parametrize("q_dtype,group,block_size", [
    (torch.float16, 1, 16),          # vector walker
    (torch.bfloat16, 1, 8),
    (torch.float32, 1, 64),
    (torch.bfloat16, 2, 16),         # matrix-core walker
    (torch.float16, 4, 32),
    (torch.bfloat16, 8, 128),
])
def test_attention_matches_oracle(q_dtype, group, block_size, partition):
    w = fp8_workload(RAGGED, q_dtype, group, block_size)
    d = Device(w)
    d.copy_and_append()
    out = d.attention(partition_size=partition)
    assert torch.isfinite(out).all()
    ref = expected_attention(w, *expected_pools(w))
    assert max_err(out, ref) <= tol(w), f"max abs error {max_err(out, ref):.3e}"


@pytest.mark.parametrize("group", [1, 8])
def test_every_finite_code_decodes_exactly(group):
    """Length-1 sequences return their value row: with V rows holding every
    finite code, the output is value(code) * v_scale (power-of-two scale, so
    exact)."""
    finite = np.nonzero(np.isfinite(fp8_decode(np.arange(256))))[0].astype(np.uint8)
    rows = np.resize(finite, (2, 128))
    w = fp8_workload([1, 1], torch.float16, group, hkv=1, poison=False)
    w.v_scales[:] = 2.0 ** -4
    d = Device(w)
    tables = w.block_tables
    for i in range(2):
        d.v_pool[int(tables[i, 0]), 0, 0] = torch.from_numpy(rows[i]).to(d.v_pool.device)
    out = d.attention(partition_size=0).cpu().double().numpy()
    for i in range(2):
        want = fp8_decode(rows[i]) * 2.0 ** -4
        for h in range(group):
            assert np.array_equal(out[i, h], want)


def test_copy_blocks_moves_fp8_blocks():
    w = fp8_workload(RAGGED, torch.float16, 1)
    d = Device(w)
    pairs = torch.tensor([[int(w.block_tables[9, 0]), int(w.block_tables[0, 0])],
                          [int(w.block_tables[10, 3]), 0]], dtype=torch.int32, device="cuda")
    import paged_kv_cache_440_amd as pkv
    from oracle import pool_after_copy
    pkv.copy_blocks(d.k_pool, d.v_pool, pairs)
    kb, vb = pool_after_copy(bits(w.k_pool), bits(w.v_pool), pairs.cpu().numpy())
    assert np.array_equal(bits(d.k_pool), kb) and np.array_equal(bits(d.v_pool), vb)


@pytest.mark.parametrize("group", [1, 8])
def test_block_relabelling_is_bit_exact(group):
    w = fp8_workload(RAGGED, torch.bfloat16, group)
    d = Device(w)
    d.copy_and_append()
    ref = d.attention(partition_size=BAL).cpu()
    perm = np.random.default_rng(5).permutation(w.num_blocks)
    inv = np.argsort(perm)
    w2 = fp8_workload(RAGGED, torch.bfloat16, group)
    w2.k_pool = w2.k_pool[torch.from_numpy(perm)].contiguous()
    w2.v_pool = w2.v_pool[torch.from_numpy(perm)].contiguous()
    w2.block_tables = np.where(w2.block_tables >= 0, inv[np.maximum(w2.block_tables, 0)],
                               -1).astype(np.int32)
    d2 = Device(w2)
    d2.copy_and_append()
    assert torch.equal(d2.attention(partition_size=BAL).cpu(), ref)


FULL = {
    "opt13b_fp8": lambda: wl.opt13b_fp8(),
    "long_gqa_fp8_bs16": lambda: wl.long_gqa_fp8(block_size=16),
}


@pytest.mark.parametrize("partition", [512, BAL])
@pytest.mark.parametrize("name", list(FULL))
def test_full_size_matches_oracle(name, partition):
    """Full-size FP8 workloads under both schedules the bench uses (512-token
    partitions for the OPT-13B layer, balanced for the long GQA layer)."""
    w = FULL[name]()
    d = Device(w)
    d.copy_and_append()
    out = d.attention(partition_size=partition)
    kb, vb = expected_pools(w)
    assert np.array_equal(bits(d.k_pool), kb) and np.array_equal(bits(d.v_pool), vb)
    del d
    err = max_err(out, expected_attention(w, kb, vb))
    path = "fp8_mfma" if w.num_heads > w.num_kv_heads else "fp8_vector"
    check_error(path, err, tol(w), f"{name} partition {partition}")


@pytest.mark.parametrize("group", [1, 8])
def test_kv_policies_give_identical_bits(group):
    w = fp8_workload(RAGGED, torch.bfloat16, group)
    d = Device(w)
    d.copy_and_append()
    for partition in (512, BAL):
        a = d.attention(partition_size=partition, kv_reuse=False).cpu()
        b = d.attention(partition_size=partition, kv_reuse=True).cpu()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
