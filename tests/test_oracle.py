"""Pins for the float64 oracle, against facts that do not come from the oracle.

Each pin is chosen so that a plausible mistake in the oracle fails at least
one of them (tests/test_oracle_mutants.py plants such mistakes and checks):
  * the worked block-table example of the Day 3 page, section 4.2 (golden file);
  * torch's CPU scaled_dot_product_attention in float64 on contiguous K/V,
    including its grouped-query mode (an independent library routine);
  * closed forms: one token returns V_0; equal scores return the mean of V;
    two tokens in one dimension give v0 + (v1 - v0) * sigmoid(s1 - s0); a
    huge score gap returns the arg-max value;
  * invariants of paging: relabelling physical blocks, a contiguous table,
    another block size, or aliased (shared) blocks leave the result identical;
  * 50-digit mpmath evaluation on tiny inputs;
  * block moves between two pools of different sizes (swapping) checked
    against blocks whose every element spells out its own block id.
"""

import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

from oracle import (block_and_slot, dense_decode_attention, gather_sequence,
                    paged_decode_attention, pool_after_append, pool_after_copy,
                    pool_after_swap)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers

def _random_paged(rng, seq_lens, num_heads, num_kv_heads, head_dim, block_size,
                  extra_blocks=3):
    """Independent random sequences laid into a shuffled pool (float64)."""
    nb = [-(-n // block_size) for n in seq_lens]
    num_blocks = sum(nb) + extra_blocks
    perm = rng.permutation(num_blocks)
    tables = np.full((len(seq_lens), max(nb + [1])), -1, dtype=np.int64)
    k_pool = np.full((num_blocks, num_kv_heads, block_size, head_dim), np.nan)
    v_pool = np.full_like(k_pool, np.nan)
    ks, vs = [], []
    c = 0
    for i, n in enumerate(seq_lens):
        tables[i, :nb[i]] = perm[c:c + nb[i]]
        c += nb[i]
        k = rng.standard_normal((n, num_kv_heads, head_dim))
        v = rng.standard_normal((n, num_kv_heads, head_dim))
        for t in range(n):  # lay the history out by hand (test-side layout)
            k_pool[tables[i, t // block_size], :, t % block_size] = k[t]
            v_pool[tables[i, t // block_size], :, t % block_size] = v[t]
        ks.append(k)
        vs.append(v)
    q = rng.standard_normal((len(seq_lens), num_heads, head_dim))
    return q, k_pool, v_pool, tables, ks, vs


def _sdpa(q, k, v, scale):
    """torch float64 SDPA for one decode query: q [H][D], k/v [L][Hkv][D]."""
    qt = torch.from_numpy(q)[None, :, None, :]                 # [1, H, 1, D]
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]  # [1, Hkv, L, D]
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    gqa = q.shape[0] != k.shape[1]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, scale=scale, enable_gqa=gqa)
    return o[0, :, 0, :].numpy()


# ------------------------------------------------------- worked example

def test_worked_example_gather():
    fx = json.load(open(os.path.join(GOLDEN, "worked_example_block_table.json")))
    bs, n, table = fx["block_size"], fx["seq_len"], fx["block_table"]
    nblk = 12
    # every slot carries a tag = physical_block * 1000 + slot
    pool = np.zeros((nblk, 1, bs, 1))
    for b in range(nblk):
        for s in range(bs):
            pool[b, 0, s, 0] = b * 1000 + s
    seq = gather_sequence(pool, table, n, bs)[:, 0, 0]
    phys = (seq // 1000).astype(int)
    slot = (seq % 1000).astype(int)
    counts = {str(b): int((phys == b).sum()) for b in set(phys.tolist())}
    assert counts == fx["tokens_held"]
    # logical order: the blocks are visited in table order, slots ascending
    order = [table.index(p) for p in phys]
    assert order == sorted(order)
    for b in table:
        assert list(slot[phys == b]) == list(range(fx["tokens_held"][str(b)]))
    # the last token sits in the partially used last block
    assert phys[-1] == table[-1] and slot[-1] == fx["tokens_held"][str(table[-1])] - 1
    assert block_and_slot(n - 1, bs) == (len(table) - 1, fx["tokens_held"][str(table[-1])] - 1)


def test_worked_example_append_goes_to_last_block_only():
    fx = json.load(open(os.path.join(GOLDEN, "worked_example_block_table.json")))
    bs, n, table = fx["block_size"], fx["seq_len"], fx["block_table"]
    k_pool = np.arange(12 * 2 * bs * 4, dtype=np.int32).reshape(12, 2, bs, 4)
    v_pool = -k_pool
    k_new = np.full((1, 2, 4), 7777, dtype=np.int32)
    v_new = np.full((1, 2, 4), -7777, dtype=np.int32)
    k2, v2 = pool_after_append(k_pool, v_pool, k_new, v_new, np.array([table]), [n], bs)
    changed = np.argwhere(k2 != k_pool)
    assert set(map(tuple, changed[:, :3].tolist())) == {(9, 0, 4), (9, 1, 4)}
    assert (k2[9, :, 4] == 7777).all() and (v2[9, :, 4] == -7777).all()
    assert int((v2 != v_pool).sum()) == 8


# ------------------------------------------------ library routine (SDPA)

@pytest.mark.parametrize("seed", range(6))
def test_matches_torch_sdpa_mha(seed):
    rng = np.random.default_rng(seed)
    lens = list(rng.integers(1, 90, size=3))
    d = [16, 64, 128][seed % 3]
    q, kp, vp, tables, ks, vs = _random_paged(rng, lens, 3, 3, d, 16)
    scale = 1.0 / math.sqrt(d)
    out = paged_decode_attention(q, kp, vp, tables, lens, 16, scale)
    for i in range(len(lens)):
        np.testing.assert_allclose(out[i], _sdpa(q[i], ks[i], vs[i], scale), rtol=0, atol=1e-12)


@pytest.mark.parametrize("group", [2, 4, 8])
def test_matches_torch_sdpa_gqa(group):
    rng = np.random.default_rng(100 + group)
    lens = [5, 33, 70]
    q, kp, vp, tables, ks, vs = _random_paged(rng, lens, 2 * group, 2, 32, 8)
    out = paged_decode_attention(q, kp, vp, tables, lens, 8, 0.3)
    for i in range(len(lens)):
        np.testing.assert_allclose(out[i], _sdpa(q[i], ks[i], vs[i], 0.3), rtol=0, atol=1e-12)


def test_per_block_normalisation_is_not_the_answer():
    """The summary page, PagedAttention design section: normalise once over all
    valid tokens, not per block. The oracle equals SDPA; a per-block normalised
    sum does not."""
    rng = np.random.default_rng(7)
    q, kp, vp, tables, ks, vs = _random_paged(rng, [40], 1, 1, 8, 16)
    out = paged_decode_attention(q, kp, vp, tables, [40], 16, 1.0)[0]
    ref = _sdpa(q[0], ks[0], vs[0], 1.0)
    per_block = sum(dense_decode_attention(q[0], ks[0][a:a + 16], vs[0][a:a + 16], 1.0)
                    for a in range(0, 40, 16))
    np.testing.assert_allclose(out, ref, atol=1e-12)
    assert np.abs(per_block - ref).max() > 0.1


# ---------------------------------------------------------- closed forms

def test_single_token_returns_v0_exactly():
    rng = np.random.default_rng(1)
    q, kp, vp, tables, ks, vs = _random_paged(rng, [1, 1], 4, 2, 64, 16)
    out = paged_decode_attention(q, kp, vp, tables, [1, 1], 16, 0.125)
    for i in range(2):
        for h in range(4):
            assert np.array_equal(out[i, h], vs[i][0, h // 2])


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    n, d = 37, 16
    k = np.repeat(rng.standard_normal((1, 1, d)), n, axis=0)
    v = rng.standard_normal((n, 1, d))
    out = dense_decode_attention(rng.standard_normal((1, d)), k, v, 0.7)
    np.testing.assert_allclose(out[0], v[:, 0].mean(axis=0), atol=1e-14)


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((20, 2, 8))
    v = rng.standard_normal((20, 2, 8))
    out = dense_decode_attention(np.zeros((4, 8)), k, v, 1.0)
    for h in range(4):
        np.testing.assert_allclose(out[h], v[:, h // 2].mean(axis=0), atol=1e-14)


def test_two_tokens_one_dim_is_a_sigmoid_blend():
    for q0, k0, k1, v0, v1, sc in [(0.3, 1.0, -2.0, 5.0, -1.0, 1.0),
                                   (-1.5, 0.2, 0.9, 0.0, 2.0, 0.5),
                                   (2.0, 3.0, 3.0, 1.0, 4.0, 1.0)]:
        out = dense_decode_attention(np.array([[q0]]), np.array([[[k0]], [[k1]]]),
                                     np.array([[[v0]], [[v1]]]), sc)
        s0, s1 = sc * q0 * k0, sc * q0 * k1
        expect = v0 + (v1 - v0) / (1.0 + math.exp(-(s1 - s0)))
        assert abs(out[0, 0] - expect) < 1e-14


def test_huge_score_gap_returns_argmax_value():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((50, 1, 8))
    v = rng.standard_normal((50, 1, 8))
    q = 1e3 * rng.standard_normal((1, 8))
    out = dense_decode_attention(q, k, v, 1.0)
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out[0], v[np.argmax(k[:, 0] @ q[0]), 0], atol=1e-12)


def test_affine_in_values():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((30, 1, 8))
    v = rng.standard_normal((30, 1, 8))
    q = rng.standard_normal((1, 8))
    base = dense_decode_attention(q, k, v, 0.4)
    np.testing.assert_allclose(dense_decode_attention(q, k, 3.0 * v - 2.0, 0.4),
                               3.0 * base - 2.0, atol=1e-13)


def test_padding_row_is_zero():
    rng = np.random.default_rng(6)
    q, kp, vp, tables, ks, vs = _random_paged(rng, [3, 0, 5], 2, 2, 8, 4)
    out = paged_decode_attention(q, kp, vp, tables, [3, 0, 5], 4, 1.0)
    assert np.array_equal(out[1], np.zeros((2, 8)))


# -------------------------------------------------------- 50-digit check

@pytest.mark.parametrize("seed", range(4))
def test_matches_mpmath_50_digits(seed):
    mpmath.mp.dps = 50
    rng = np.random.default_rng(1000 + seed)
    b, hkv, g = 3, 1 + seed % 2, 1 + seed % 3
    h, d, bs = hkv * g, 1 + seed % 4, 2
    lens = [int(x) for x in rng.integers(1, 6, size=b)]
    q, kp, vp, tables, ks, vs = _random_paged(rng, lens, h, hkv, d, bs)
    out = paged_decode_attention(q, kp, vp, tables, lens, bs, 0.9)
    for i in range(b):
        for head in range(h):
            kv = head // g
            s = [mpmath.mpf(0.9) * mpmath.fsum(mpmath.mpf(q[i, head, c]) * mpmath.mpf(ks[i][t, kv, c])
                                               for c in range(d)) for t in range(lens[i])]
            w = [mpmath.exp(x) for x in s]
            z = mpmath.fsum(w)
            for c in range(d):
                ref = mpmath.fsum(w[t] * mpmath.mpf(vs[i][t, kv, c]) for t in range(lens[i])) / z
                assert abs(float(ref) - out[i, head, c]) < 1e-12


# ------------------------------------------------------- paging invariants

def _relayout(k_pool, v_pool, tables, lens, new_bs, rng, num_blocks=None):
    """Lay the same logical histories into a fresh, shuffled pool (test-side)."""
    hkv, d = k_pool.shape[1], k_pool.shape[3]
    bs = k_pool.shape[2]
    nb = [-(-n // new_bs) for n in lens]
    total = num_blocks or sum(nb) + 2
    perm = rng.permutation(total)
    t2 = np.full((len(lens), max(nb + [1])), -1, dtype=np.int64)
    k2 = np.full((total, hkv, new_bs, d), np.nan)
    v2 = np.full_like(k2, np.nan)
    c = 0
    for i, n in enumerate(lens):
        t2[i, :nb[i]] = perm[c:c + nb[i]]
        c += nb[i]
        for t in range(n):
            src = (tables[i, t // bs], slice(None), t % bs)
            dst = (t2[i, t // new_bs], slice(None), t % new_bs)
            k2[dst] = k_pool[src]
            v2[dst] = v_pool[src]
    return k2, v2, t2


def test_block_relabelling_and_contiguous_tables_leave_output_identical():
    rng = np.random.default_rng(11)
    lens = [1, 16, 17, 37, 64]
    q, kp, vp, tables, ks, vs = _random_paged(rng, lens, 4, 4, 16, 16)
    ref = paged_decode_attention(q, kp, vp, tables, lens, 16, 0.25)
    # random relabelling of the physical blocks
    perm = rng.permutation(kp.shape[0])
    inv = np.argsort(perm)
    t_perm = np.where(tables >= 0, inv[np.maximum(tables, 0)], -1)
    out_p = paged_decode_attention(q, kp[perm], vp[perm], t_perm, lens, 16, 0.25)
    assert np.array_equal(out_p, ref)
    # one sequence, contiguous table 0, 1, 2, ... (the contiguous layout)
    for i, n in enumerate(lens):
        nb = -(-n // 16)
        kc = np.stack([kp[tables[i, j]] for j in range(nb)])
        vc = np.stack([vp[tables[i, j]] for j in range(nb)])
        out_c = paged_decode_attention(q[i:i + 1], kc, vc, np.arange(nb)[None], [n], 16, 0.25)
        assert np.array_equal(out_c[0], ref[i])
        assert np.array_equal(out_c[0], dense_decode_attention(q[i], ks[i], vs[i], 0.25))


@pytest.mark.parametrize("new_bs", [1, 8, 32, 64, 128])
def test_block_size_leaves_output_identical(new_bs):
    rng = np.random.default_rng(12)
    lens = [1, 15, 16, 17, 100, 129]
    q, kp, vp, tables, ks, vs = _random_paged(rng, lens, 2, 1, 8, 16)
    ref = paged_decode_attention(q, kp, vp, tables, lens, 16, 0.5)
    k2, v2, t2 = _relayout(kp, vp, tables, lens, new_bs, rng)
    assert np.array_equal(paged_decode_attention(q, k2, v2, t2, lens, new_bs, 0.5), ref)


def test_shared_blocks_equal_private_copies():
    """Summary page, block-sharing section: sharing is exact where the cached
    tokens are identical; aliasing a prefix equals giving each sample a copy."""
    rng = np.random.default_rng(13)
    bs, hkv, d, prefix = 4, 2, 8, 10
    samples = 3
    lens = [prefix + 1 + s for s in range(samples)]
    pre_blocks = -(-prefix // bs)
    n_full = prefix // bs
    # shared layout: blocks 0..pre_blocks-1 hold the prefix; the partial
    # prefix block is shared read-only only by the last sample, the others copy
    k = rng.standard_normal((60, hkv, bs, d))
    v = rng.standard_normal((60, hkv, bs, d))
    tables_shared = np.full((samples, 8), -1)
    tables_private = np.full((samples, 8), -1)
    nxt = pre_blocks
    kpriv, vpriv = k.copy(), v.copy()
    for s in range(samples):
        nb = -(-lens[s] // bs)
        tables_shared[s, :n_full] = np.arange(n_full)
        own = list(range(nxt, nxt + nb - n_full))
        nxt += nb - n_full
        tables_shared[s, n_full:nb] = own
        # the sample's own copy of the partial prefix block
        k[own[0], :, :prefix % bs] = k[n_full, :, :prefix % bs]
        v[own[0], :, :prefix % bs] = v[n_full, :, :prefix % bs]
    kpriv, vpriv = k.copy(), v.copy()
    for s in range(samples):
        nb = -(-lens[s] // bs)
        fresh = list(range(nxt, nxt + n_full))
        nxt += n_full
        for j, f in enumerate(fresh):
            kpriv[f] = kpriv[j]
            vpriv[f] = vpriv[j]
        tables_private[s, :n_full] = fresh
        tables_private[s, n_full:nb] = tables_shared[s, n_full:nb]
    q = rng.standard_normal((samples, 2 * hkv, d))
    a = paged_decode_attention(q, k, v, tables_shared, lens, bs, 0.3)
    b = paged_decode_attention(q, kpriv, vpriv, tables_private, lens, bs, 0.3)
    assert np.array_equal(a, b)


# ------------------------------------------------------- append and copy

def test_append_writes_exactly_the_new_slots():
    rng = np.random.default_rng(20)
    bs, hkv, d = 16, 3, 8
    lens = np.array([1, 16, 17, 37, 0])
    nb = [-(-n // bs) for n in lens]
    tables = np.full((5, 3), -1)
    perm = rng.permutation(12)
    c = 0
    for i in range(5):
        tables[i, :nb[i]] = perm[c:c + nb[i]]
        c += nb[i]
    k_pool = rng.integers(0, 2**16, size=(12, hkv, bs, d)).astype(np.uint16)
    v_pool = rng.integers(0, 2**16, size=(12, hkv, bs, d)).astype(np.uint16)
    k_new = rng.integers(0, 2**16, size=(5, hkv, d)).astype(np.uint16)
    v_new = rng.integers(0, 2**16, size=(5, hkv, d)).astype(np.uint16)
    k2, v2 = pool_after_append(k_pool, v_pool, k_new, v_new, tables, lens, bs)
    expect_slots = set()
    for i, n in enumerate(lens):
        if n == 0:
            continue
        blk, slot = tables[i, (n - 1) // bs], (n - 1) % bs
        expect_slots.add((int(blk), int(slot)))
        assert np.array_equal(k2[blk, :, slot], k_new[i])
        assert np.array_equal(v2[blk, :, slot], v_new[i])
        # and the gather sees the new token last
        assert np.array_equal(gather_sequence(k2, tables[i], n, bs)[-1], k_new[i])
    diff = np.argwhere((k2 != k_pool).any(axis=(1, 3)) | (v2 != v_pool).any(axis=(1, 3)))
    assert set(map(tuple, diff.tolist())) <= expect_slots


def test_copy_applies_pairs_in_order_and_touches_only_destinations():
    rng = np.random.default_rng(21)
    k = rng.integers(0, 1000, size=(8, 2, 4, 3))
    v = rng.integers(0, 1000, size=(8, 2, 4, 3))
    k2, v2 = pool_after_copy(k, v, [(1, 5), (5, 6), (2, 0)])
    assert np.array_equal(k2[5], k[1]) and np.array_equal(k2[6], k[1])
    assert np.array_equal(k2[0], k[2]) and np.array_equal(v2[6], v[1])
    for b in (1, 2, 3, 4, 7):
        assert np.array_equal(k2[b], k[b]) and np.array_equal(v2[b], v[b])
    k3, v3 = pool_after_copy(k, v, np.zeros((0, 2), dtype=np.int32))
    assert np.array_equal(k3, k) and np.array_equal(v3, v)


def _tagged_pool(num_blocks, hkv, bs, d, base):
    """int32 pool whose element [b][g][s][e] is base + 10000 b + 1000 g + 10 s + e
    (e < 10): every element names its block, head, slot and position."""
    b, g, s, e = np.meshgrid(np.arange(num_blocks), np.arange(hkv), np.arange(bs), np.arange(d),
                             indexing="ij")
    return (base + 10000 * b + 1000 * g + 10 * s + e).astype(np.int32)


def test_swap_moves_tagged_blocks_between_pools_of_different_sizes():
    # supersilo.blog summary, "적용 범위와 관련 연구": preempted sequences move to
    # CPU memory and back, i.e. whole blocks go from one pool to another
    hkv, bs, d = 3, 4, 6
    src_k, src_v = _tagged_pool(7, hkv, bs, d, 0), _tagged_pool(7, hkv, bs, d, -500000)
    dst_k, dst_v = _tagged_pool(11, hkv, bs, d, 900000), _tagged_pool(11, hkv, bs, d, 700000)
    saved = [x.copy() for x in (src_k, src_v, dst_k, dst_v)]
    pairs = [(5, 0), (2, 9), (6, 3), (0, 10)]          # (block of src, block of dst)
    k2, v2 = pool_after_swap(src_k, src_v, dst_k, dst_v, pairs)
    g, s, e = np.meshgrid(np.arange(hkv), np.arange(bs), np.arange(d), indexing="ij")
    for sb, db in pairs:
        # the destination block now spells the source block's id, in K and in V
        assert np.array_equal(k2[db], 10000 * sb + 1000 * g + 10 * s + e)
        assert np.array_equal(v2[db], -500000 + 10000 * sb + 1000 * g + 10 * s + e)
    for db in set(range(11)) - {d_ for _, d_ in pairs}:
        assert np.array_equal(k2[db], saved[2][db]) and np.array_equal(v2[db], saved[3][db])
    # inputs are untouched (the result is a copy), sources included
    for x, y in zip((src_k, src_v, dst_k, dst_v), saved):
        assert np.array_equal(x, y)
    # no pairs: the destination comes back unchanged
    k3, v3 = pool_after_swap(src_k, src_v, dst_k, dst_v, np.zeros((0, 2), dtype=np.int32))
    assert np.array_equal(k3, dst_k) and np.array_equal(v3, dst_v)
