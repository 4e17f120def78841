"""Pins for the oracle's multi-query paged attention: torch's causal
scaled_dot_product_attention on the contiguous history (an independent
library routine), the single-query oracle as the one-query case, 50-digit
mpmath on tiny inputs, and the append of several tokens."""

import mpmath
import numpy as np
import pytest
import torch

from oracle import (paged_decode_attention, paged_multi_query_attention, pool_after_append,
                    pool_after_append_multi)


def random_paged(rng, lens, hkv, d, bs, extra=3):
    nb = sum(-(-n // bs) for n in lens) + extra
    perm = rng.permutation(nb)
    k_pool = rng.standard_normal((nb, hkv, bs, d))
    v_pool = rng.standard_normal((nb, hkv, bs, d))
    tables = np.full((len(lens), max(-(-n // bs) for n in lens)), -1)
    cur = 0
    for i, n in enumerate(lens):
        m = -(-n // bs)
        tables[i, :m] = perm[cur:cur + m]
        cur += m
    return k_pool, v_pool, tables


def contiguous(pool, table, n, bs):
    return np.stack([pool[table[t // bs], :, t % bs] for t in range(n)])


@pytest.mark.parametrize("nq,group", [(1, 1), (3, 1), (4, 2), (8, 4), (16, 1)])
def test_matches_torch_causal_sdpa(nq, group):
    rng = np.random.default_rng(nq * 10 + group)
    hkv, d, bs = 2, 8, 4
    lens = [nq, nq + 1, 23, 40]
    k_pool, v_pool, tables = random_paged(rng, lens, hkv, d, bs)
    q = rng.standard_normal((len(lens), nq, hkv * group, d))
    scale = 0.3
    out = paged_multi_query_attention(q, k_pool, v_pool, tables, lens, bs, scale)
    for i, n in enumerate(lens):
        k = torch.from_numpy(contiguous(k_pool, tables[i], n, bs)).permute(1, 0, 2)   # [Hkv][L][D]
        v = torch.from_numpy(contiguous(v_pool, tables[i], n, bs)).permute(1, 0, 2)
        k = k.repeat_interleave(group, 0)
        v = v.repeat_interleave(group, 0)
        qq = torch.from_numpy(q[i]).permute(1, 0, 2)                                 # [H][nq][D]
        mask = torch.arange(n)[None, :] <= (n - nq + torch.arange(nq))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, k, v, attn_mask=mask,
                                                               scale=scale)
        assert np.abs(out[i] - ref.permute(1, 0, 2).numpy()).max() < 1e-12


def test_one_query_is_the_decode_oracle():
    rng = np.random.default_rng(3)
    lens = [1, 16, 17, 37]
    k_pool, v_pool, tables = random_paged(rng, lens, 2, 8, 16)
    q = rng.standard_normal((4, 1, 4, 8))
    a = paged_multi_query_attention(q, k_pool, v_pool, tables, lens, 16, 0.5)[:, 0]
    b = paged_decode_attention(q[:, 0], k_pool, v_pool, tables, lens, 16, 0.5)
    assert np.array_equal(a, b)


def test_queries_before_the_start_are_zero():
    rng = np.random.default_rng(4)
    k_pool, v_pool, tables = random_paged(rng, [2], 1, 4, 4)
    q = rng.standard_normal((1, 5, 1, 4))
    out = paged_multi_query_attention(q, k_pool, v_pool, tables, [2], 4, 1.0)
    assert (out[0, :3] == 0).all() and np.abs(out[0, 3:]).sum() > 0


def test_matches_mpmath_50_digits():
    mpmath.mp.dps = 50
    rng = np.random.default_rng(5)
    lens, nq, d, bs = [5, 3], 3, 3, 2
    k_pool, v_pool, tables = random_paged(rng, lens, 1, d, bs)
    q = rng.standard_normal((2, nq, 1, d))
    out = paged_multi_query_attention(q, k_pool, v_pool, tables, lens, bs, 0.7)
    for i, n in enumerate(lens):
        k, v = contiguous(k_pool, tables[i], n, bs), contiguous(v_pool, tables[i], n, bs)
        for j in range(nq):
            pos = n - nq + j
            s = [mpmath.mpf(0.7) * mpmath.fsum(mpmath.mpf(q[i, j, 0, x]) * mpmath.mpf(k[t, 0, x])
                                               for x in range(d)) for t in range(pos + 1)]
            e = [mpmath.exp(x) for x in s]
            z = mpmath.fsum(e)
            for x in range(d):
                want = mpmath.fsum(e[t] * mpmath.mpf(v[t, 0, x]) for t in range(pos + 1)) / z
                assert abs(float(want) - out[i, j, 0, x]) < 1e-13


def test_append_multi_equals_repeated_single_appends():
    rng = np.random.default_rng(6)
    lens, nq, hkv, d, bs = [3, 17, 40], 4, 2, 4, 8
    k_pool, v_pool, tables = random_paged(rng, lens, hkv, d, bs)
    kn = rng.standard_normal((3, nq, hkv, d))
    vn = rng.standard_normal((3, nq, hkv, d))
    a = pool_after_append_multi(k_pool, v_pool, kn, vn, tables, lens, bs)
    kb, vb = k_pool, v_pool
    for j in range(nq):
        step = [n - nq + j + 1 if n - nq + j >= 0 else 0 for n in lens]
        kb, vb = pool_after_append(kb, vb, kn[:, j], vn[:, j], tables, step, bs)
    assert np.array_equal(a[0], kb) and np.array_equal(a[1], vb)
