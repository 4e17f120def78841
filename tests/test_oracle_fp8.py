"""Pins for the oracle's FP8 (OCP E4M3) quantisation, against facts that do
not come from the oracle: fixed values of the format, torch's independent
float8_e4m3fn conversion, brute force and round trips."""

import numpy as np
import pytest
import torch

from oracle import (fp8_decode, fp8_dequantize_pool, fp8_encode, fp8_quantize,
                    pool_after_append_fp8, pool_after_append_multi_fp8)
from oracle.fp8 import _encode_one

ALL = np.arange(256, dtype=np.uint8)


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def torch_encode(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_fixed_values_of_the_format():
    v = fp8_decode(ALL)
    assert v[0x00] == 0.0 and not np.signbit(v[0x00])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9                  # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9              # largest subnormal
    assert v[0x08] == 2.0 ** -6                  # smallest normal
    assert v[0x38] == 1.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254
    assert np.all(np.diff(v[:0x7F]) > 0)         # codes 0..126 increase


def test_decode_matches_torch_for_every_code():
    ours, ref = fp8_decode(ALL), torch_decode(ALL)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 150.0)])
    x = x[np.abs(x) <= 464].astype(np.float32)
    assert np.array_equal(fp8_encode(x), torch_encode(x))


def test_midpoints_round_to_the_even_code():
    v = fp8_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)     # exact in float32
    codes = fp8_encode(mids)
    lower = np.arange(0x7E)
    want = np.where(lower % 2 == 0, lower, lower + 1)
    assert np.array_equal(codes, want.astype(np.uint8))
    assert np.array_equal(codes, torch_encode(mids))
    assert np.array_equal(fp8_encode(-mids), (want | 0x80).astype(np.uint8))


def test_round_trip_of_every_finite_code():
    finite = ALL[np.isfinite(fp8_decode(ALL))]
    assert np.array_equal(fp8_encode(fp8_decode(finite)), finite)


def test_saturation_signed_zero_and_nan():
    assert fp8_encode(np.float32(1e6)) == 0x7E and fp8_encode(np.float32(-1e6)) == 0xFE
    assert fp8_encode(np.float32(470.0)) == 0x7E       # torch gives NaN here; we saturate
    assert fp8_encode(np.float32(0.0)) == 0x00 and fp8_encode(np.float32(-0.0)) == 0x80
    assert fp8_encode(np.float32(np.nan)) == 0x7F
    assert fp8_encode(np.float32(2.0 ** -10)) == 0x00   # half the smallest subnormal: tie to even
    assert fp8_encode(np.float32(3 * 2.0 ** -10)) == 0x02


def test_vectorised_encode_equals_brute_force():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(400) * s for s in (1e-3, 0.1, 5.0, 200.0, 1000.0)])
    x = x.astype(np.float32)
    brute = np.array([_encode_one(float(y)) for y in x], dtype=np.uint8)
    assert np.array_equal(fp8_encode(x), brute)


def test_quantize_divides_in_float32():
    x = np.array([1.0, -3.0, 0.3], dtype=np.float32)
    s = np.float32(1.0 / 56)
    y = x / s
    assert y.dtype == np.float32
    assert np.array_equal(fp8_quantize(x, s), fp8_encode(y))


def test_append_fp8_writes_only_the_new_slots():
    rng = np.random.default_rng(3)
    nb, hkv, bs, d = 6, 2, 16, 8
    k = rng.integers(0, 255, (nb, hkv, bs, d)).astype(np.uint8)
    v = rng.integers(0, 255, (nb, hkv, bs, d)).astype(np.uint8)
    tables = np.array([[5, 1, 3], [2, -1, -1], [0, -1, -1]], dtype=np.int32)
    lens = np.array([37, 16, 0], dtype=np.int32)
    kn = rng.standard_normal((3, hkv, d)).astype(np.float32)
    vn = rng.standard_normal((3, hkv, d)).astype(np.float32)
    ks, vs = np.array([0.02, 0.03], np.float32), np.array([0.05, 0.01], np.float32)
    k2, v2 = pool_after_append_fp8(k, v, kn, vn, ks, vs, tables, lens, bs)
    changed = np.argwhere(np.any(k2 != k, axis=-1) | np.any(v2 != v, axis=-1))
    allowed = {(3, g, 4) for g in range(hkv)} | {(2, g, 15) for g in range(hkv)}
    assert {tuple(c) for c in changed} <= allowed
    for g in range(hkv):
        assert np.array_equal(k2[3, g, 4], torch_encode(kn[0, g] / ks[g]))
        assert np.array_equal(v2[2, g, 15], torch_encode(vn[1, g] / vs[g]))


def test_dequantize_pool_scales_each_head_by_its_own_factor():
    # A pool of codes read back as values: code value (torch's own
    # float8_e4m3fn conversion) times the scale of the code's kv head. The
    # pool is 4 x 4 x 4 x 16 so that a scale applied along the block or slot
    # axis still broadcasts and has to be caught by its values; the scales are
    # distinct powers of two, so every product is exact.
    rng = np.random.default_rng(31)
    codes = rng.integers(0, 256, size=(4, 4, 4, 16)).astype(np.uint8)
    codes[codes & 0x7F == 0x7F] = 0x38                       # no NaN codes here
    codes[1, :, 2, 5] = 0x38                                 # 1.0 in every head
    scales = np.array([2.0 ** -3, 2.0 ** 1, 2.0 ** 5, 2.0 ** -7], dtype=np.float32)
    got = fp8_dequantize_pool(codes, scales)
    ref = torch_decode(codes)
    for g in range(4):
        assert np.array_equal(got[:, g], ref[:, g] * float(scales[g]))
        assert got[1, g, 2, 5] == float(scales[g])
    # the NaN code stays NaN, whatever the head's scale
    nan_pool = np.full((1, 4, 1, 2), 0x7F, dtype=np.uint8)
    assert np.isnan(fp8_dequantize_pool(nan_pool, scales)).all()


def test_multi_token_append_equals_one_token_appends_in_order():
    # nq new tokens per sequence at positions L-nq .. L-1 (blog.aqudi.me
    # section 4: several tokens per pass); stored one at a time by the
    # single-token append with lengths L-nq+1 .. L, the pools must be the same
    rng = np.random.default_rng(41)
    bs, hkv, d, nq = 8, 3, 16, 5
    lens = np.array([0, 3, 5, 9, 17, 40], dtype=np.int32)      # includes L < nq and L = 0
    nblk = [-(-int(n) // bs) for n in lens]
    perm = rng.permutation(sum(nblk) + 4)
    tables = np.full((len(lens), max(nblk)), -1, dtype=np.int32)
    c = 0
    for i, nb in enumerate(nblk):
        tables[i, :nb] = perm[c:c + nb]
        c += nb
    k_pool = rng.integers(0, 256, size=(len(perm), hkv, bs, d)).astype(np.uint8)
    v_pool = rng.integers(0, 256, size=(len(perm), hkv, bs, d)).astype(np.uint8)
    k_new = (rng.standard_normal((len(lens), nq, hkv, d)) * 3).astype(np.float32)
    v_new = (rng.standard_normal((len(lens), nq, hkv, d)) * 3).astype(np.float32)
    ks = np.array([0.5, 0.03125, 2.0], dtype=np.float32)
    vs = np.array([0.25, 1.0, 0.0078125], dtype=np.float32)
    k2, v2 = pool_after_append_multi_fp8(k_pool, v_pool, k_new, v_new, ks, vs, tables, lens, bs)
    kr, vr = k_pool, v_pool
    for j in range(nq):
        step_lens = np.where(lens - nq + j >= 0, lens - nq + j + 1, 0)
        kr, vr = pool_after_append_fp8(kr, vr, k_new[:, j], v_new[:, j], ks, vs, tables,
                                       step_lens, bs)
    assert np.array_equal(k2, kr) and np.array_equal(v2, vr)
    # sequence 3 (L = 9): token 4 (the last) sits at position 8: block 1, slot 0
    assert np.array_equal(k2[tables[3, 1], :, 0], np.stack([fp8_quantize(k_new[3, 4, g], ks[g])
                                                           for g in range(hkv)]))
