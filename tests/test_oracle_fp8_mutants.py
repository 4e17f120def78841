"""Plausible mistakes planted in the oracle's FP8 quantisation; each must make
at least one pin of tests/test_oracle_fp8.py fail."""

import numpy as np
import pytest

import oracle.fp8 as f8
from tests import test_oracle_fp8 as pins

PINS = [name for name in dir(pins) if name.startswith("test_")]


def _value_with(bias=7, sub_exp=-6):
    def value(code):
        code = int(code) & 0xFF
        sign = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 0xF, code & 0x7
        if e == 0xF and m == 0x7:
            return float("nan")
        if e == 0:
            return sign * (2.0 ** sub_exp) * (m / 8.0)
        return sign * (2.0 ** (e - bias)) * (1.0 + m / 8.0)
    return value


def _decode_with(value):
    def decode(codes):
        table = np.array([value(c) for c in range(256)], dtype=np.float64)
        return table[np.asarray(codes, dtype=np.uint8)]
    return decode


def _encode_variant(tie_to_upper=False, saturate=True, keep_sign=True):
    def encode(values):
        v = np.asarray(values, dtype=np.float64)
        pos = np.array([f8.e4m3_value(c) for c in range(0x7F)], dtype=np.float64)
        a = np.abs(v) if not saturate else np.minimum(np.abs(v), f8.MAX_FINITE)
        hi = np.clip(np.searchsorted(pos, a, side="left"), 0, 0x7E)
        lo = np.clip(hi - 1, 0, 0x7E)
        d_lo, d_hi = a - pos[lo], pos[hi] - a
        tie = hi if tie_to_upper else np.where(lo % 2 == 0, lo, hi)
        pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, tie))
        if not saturate:
            pick = np.where(np.abs(v) > f8.MAX_FINITE, 0x7F, pick)
        sign = np.where(np.signbit(v), 0x80, 0x00) if keep_sign else 0
        codes = (sign | pick).astype(np.uint8)
        return np.where(np.isnan(v), f8.NAN_CODE, codes).astype(np.uint8)
    return encode


def _dequant_scale_axis(axis=1, head0=False):
    def dequantize_pool(pool, scales):
        sc = np.asarray(scales, dtype=np.float64)
        if head0:
            sc = np.full_like(sc, sc[0])
        shape = [1, 1, 1, 1]
        shape[axis] = -1
        return f8.decode(pool) * sc.reshape(shape)
    return dequantize_pool


def _multi_append_variant(reverse=False, shift=0):
    def pool_after_append_multi_fp8(k_pool, v_pool, k_new, v_new, ks, vs, tables, lens, bs):
        k_out, v_out = k_pool.copy(), v_pool.copy()
        nq = k_new.shape[1]
        for i in range(len(lens)):
            n = int(lens[i])
            for j in range(nq):
                pos = n - nq + j + shift
                src = nq - 1 - j if reverse else j
                if n <= 0 or pos < 0 or pos >= n:
                    continue
                b = int(tables[i][pos // bs])
                for g in range(k_pool.shape[1]):
                    k_out[b, g, pos % bs] = f8.quantize(k_new[i][src][g], ks[g])
                    v_out[b, g, pos % bs] = f8.quantize(v_new[i][src][g], vs[g])
        return k_out, v_out
    return pool_after_append_multi_fp8


MUTANTS = {
    "exponent_bias_8": {"fp8_decode": _decode_with(_value_with(bias=8))},
    "subnormal_scale_2^-7": {"fp8_decode": _decode_with(_value_with(sub_exp=-7))},
    "ties_to_upper": {"fp8_encode": _encode_variant(tie_to_upper=True)},
    "overflow_to_nan": {"fp8_encode": _encode_variant(saturate=False)},
    "sign_dropped": {"fp8_encode": _encode_variant(keep_sign=False)},
    "dequant_head0_scale_everywhere": {"fp8_dequantize_pool": _dequant_scale_axis(head0=True)},
    "dequant_scale_on_block_axis": {"fp8_dequantize_pool": _dequant_scale_axis(axis=0)},
    "dequant_scale_on_slot_axis": {"fp8_dequantize_pool": _dequant_scale_axis(axis=2)},
    "multi_append_tokens_reversed": {"pool_after_append_multi_fp8": _multi_append_variant(reverse=True)},
    "multi_append_one_early": {"pool_after_append_multi_fp8": _multi_append_variant(shift=-1)},
}


def _failing_pins():
    failed = []
    for name in PINS:
        try:
            getattr(pins, name)()
        except Exception:
            failed.append(name)
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_fp8_pins_catch_mutant(mutant, monkeypatch):
    for attr, fn in MUTANTS[mutant].items():
        monkeypatch.setattr(pins, attr, fn)
    assert _failing_pins(), f"no pin catches {mutant}"


def test_unmutated_fp8_oracle_passes_every_pin():
    assert _failing_pins() == []
