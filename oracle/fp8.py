"""FP8 (OCP E4M3) KV-cache quantisation, plain and slow, for the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): imported by tests/, the
smoke check and the bench's CPU-baseline leg, never by the product path.

The pages name quantisation of the KV cache as a way to save memory and
bandwidth (blog.aqudi.me, "벤치마크가 다가 아니야! vLLM으로 보는 LLM 추론
최적화", section 4) without fixing a format. The reading taken here:

* Storage format: OCP 8-bit floating point E4M3 ("e4m3fn"). A code is
  s eeee mmm: bias 7; e = 0 encodes subnormals (-1)^s * 2^-6 * m/8;
  e = 1..15 encodes (-1)^s * 2^(e-7) * (1 + m/8), except e = 15, m = 7, which
  is NaN. There is no infinity; the largest finite magnitude is 448.
* Scales: one float per kv head for K and one for V, chosen by the caller.
  A stored value means code_value * scale.
* Appending quantises in float32: y = float32(x) / float32(scale) (IEEE
  division), then y is rounded to the nearest E4M3 value, ties to the even
  code; magnitudes beyond 448 saturate to 448 (NaN stays NaN).
"""

import numpy as np

MAX_FINITE = 448.0
NAN_CODE = 0x7F


def e4m3_value(code):
    """Exact value (float64) of one E4M3 code, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (2.0 ** -6) * (m / 8.0)
    return sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


def decode(codes):
    """uint8 codes (any shape) -> float64 values."""
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def _encode_one(y):
    """Nearest E4M3 code of one float (ties to the even code), saturating:
    a brute-force search over every non-negative finite code."""
    if np.isnan(y):
        return NAN_CODE
    sign = 0x80 if (y < 0 or (y == 0 and np.signbit(y))) else 0x00
    a = abs(float(y))
    if a >= MAX_FINITE:
        return sign | 0x7E
    best, best_err = 0, None
    for c in range(0x7F):
        err = abs(e4m3_value(c) - a)
        if best_err is None or err < best_err or (err == best_err and c % 2 == 0):
            best, best_err = c, err
    return sign | best


def encode(values):
    """float32/float64 values (any shape) -> uint8 E4M3 codes: the nearest
    finite value, ties to the even code, magnitudes beyond 448 saturating.
    Codes 0x00 .. 0x7E are the non-negative finite values in increasing
    order, so the nearest one is one of the two neighbours of |y| in that
    list."""
    v = np.asarray(values, dtype=np.float64)
    pos = np.array([e4m3_value(c) for c in range(0x7F)], dtype=np.float64)
    a = np.minimum(np.abs(v), MAX_FINITE)
    hi = np.clip(np.searchsorted(pos, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - pos[lo]
    d_hi = pos[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    sign = np.where(np.signbit(v), 0x80, 0x00)
    codes = (sign | pick).astype(np.uint8)
    return np.where(np.isnan(v), NAN_CODE, codes).astype(np.uint8)


def quantize(x, scale):
    """Codes of x (float32-representable input) under `scale`: the division
    is done in float32, as the append does."""
    y = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return encode(y.astype(np.float32))


def pool_after_append_fp8(k_pool, v_pool, k_new, v_new, k_scales, v_scales, block_tables,
                          seq_lens, block_size):
    """uint8 pools after each sequence stores its new token, quantised per kv
    head: slot (L-1) % block_size of block table[(L-1) // block_size] gets
    quantize(k_new[i][g], k_scales[g]) (and V likewise). Length-0 rows store
    nothing. Returns copies."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    num_kv_heads = k_pool.shape[1]
    for i in range(len(seq_lens)):
        n = int(seq_lens[i])
        if n <= 0:
            continue
        logical, slot = (n - 1) // block_size, (n - 1) % block_size
        physical = int(block_tables[i][logical])
        for g in range(num_kv_heads):
            k_out[physical, g, slot, :] = quantize(k_new[i][g], k_scales[g])
            v_out[physical, g, slot, :] = quantize(v_new[i][g], v_scales[g])
    return k_out, v_out


def pool_after_append_multi_fp8(k_pool, v_pool, k_new, v_new, k_scales, v_scales, block_tables,
                                seq_lens, block_size):
    """uint8 pools after each sequence stores nq new tokens, quantised per kv
    head: k_new, v_new [B][nq][H_kv][D]; token j of a sequence of (new)
    length L goes to position L - nq + j (skipped when negative), i.e. slot
    (L - nq + j) % block_size of block table[(L - nq + j) // block_size].
    Returns copies."""
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    nq = k_new.shape[1]
    num_kv_heads = k_pool.shape[1]
    for i in range(len(seq_lens)):
        n = int(seq_lens[i])
        for j in range(nq):
            pos = n - nq + j
            if n <= 0 or pos < 0:
                continue
            physical = int(block_tables[i][pos // block_size])
            for g in range(num_kv_heads):
                k_out[physical, g, pos % block_size, :] = quantize(k_new[i][j][g], k_scales[g])
                v_out[physical, g, pos % block_size, :] = quantize(v_new[i][j][g], v_scales[g])
    return k_out, v_out


def dequantize_pool(pool, scales):
    """float64 values of a uint8 pool [num_blocks][Hkv][bs][D] with per-head scales."""
    return decode(pool) * np.asarray(scales, dtype=np.float64)[None, :, None, None]
