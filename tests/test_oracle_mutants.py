"""Plants plausible mistakes in the oracle (on the CPU) and checks that the
pins in test_oracle.py catch every one of them.

Each mutant replaces one oracle function, inside both the oracle module and
the pin module's namespace; the pins are then re-run and at least one must
fail. Nothing here touches the GPU or the HIP library.
"""

import numpy as np
import pytest

import oracle.paged_attention as pa
import tests.test_oracle as pins

ALL_PINS = [name for name in dir(pins) if name.startswith("test_")]


def _dense_per_block(q, k, v, scale):
    out = np.zeros((q.shape[0], q.shape[1]))
    for a in range(0, k.shape[0], 16):
        out += _ORIG["dense_decode_attention"](q, k[a:a + 16], v[a:a + 16], scale)
    return out


def _dense_mod_group(q, k, v, scale):
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    out = np.zeros(q.shape)
    for h in range(q.shape[0]):
        g = h % k.shape[1]
        s = scale * (k[:, g] @ q[h])
        w = np.exp(s - s.max())
        out[h] = w @ v[:, g] / w.sum()
    return out


def _dense_variant(score_fn, normalise=True):
    def f(q, k, v, scale):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        out = np.zeros(q.shape)
        if k.shape[0] == 0:
            return out
        grp = q.shape[0] // k.shape[1]
        for h in range(q.shape[0]):
            s = score_fn(scale, k[:, h // grp], q[h])
            w = np.exp(s - s.max())
            out[h] = w @ v[:, h // grp] / (w.sum() if normalise else 1.0)
        return out
    return f


def _paged_drop_current(q, k_pool, v_pool, tables, lens, bs, scale):
    return _ORIG["paged_decode_attention"](q, k_pool, v_pool, tables,
                                           [max(0, int(n) - 1) for n in lens], bs, scale)


def _slot_reversed(position, block_size):
    return position // block_size, block_size - 1 - position % block_size


def _append_one_late(k_pool, v_pool, k_new, v_new, tables, lens, bs):
    return _ORIG["pool_after_append"](k_pool, v_pool, k_new, v_new, tables,
                                      [int(n) + 1 if n > 0 else 0 for n in lens], bs)


def _copy_backwards(k_pool, v_pool, pairs):
    return _ORIG["pool_after_copy"](k_pool, v_pool,
                                    [(d, s) for s, d in np.asarray(pairs).reshape(-1, 2)])


def _swap_pairs_reversed(src_k, src_v, dst_k, dst_v, pairs):
    k_out, v_out = dst_k.copy(), dst_v.copy()
    for s, d in np.asarray(pairs).reshape(-1, 2):
        k_out[int(s)] = src_k[int(d)]
        v_out[int(s)] = src_v[int(d)]
    return k_out, v_out


def _swap_k_and_v_crossed(src_k, src_v, dst_k, dst_v, pairs):
    k_out, v_out = dst_k.copy(), dst_v.copy()
    for s, d in np.asarray(pairs).reshape(-1, 2):
        k_out[int(d)] = src_v[int(s)]
        v_out[int(d)] = src_k[int(s)]
    return k_out, v_out


def _swap_in_place(src_k, src_v, dst_k, dst_v, pairs):
    for s, d in np.asarray(pairs).reshape(-1, 2):
        dst_k[int(d)] = src_k[int(s)]
        dst_v[int(d)] = src_v[int(s)]
    return dst_k, dst_v


_ORIG = {name: getattr(pa, name) for name in
         ("dense_decode_attention", "paged_decode_attention", "block_and_slot",
          "pool_after_append", "pool_after_copy")}

MUTANTS = {
    "per_block_softmax": ("dense_decode_attention", _dense_per_block),
    "kv_head_h_mod_hkv": ("dense_decode_attention", _dense_mod_group),
    "no_scale": ("dense_decode_attention", _dense_variant(lambda sc, k, q: k @ q)),
    "negated_scores": ("dense_decode_attention", _dense_variant(lambda sc, k, q: -sc * (k @ q))),
    "scale_squared": ("dense_decode_attention", _dense_variant(lambda sc, k, q: sc * sc * (k @ q))),
    "unnormalised": ("dense_decode_attention",
                     _dense_variant(lambda sc, k, q: sc * (k @ q), normalise=False)),
    "drop_current_token": ("paged_decode_attention", _paged_drop_current),
    "slot_reversed": ("block_and_slot", _slot_reversed),
    "append_one_late": ("pool_after_append", _append_one_late),
    "copy_backwards": ("pool_after_copy", _copy_backwards),
    "swap_pairs_reversed": ("pool_after_swap", _swap_pairs_reversed),
    "swap_k_and_v_crossed": ("pool_after_swap", _swap_k_and_v_crossed),
    "swap_writes_its_input": ("pool_after_swap", _swap_in_place),
}


def _run_pins():
    """Names of pins that fail (assertion or error) under the current oracle."""
    failed = []
    for name in ALL_PINS:
        fn = getattr(pins, name)
        params = getattr(fn, "pytestmark", [])
        argsets = [()]
        for m in params:
            if m.name == "parametrize":
                argsets = [(v,) for v in m.args[1]]
        for args in argsets:
            try:
                fn(*args)
            except Exception:
                failed.append(name)
                break
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant, monkeypatch):
    target, replacement = MUTANTS[mutant]
    monkeypatch.setattr(pa, target, replacement)
    if hasattr(pins, target):
        monkeypatch.setattr(pins, target, replacement)
    failed = _run_pins()
    assert failed, f"no pin catches mutant {mutant}"


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins() == []
