"""Plausible mistakes planted in the oracle's multi-query attention and
multi-token append; each must make at least one pin of
tests/test_oracle_multi_query.py fail."""

import numpy as np
import pytest

import oracle.paged_attention as opa
from tests import test_oracle_multi_query as pins

PINS = [name for name in dir(pins) if name.startswith("test_")]


def _attention(visible):
    """Multi-query attention where query j of a sequence of length n sees
    the positions visible(n, nq, j) returns (a range end), None = zero row."""
    def attend(q, k_pool, v_pool, block_tables, seq_lens, block_size, scale):
        batch, nq, num_heads, head_dim = q.shape
        out = np.zeros((batch, nq, num_heads, head_dim))
        for i in range(batch):
            n = int(seq_lens[i])
            for j in range(nq):
                end = visible(n, nq, j)
                if end is None:
                    continue
                k = opa.gather_sequence(k_pool, block_tables[i], end, block_size)
                v = opa.gather_sequence(v_pool, block_tables[i], end, block_size)
                out[i, j] = opa.dense_decode_attention(q[i, j], k, v, scale)
        return out
    return attend


def _append(position):
    def append(k_pool, v_pool, k_new, v_new, block_tables, seq_lens, block_size):
        k_out, v_out = k_pool.copy(), v_pool.copy()
        nq = k_new.shape[1]
        for i in range(len(seq_lens)):
            n = int(seq_lens[i])
            for j in range(nq):
                pos = position(n, nq, j)
                if pos < 0:
                    continue
                logical, slot = opa.block_and_slot(pos, block_size)
                phys = int(block_tables[i][logical])
                k_out[phys, :, slot, :] = k_new[i, j]
                v_out[phys, :, slot, :] = v_new[i, j]
        return k_out, v_out
    return append


MUTANTS = {
    # every new token sees the whole history, its successors included
    "no_causal_mask": {"paged_multi_query_attention": _attention(
        lambda n, nq, j: n if n - nq + j >= 0 else None)},
    # a new token does not see itself
    "excludes_itself": {"paged_multi_query_attention": _attention(
        lambda n, nq, j: (n - nq + j) if n - nq + j > 0 else None)},
    # new tokens taken in reverse order
    "reversed_positions": {"paged_multi_query_attention": _attention(
        lambda n, nq, j: (n - j) if n - 1 - j >= 0 else None)},
    # a query before the start sees the first token instead of nothing
    "clamped_start": {"paged_multi_query_attention": _attention(
        lambda n, nq, j: max(n - nq + j, 0) + 1 if n > 0 else None)},
    # the new tokens stored in reverse order
    "append_reversed": {"pool_after_append_multi": _append(lambda n, nq, j: n - 1 - j)},
}


def _failing():
    failed = []
    for name in PINS:
        fn = getattr(pins, name)
        args = [()]
        for m in getattr(fn, "pytestmark", []):
            if m.name == "parametrize":
                names = [s.strip() for s in m.args[0].split(",")]
                args = [tuple(v) if len(names) > 1 else (v,) for v in m.args[1]]
        for a in args:
            try:
                fn(*a)
            except (Exception, pytest.fail.Exception):
                failed.append(name)
                break
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_multi_query_pins_catch_mutant(mutant, monkeypatch):
    for attr, fn in MUTANTS[mutant].items():
        monkeypatch.setattr(pins, attr, fn)
    assert _failing(), f"no pin catches {mutant}"


def test_unmutated_multi_query_oracle_passes_every_pin():
    assert _failing() == []
