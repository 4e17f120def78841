"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before enqueuing anything. None
of these calls reaches the GPU (every call here fails validation or is a
no-op), so they run without one."""

import os
import re
import subprocess

import pytest

from paged_kv_cache_440_amd import _lib
from paged_kv_cache_440_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = 0x10000           # an aligned non-null address; never dereferenced here


def declared_symbols():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"PKV_API\s+[\w\s\*]*?\b(pkv_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        pytest.skip("libpkv.so not built")
    return _lib.library()


def test_header_declares_the_three_operations():
    names = declared_symbols()
    for n in ("pkv_kv_cache_append", "pkv_copy_blocks", "pkv_paged_attention_decode",
              "pkv_paged_attention_workspace_size", "pkv_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(declared_symbols()) <= exported
    # nothing else of ours leaks out of the library
    assert not [s for s in exported if "pkv" in s and s not in declared_symbols()]


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert _lib.status_string(code) and _lib.status_string(code) != "unknown status"
    assert _lib.status_string(42) == "unknown status"


def attn(lib, **kw):
    args = dict(out=FAKE, out_dtype=0, q=FAKE, k=FAKE, v=FAKE, tables=FAKE, max_blocks=8,
                lens=FAKE, max_seq_len=100, B=2, H=4, Hkv=4, D=128, bs=16, nb=32,
                scale=0.1, part=0, ws=0, ws_bytes=0, dtype=1, policy=0)
    args.update(kw)
    a = args
    return lib.pkv_paged_attention_decode(a["out"], a["out_dtype"], a["q"], a["k"], a["v"],
                                          a["tables"], a["max_blocks"], a["lens"],
                                          a["max_seq_len"], a["B"], a["H"], a["Hkv"], a["D"],
                                          a["bs"], a["nb"], a["scale"], a["part"], a["ws"],
                                          a["ws_bytes"], a["dtype"], a["policy"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INVALID),
    (dict(H=6, Hkv=4), INVALID),            # heads not a multiple of kv heads
    (dict(H=12, Hkv=4), UNSUPPORTED),       # group 3
    (dict(H=64, Hkv=4), UNSUPPORTED),       # group 16
    (dict(D=96), UNSUPPORTED),
    (dict(bs=12), UNSUPPORTED),
    (dict(bs=4), UNSUPPORTED),
    (dict(bs=512), UNSUPPORTED),
    (dict(dtype=3), UNSUPPORTED),            # FP8 pools go through the _fp8 entry point
    (dict(dtype=4), INVALID),
    (dict(out_dtype=7), INVALID),
    (dict(part=100), INVALID),              # not a multiple of 64
    (dict(part=-64), INVALID),
    (dict(part=-2), INVALID),
    (dict(part=-1, ws=0), WORKSPACE),        # the balanced schedule always needs one
    (dict(part=-1, ws=FAKE, ws_bytes=1 << 20), WORKSPACE),
    (dict(max_seq_len=8 * 16 + 1), INVALID),  # beyond the table's capacity
    (dict(scale=float("nan")), INVALID),
    (dict(q=0), INVALID),
    (dict(k=0), INVALID),
    (dict(tables=0), INVALID),
    (dict(lens=0), INVALID),
    (dict(out=0), INVALID),
    (dict(q=FAKE + 4), INVALID),            # misaligned
    (dict(out=FAKE + 8), INVALID),          # output rows are written 16 bytes at a time
    (dict(part=64, ws=0), WORKSPACE),       # 100 tokens in 64-token partitions need a workspace
    (dict(part=64, ws=FAKE, ws_bytes=16), WORKSPACE),
    (dict(part=64, ws=FAKE + 8, ws_bytes=1 << 20), WORKSPACE),
    (dict(policy=2), INVALID),              # neither PKV_KV_STREAM nor PKV_KV_REUSE
    (dict(policy=-1), INVALID),
    (dict(B=0), OK),                        # nothing to do, nothing enqueued
    (dict(B=0, policy=1), OK),
    (dict(B=0, policy=0x10), OK),           # PKV_STAGE_WALK
    (dict(B=0, policy=0x21), OK),           # PKV_STAGE_MERGE with PKV_KV_REUSE
    (dict(policy=0x30), INVALID),           # both stages
    (dict(policy=0x12), INVALID),           # a stage with an unknown policy
    (dict(policy=0x80), INVALID),           # an unknown flag
    (dict(B=0, policy=0x40), OK),           # PKV_WALKER_VECTOR
    (dict(policy=0x41), UNSUPPORTED),       # ... with cached loads
])
def test_attention_validation(lib, kw, status):
    assert attn(lib, **kw) == status


def test_workspace_size_formula(lib):
    f = _lib.paged_attention_workspace_size
    assert f(64, 40, 40, 128, 2048, 0) == 0
    assert f(64, 40, 40, 128, 512, 512) == 0
    assert f(64, 40, 40, 128, 2048, 512) == 64 * 40 * 4 * (128 + 2) * 4
    assert f(64, 40, 40, 128, 2049, 512) == 64 * 40 * 5 * (128 + 2) * 4
    assert f(16, 64, 8, 128, 32768, 512) == 16 * 64 * 64 * 130 * 4
    assert f(-1, 40, 40, 128, 2048, 512) == 0
    # balanced: two records of G rows per persistent wave (at most 4096
    # waves), then two ints of merge information per wave
    assert f(64, 40, 40, 128, 2048, -1) == 2 * 4096 * 1 * 130 * 4 + 2 * 4096 * 4
    assert f(16, 64, 8, 128, 32768, -1) == 2 * 4096 * 8 * 130 * 4 + 2 * 4096 * 4
    assert f(1, 4, 4, 64, 1, -1) == 2 * 4096 * 1 * 66 * 4 + 2 * 4096 * 4
    assert f(0, 4, 4, 64, 1, -1) == 0
    assert f(64, 40, 40, 128, 2048, -2) == 0
    assert f(64, 40, 0, 128, 2048, -1) == 0
    assert f(64, 40, 3, 128, 2048, -1) == 0


def append(lib, **kw):
    a = dict(kn=FAKE, vn=FAKE, kp=FAKE, vp=FAKE, tables=FAKE, max_blocks=4, lens=FAKE, B=3,
             Hkv=2, D=64, bs=16, nb=10, dtype=0)
    a.update(kw)
    return lib.pkv_kv_cache_append(a["kn"], a["vn"], a["kp"], a["vp"], a["tables"],
                                   a["max_blocks"], a["lens"], a["B"], a["Hkv"], a["D"], a["bs"],
                                   a["nb"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-2), INVALID), (dict(Hkv=0), INVALID), (dict(nb=0), INVALID),
    (dict(max_blocks=0), INVALID), (dict(dtype=5), INVALID), (dict(dtype=3), UNSUPPORTED),
    (dict(D=80), UNSUPPORTED),
    (dict(bs=24), UNSUPPORTED), (dict(kn=0), INVALID), (dict(vp=0), INVALID),
    (dict(tables=0), INVALID), (dict(lens=0), INVALID), (dict(kp=FAKE + 2), INVALID),
    (dict(B=0), OK),
])
def test_append_validation(lib, kw, status):
    assert append(lib, **kw) == status


def copy(lib, **kw):
    a = dict(kp=FAKE, vp=FAKE, mapping=FAKE, n=3, Hkv=2, D=64, bs=16, nb=10, dtype=2)
    a.update(kw)
    return lib.pkv_copy_blocks(a["kp"], a["vp"], a["mapping"], a["n"], a["Hkv"], a["D"], a["bs"],
                               a["nb"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), INVALID), (dict(Hkv=-1), INVALID), (dict(nb=0), INVALID),
    (dict(dtype=-1), INVALID), (dict(D=32), UNSUPPORTED), (dict(bs=3), UNSUPPORTED),
    (dict(kp=0), INVALID), (dict(mapping=0), INVALID), (dict(vp=FAKE + 1), INVALID),
    (dict(n=0, mapping=0), OK),
])
def test_copy_validation(lib, kw, status):
    assert copy(lib, **kw) == status


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.library()


def test_probe_validation(lib):
    assert lib.pkv_probe_read(0, 1 << 20, FAKE, None) == INVALID
    assert lib.pkv_probe_read(FAKE, 0, FAKE, None) == INVALID
    assert lib.pkv_probe_read(FAKE, 24, FAKE, None) == INVALID        # not a multiple of 16
    assert lib.pkv_probe_read(FAKE + 8, 1 << 20, FAKE, None) == INVALID
    assert lib.pkv_probe_read(FAKE, 1 << 20, 0, None) == INVALID
    assert lib.pkv_probe_copy(FAKE, 0, 1 << 20, None) == INVALID
    assert lib.pkv_probe_copy(FAKE + 4, FAKE, 1 << 20, None) == INVALID
    assert lib.pkv_probe_copy(FAKE, FAKE, 17, None) == INVALID
    words = _lib.library().pkv_probe_read_sink_words
    assert words(0) == 0 and words(24) == 0
    assert words(16) == 1
    assert words(256 * 8 * 16) == 1 and words(256 * 8 * 16 + 16) == 2
    assert words(1 << 34) == 256 * 32                                  # capped grid


def attn_fp8(lib, **kw):
    a = dict(out=FAKE, out_dtype=0, q=FAKE, q_dtype=1, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE,
             tables=FAKE, max_blocks=8, lens=FAKE, max_seq_len=100, B=2, H=4, Hkv=4, D=128,
             bs=16, nb=32, scale=0.1, part=0, ws=0, ws_bytes=0)
    a.update(kw)
    f = lib.pkv_paged_attention_decode_fp8           # argument types set by the binding
    return f(a["out"], a["out_dtype"], a["q"], a["q_dtype"], a["k"], a["v"], a["ks"], a["vs"],
             a["tables"], a["max_blocks"], a["lens"], a["max_seq_len"], a["B"], a["H"], a["Hkv"],
             a["D"], a["bs"], a["nb"], a["scale"], a["part"], a["ws"], a["ws_bytes"],
             a.get("policy", 0), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q_dtype=3), INVALID),               # q is never FP8
    (dict(q_dtype=9), INVALID),
    (dict(D=64), UNSUPPORTED),
    (dict(H=8, Hkv=4, q_dtype=0), UNSUPPORTED),   # fp32 q only with one q head per kv head
    (dict(ks=0), INVALID),
    (dict(vs=0), INVALID),
    (dict(k=FAKE + 8), INVALID),
    (dict(part=64, ws=0), WORKSPACE),
    (dict(B=-1), INVALID),
    (dict(policy=5), INVALID),
    (dict(B=0), OK),
])
def test_attention_fp8_validation(lib, kw, status):
    assert attn_fp8(lib, **kw) == status


def append_fp8(lib, **kw):
    a = dict(kn=FAKE, vn=FAKE, new_dtype=1, kp=FAKE, vp=FAKE, ks=FAKE, vs=FAKE, tables=FAKE,
             max_blocks=4, lens=FAKE, B=3, Hkv=2, D=128, bs=16, nb=10)
    a.update(kw)
    f = lib.pkv_kv_cache_append_fp8                  # argument types set by the binding
    return f(a["kn"], a["vn"], a["new_dtype"], a["kp"], a["vp"], a["ks"], a["vs"], a["tables"],
             a["max_blocks"], a["lens"], a["B"], a["Hkv"], a["D"], a["bs"], a["nb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(new_dtype=3), INVALID), (dict(D=64), UNSUPPORTED), (dict(bs=12), UNSUPPORTED),
    (dict(ks=0), INVALID), (dict(vs=0), INVALID), (dict(kp=FAKE + 1), INVALID),
    (dict(B=-1), INVALID), (dict(B=0), OK),
])
def test_append_fp8_validation(lib, kw, status):
    assert append_fp8(lib, **kw) == status


def test_copy_blocks_accepts_fp8_pools(lib):
    # a zero-pair call validates the arguments and enqueues nothing
    assert copy(lib, dtype=3, n=0, mapping=0) == OK
    assert copy(lib, dtype=3, D=32) == UNSUPPORTED


def attn_multi(lib, **kw):
    a = dict(out=FAKE, out_dtype=0, q=FAKE, k=FAKE, v=FAKE, tables=FAKE, max_blocks=8, lens=FAKE,
             max_seq_len=100, B=2, nq=4, H=4, Hkv=4, D=128, bs=16, nb=32, scale=0.1, part=0,
             ws=0, ws_bytes=0, dtype=1, policy=0)
    a.update(kw)
    return _lib.library().pkv_paged_attention_multi(
        a["out"], a["out_dtype"], a["q"], a["k"], a["v"], a["tables"], a["max_blocks"], a["lens"],
        a["max_seq_len"], a["B"], a["nq"], a["H"], a["Hkv"], a["D"], a["bs"], a["nb"], a["scale"],
        a["part"], a["ws"], a["ws_bytes"], a["dtype"], a["policy"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(nq=0), INVALID), (dict(nq=-1), INVALID),
    (dict(dtype=0), UNSUPPORTED),              # fp32 K/V
    (dict(dtype=3), UNSUPPORTED),              # FP8 pools
    (dict(D=64), UNSUPPORTED),
    (dict(nq=5, H=16, Hkv=4, B=0), OK),        # 5 tokens x 4 heads: 16-column groups (no launch)
    (dict(nq=300, H=16, Hkv=2, dtype=0), UNSUPPORTED),   # any column count, but not fp32 K/V
    (dict(part=64, ws=0), WORKSPACE),
    (dict(policy=3), INVALID),
    (dict(B=0), OK),
])
def test_attention_multi_validation(lib, kw, status):
    assert attn_multi(lib, **kw) == status


def test_append_multi_validation(lib):
    f = _lib.library().pkv_kv_cache_append_multi
    args = lambda **kw: [kw.get(k, v) for k, v in (
        ("kn", FAKE), ("vn", FAKE), ("kp", FAKE), ("vp", FAKE), ("tables", FAKE),
        ("max_blocks", 4), ("lens", FAKE), ("B", 3), ("nq", 2), ("Hkv", 2), ("D", 64),
        ("bs", 16), ("nb", 10), ("dtype", 1), ("stream", None))]
    assert f(*args(nq=0)) == INVALID
    assert f(*args(B=-1)) == INVALID
    assert f(*args(D=80)) == UNSUPPORTED
    assert f(*args(kn=0)) == INVALID
    assert f(*args(vp=FAKE + 2)) == INVALID
    assert f(*args(B=0)) == OK


def swap(lib, **kw):
    a = dict(sk=FAKE, sv=FAKE, snb=10, dk=FAKE, dv=FAKE, dnb=20, mapping=FAKE, n=3, Hkv=2, D=64,
             bs=16, dtype=1)
    a.update(kw)
    return lib.pkv_swap_blocks(a["sk"], a["sv"], a["snb"], a["dk"], a["dv"], a["dnb"],
                               a["mapping"], a["n"], a["Hkv"], a["D"], a["bs"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=-1), INVALID), (dict(Hkv=0), INVALID), (dict(snb=0), INVALID), (dict(dnb=-2), INVALID),
    (dict(dtype=9), INVALID), (dict(D=96), UNSUPPORTED), (dict(bs=12), UNSUPPORTED),
    (dict(sk=0), INVALID), (dict(dv=0), INVALID), (dict(mapping=0), INVALID),
    (dict(dk=FAKE + 8), INVALID), (dict(n=0, mapping=0), OK), (dict(n=0, dtype=3), OK),
])
def test_swap_validation(lib, kw, status):
    assert swap(lib, **kw) == status


def test_swap_refuses_memory_the_device_cannot_reach(lib):
    """Pageable host memory (a numpy array) and unknown addresses never reach
    a launch: PKV_ERR_INVALID where a GPU is present, PKV_ERR_HIP where the
    runtime has no device to ask."""
    import numpy as np
    pageable = np.zeros(20 * 2 * 16 * 64, dtype=np.float16)
    mapping = np.zeros((3, 2), dtype=np.int32)
    p = pageable.ctypes.data
    for kw in (dict(), dict(sk=p, sv=p, dk=p, dv=p, mapping=mapping.ctypes.data)):
        assert swap(lib, **kw) in (INVALID, -4)


def attn_grouped(lib, **kw):
    a = dict(out=FAKE, out_dtype=0, q=FAKE, k=FAKE, v=FAKE, tables=FAKE, max_blocks=8, lens=FAKE,
             max_seq_len=100, B=8, H=4, Hkv=4, D=128, bs=16, nb=32, scale=0.1, part=64,
             gs=4, shared=FAKE, ws=FAKE, ws_bytes=1 << 20, dtype=1, policy=1)
    a.update(kw)
    return lib.pkv_paged_attention_decode_grouped(
        a["out"], a["out_dtype"], a["q"], a["k"], a["v"], a["tables"], a["max_blocks"], a["lens"],
        a["max_seq_len"], a["B"], a["H"], a["Hkv"], a["D"], a["bs"], a["nb"], a["scale"],
        a["part"], a["gs"], a["shared"], a["ws"], a["ws_bytes"], a["dtype"], a["policy"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(part=0), INVALID),                  # fixed partitions only
    (dict(part=-1), INVALID),
    (dict(gs=0), INVALID),
    (dict(B=6), INVALID),                     # not a multiple of the group size
    (dict(shared=0), INVALID),
    (dict(dtype=0), UNSUPPORTED),             # fp32 K/V
    (dict(dtype=3), UNSUPPORTED),             # FP8 pools
    (dict(D=64), UNSUPPORTED),
    (dict(gs=8, H=16, Hkv=4), UNSUPPORTED),   # 8 samples x 4 heads > 16 columns
    (dict(ws=0), WORKSPACE),
    (dict(policy=7), INVALID),
    (dict(B=0), OK),
])
def test_attention_grouped_validation(lib, kw, status):
    assert attn_grouped(lib, **kw) == status


def test_stage_keyword_maps_to_the_flags():
    """The bindings' stage keyword ORs PKV_STAGE_WALK / PKV_STAGE_MERGE into
    kv_policy and refuses anything else before reaching the library."""
    assert _lib._policy(False) == 0 and _lib._policy(True) == 1
    assert _lib._policy(False, "walk") == 0x10 and _lib._policy(True, "merge") == 0x21
    with pytest.raises(ValueError):
        _lib._policy(False, "reduce")


@pytest.mark.parametrize("stage", ["walk", "merge"])
def test_split_stages_refuse_an_internal_workspace(lib, stage):
    """A walk call leaves partial results in its workspace for the merge call:
    the binding must not allocate one of its own for either half (it would be
    dropped, and its memory reused, between the two calls). The refusal comes
    before any tensor reaches the library, so CPU tensors do here."""
    import torch
    q = torch.zeros(2, 4, 128, dtype=torch.float16)
    pool = torch.zeros(8, 4, 16, 128, dtype=torch.float16)
    tables = torch.zeros(2, 8, dtype=torch.int32)
    lens = torch.full((2,), 100, dtype=torch.int32)
    with pytest.raises(ValueError, match="caller-owned workspace"):
        _lib.paged_attention_decode(torch.empty_like(q, dtype=torch.float32), q, pool, pool,
                                    tables, lens, 128, 0.1, partition_size=64, stage=stage)
    # the whole call, or a single pass (nothing to merge), needs no caller workspace
    assert _lib._workspace(0, None, "cpu", None, stage) is None


def test_noalloc_refuses_a_call_beyond_its_static_scratch(lib):
    """pkv_paged_attention_decode_noalloc checks the call's workspace need
    against its static scratch before touching the device: PKV_ERR_SCRATCH
    for more, the ordinary validation of pkv_paged_attention_decode
    otherwise (here a missing pointer)."""
    import ctypes
    SCRATCH = -6
    assert _lib.paged_attention_workspace_size(256, 40, 40, 128, 4096, 64) > _lib.NOALLOC_SCRATCH_BYTES
    args = [FAKE, 0, FAKE, FAKE, FAKE, FAKE, 256, FAKE, 4096, 256, 40, 40, 128, 16, 100000,
            ctypes.c_float(0.1), 64, 1, 0, None]
    assert lib.pkv_paged_attention_decode_noalloc(*args) == SCRATCH
    assert _lib.paged_attention_workspace_size(256, 40, 40, 128, 4096, 1024) <= _lib.NOALLOC_SCRATCH_BYTES
    args[9] = -1                                     # a negative batch is the decode call's error
    assert lib.pkv_paged_attention_decode_noalloc(*args) == INVALID
    args[9] = 0                                      # an empty batch enqueues nothing
    assert lib.pkv_paged_attention_decode_noalloc(*args) == OK


def test_fp8_multi_and_grouped_validation(lib):
    """The FP8 multi-query, multi-token append and grouped entry points refuse
    bad arguments before anything is enqueued (no call here reaches a GPU)."""
    import ctypes
    f = ctypes.c_float(0.1)

    def multi(**kw):
        a = dict(out=FAKE, out_dtype=0, q=FAKE, q_dtype=1, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE,
                 tables=FAKE, max_blocks=8, lens=FAKE, max_seq_len=100, B=2, nq=4, H=4, Hkv=4,
                 D=128, bs=16, nb=32, part=0, ws=0, ws_bytes=0, policy=0)
        a.update(kw)
        return lib.pkv_paged_attention_multi_fp8(
            a["out"], a["out_dtype"], a["q"], a["q_dtype"], a["k"], a["v"], a["ks"], a["vs"],
            a["tables"], a["max_blocks"], a["lens"], a["max_seq_len"], a["B"], a["nq"], a["H"],
            a["Hkv"], a["D"], a["bs"], a["nb"], f, a["part"], a["ws"], a["ws_bytes"], a["policy"],
            None)

    assert multi(q_dtype=0) == UNSUPPORTED            # fp32 q
    assert multi(D=64) == UNSUPPORTED
    assert multi(nq=0) == INVALID
    assert multi(ks=0) == INVALID
    assert multi(part=64) == WORKSPACE
    assert multi(B=0) == OK

    def grouped(**kw):
        a = dict(q_dtype=2, B=8, group_size=4, shared=FAKE, part=64, ws=FAKE, ks=FAKE)
        a.update(kw)
        return lib.pkv_paged_attention_decode_grouped_fp8(
            FAKE, 0, FAKE, a["q_dtype"], FAKE, FAKE, a["ks"], FAKE, FAKE, 8, FAKE, 100, a["B"], 8,
            2, 128, 16, 32, f, a["part"], a["group_size"], a["shared"], a["ws"], 1 << 24, 0, None)

    assert grouped(q_dtype=0) == UNSUPPORTED
    assert grouped(group_size=3) == INVALID            # 8 sequences not a multiple of 3
    assert grouped(part=0) == INVALID                  # fixed partitions only
    assert grouped(shared=0) == INVALID                # no shared-token counts
    assert grouped(ws=0) == WORKSPACE
    assert grouped(B=0) == OK

    def append(**kw):
        a = dict(nq=3, D=128, B=2, ks=FAKE)
        a.update(kw)
        return lib.pkv_kv_cache_append_multi_fp8(FAKE, FAKE, 1, FAKE, FAKE, a["ks"], FAKE, FAKE, 8,
                                                 FAKE, a["B"], a["nq"], 4, a["D"], 16, 32, None)

    assert append(nq=0) == INVALID
    assert append(D=64) == UNSUPPORTED
    assert append(ks=0) == INVALID
    assert append(B=0) == OK


def test_gather_probe_validation(lib):
    args = dict(k=FAKE, v=FAKE, tables=FAKE, max_blocks=8, lens=FAKE, B=2, Hkv=4, row=256, bs=16,
                nb=32, waves=64, loads=4, sink=FAKE)

    def g(**kw):
        a = dict(args)
        a.update(kw)
        return lib.pkv_probe_gather(a["k"], a["v"], a["tables"], a["max_blocks"], a["lens"], a["B"],
                                    a["Hkv"], a["row"], a["bs"], a["nb"], a["waves"], a["loads"],
                                    a["sink"], None)

    def gm(**kw):
        a = dict(args, loads=1)
        a.update(kw)
        return lib.pkv_probe_gather_mfma(a["k"], a["v"], a["tables"], a["max_blocks"], a["lens"],
                                         a["B"], a["Hkv"], a["row"], a["bs"], a["nb"], a["waves"],
                                         a["loads"], a["sink"], None)

    for f in (g, gm):
        assert f(row=64) == UNSUPPORTED
        assert f(bs=12) == UNSUPPORTED
        assert f(sink=0) == INVALID
        assert f(waves=0) == INVALID
        assert f(k=FAKE + 4) == INVALID
    assert gm(loads=4) == UNSUPPORTED
    assert gm(loads=0) == UNSUPPORTED
    assert g(row=64) == UNSUPPORTED
    assert g(loads=3) == UNSUPPORTED
    assert g(bs=12) == UNSUPPORTED
    assert g(sink=0) == INVALID
    assert g(waves=0) == INVALID
    assert g(k=FAKE + 4) == INVALID
