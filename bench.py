"""Decode-step benchmark: paged KV cache append + paged attention on one GPU.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--partition P]

A step is one pass of the whole hot path over one batch: the workload's
copy-on-write block copies (none for the OPT-13B layer), the append of each
sequence's new K/V, and paged decode attention (partition pass plus the
log-sum-exp reduce). Inputs are generated on the host, uploaded once, and
are resident in HBM when timing starts. Prints ONE JSON line on stdout.

The CPU baseline is the float64 oracle (append + attention over the same
host inputs), timed on the host after the GPU measurement.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attention tokens/s + achieved KV HBM GB/s (% of MI355X peak)"
PEAK_HBM_GBPS = 8000.0
DTYPE_NAMES = {"torch.float32": "f32", "torch.float16": "f16", "torch.bfloat16": "bf16",
               "torch.uint8": "fp8_e4m3"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and blank space removed, so
    that a counter record stays valid across comment-only edits."""
    import re
    csrc = os.path.join(ROOT, "paged_kv_cache_440_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            text = open(os.path.join(csrc, f), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(f.encode())
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, partition: int, policy: str):
    """HBM bytes per attention launch from the committed rocprofv3 --pmc
    summary, if it was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_p{partition}_{policy}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


# The schedule each workload is timed with: the faster of the balanced
# schedule and 512-token partitions as measured on MI355X. Balanced wins when
# sequences are long and their lengths spread (few segments per persistent
# wave); fixed partitions win for many short sequences, for sequences that
# share prefix blocks (neighbours run side by side and hit the cache) and for
# the FP8 vector walker. The K/V load policy follows the workload: cached
# loads (kv_reuse) where tables share blocks and the plain decode call reads
# them once per sequence, streaming loads otherwise (the grouped call reads
# shared blocks once per group).
DEFAULT_SCHEDULE = {
    "opt13b_fp16": "balanced",
    "long_gqa_bf16": "balanced",
    "long_gqa_fp8": "balanced",
    "llama13b_bf16": "balanced",
    "shared_prefix_fp16": 1024,          # grouped call (512 for --no-grouped)
    "shared_prefix_cow_fp16": 1024,
    "opt13b_fp8": 512,
    "opt13b_spec4_fp16": "balanced",
    "opt13b_spec4_fp8": "balanced",
    "opt13b_prefill256_fp16": "balanced",   # a single pass per 16-column tile
    "shared_prefix_fp8": 1024,           # grouped call over an FP8 cache
    "shared_prefix_cow_fp8": 1024,
    "tiny_fp32": 512,
}


def pkv_balanced() -> int:
    from paged_kv_cache_440_amd._lib import PARTITION_BALANCED
    return PARTITION_BALANCED


def cpu_baseline(w, min_seconds: float = 10.0):
    """The oracle, as it stands, on the host cores: decode steps over the
    whole batch (the append, then attention), float64 numpy, repeated for
    about min_seconds. The append is one scatter on one thread; attention is
    split over the sequences across a thread pool of the host's cores (at
    most 16, one GPU's share of the box), one BLAS thread each."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    from oracle import (fp8_dequantize_pool, paged_decode_attention, paged_multi_query_attention,
                        pool_after_append, pool_after_append_fp8, pool_after_append_multi,
                        pool_after_append_multi_fp8)

    def bits(t):
        ints = {1: torch.uint8, 2: torch.int16, 4: torch.int32}
        return t.contiguous().view(ints[t.element_size()]).numpy()

    def widen(a):
        t = torch.from_numpy(a).view(w.dtype)
        return t.numpy() if w.dtype == torch.float16 else t.float().numpy()

    q = widen(bits(w.q))
    kb, vb = bits(w.k_pool), bits(w.v_pool)
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    parts = [p for p in np.array_split(np.arange(w.num_seqs), min(w.num_seqs, 4 * workers))
             if p.size]

    def attention(idx, kf, vf):
        fn = paged_multi_query_attention if w.num_queries > 1 else paged_decode_attention
        fn(q[idx], kf, vf, w.block_tables[idx], w.seq_lens[idx], w.block_size, w.scale)

    spent = {"append": 0.0, "attention": 0.0}

    def one_step(ex):
        t_a = time.perf_counter()
        if w.fp8:
            ks, vs = w.k_scales.numpy(), w.v_scales.numpy()
            app = pool_after_append_multi_fp8 if w.num_queries > 1 else pool_after_append_fp8
            k2, v2 = app(kb, vb, w.k_new.float().numpy(), w.v_new.float().numpy(), ks, vs,
                         w.block_tables, w.seq_lens, w.block_size)
            kf, vf = fp8_dequantize_pool(k2, ks), fp8_dequantize_pool(v2, vs)
        else:
            app = pool_after_append_multi if w.num_queries > 1 else pool_after_append
            k2, v2 = app(kb, vb, bits(w.k_new), bits(w.v_new), w.block_tables, w.seq_lens,
                         w.block_size)
            kf, vf = widen(k2), widen(v2)
        t_b = time.perf_counter()
        list(ex.map(lambda idx: attention(idx, kf, vf), parts))
        spent["append"] += t_b - t_a
        spent["attention"] += time.perf_counter() - t_b

    # whole steps until at least min_seconds of oracle work (one step at least)
    with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
        steps = 0
        t0 = time.perf_counter()
        while True:
            one_step(ex)
            steps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    tokens = steps * w.num_seqs * w.num_queries
    attn_rate = tokens / spent["attention"]
    return {"value": tokens / dt, "unit": "tokens/s",
            "cores": workers, "kind": "oracle",
            "attention_only_tokens_per_s": attn_rate,
            "append_s_per_step": spent["append"] / steps,
            "attention_s_per_step": spent["attention"] / steps,
            "sample": f"{steps} whole decode steps of the batch ({w.num_seqs} sequences, all "
                      f"heads: append + attention), float64 numpy; attention over {workers} "
                      f"threads, the append on one; {dt:.1f} s wall, of which the append "
                      f"(the oracle's functional copy of both pools plus the scatter) "
                      f"{spent['append']:.1f} s and attention {spent['attention']:.1f} s: "
                      f"attention alone runs at {attn_rate:.1f} tokens/s"}


def block_manager_bench(steps: int, warmup: int) -> None:
    """Host bookkeeping of one decode step of the shared-prefix workload:
    reserve a slot for each of 256 samples (copy-on-write of the shared
    partial block on the first step), collect the copy pairs and build the
    launch's block tables. The C++ manager (one call each) against the
    oracle's plain Python manager on the same operations."""
    from paged_kv_cache_440_amd.block_manager import BlockManager
    from oracle.block_manager import BlockManagerOracle

    prompts, samples, prefix, bs = 32, 8, 1032, 16
    steps = max(1, min(steps, 200))
    nb = prompts * (prefix // bs + 1) + prompts * samples * (2 + (steps + 1) // bs + 1)
    ids = [p * samples + s + 1 for p in range(prompts) for s in range(samples)]
    max_blocks = (prefix + steps + 2 * bs) // bs + 1

    def setup(mgr):
        for p in range(prompts):
            root = -(p + 1)
            mgr.add_sequence(root)
            for _ in range(prefix):
                mgr.append_token(root)
            for s in range(samples):
                mgr.fork(root, p * samples + s + 1)
            mgr.free_sequence(root)

    def run(step_fn, n):
        t0 = time.perf_counter()
        for _ in range(n):
            step_fn()
        return (time.perf_counter() - t0) / n

    bm = BlockManager(nb, bs)
    setup(bm)
    ids_np = np.asarray(ids, dtype=np.int64)

    def cxx_step():
        bm.append_batch(ids_np)
        bm.take_copies()
        bm.build_batch(ids_np, max_blocks)

    for _ in range(min(warmup, 5)):
        cxx_step()
    cxx = run(cxx_step, steps)

    orc = BlockManagerOracle(nb, bs)
    setup(orc)

    def oracle_step():
        for s in ids:
            orc.append_token(s)
        orc.take_copies()
        tables = np.full((len(ids), max_blocks), -1, dtype=np.int32)
        for i, s in enumerate(ids):
            tables[i, :len(orc.tables[s])] = orc.tables[s]
        np.array([orc.lens[s] for s in ids], dtype=np.int32)

    for _ in range(min(warmup, 5)):
        oracle_step()
    ora = run(oracle_step, steps)
    print(json.dumps({
        "metric": "block manager decode-step bookkeeping (steps/s)", "value": 1.0 / cxx,
        "unit": "steps/s", "us_per_step": cxx * 1e6, "sequences": len(ids), "steps": steps,
        "higher_is_better": True, "data": "synthetic",
        "config": {"workload": "shared_prefix_fp16 bookkeeping", "prompts": prompts,
                   "samples": samples, "prefix": prefix, "block_size": bs},
        "cpu_baseline": {"value": 1.0 / ora, "unit": "steps/s", "cores": 1, "kind": "oracle",
                         "sample": f"the same {steps} steps in the Python oracle manager"},
    }), flush=True)


PEAK_HOST_LINK_GBPS = 64.0      # PCIe 5.0 x16, one direction


def swap_bench(steps: int, warmup: int, with_cpu: bool) -> None:
    """Swap a quarter of the OPT-13B layer's batch (16 of 64 sequences, all
    their blocks) out to a pinned host pool and back in, with pkv_swap_blocks
    (one launch per direction). A step is that round trip. Beside it, one
    contiguous DMA copy (torch copy_) of the same byte count in each
    direction: the practical ceiling of the host link."""
    import torch
    import paged_kv_cache_440_amd as pkv
    from paged_kv_cache_440_amd import workloads as wl

    w = wl.opt13b_fp16()
    preempt = 16
    used = [-(-int(w.seq_lens[i]) // w.block_size) for i in range(preempt)]
    blocks = np.concatenate([w.block_tables[i, :used[i]] for i in range(preempt)]).astype(np.int32)
    n = len(blocks)
    host = np.arange(n, dtype=np.int32)
    dk, dv = w.k_pool.cuda(), w.v_pool.cuda()
    hk = torch.empty((n,) + tuple(dk.shape[1:]), dtype=dk.dtype).pin_memory()
    hv = torch.empty_like(hk).pin_memory()
    out_map = torch.from_numpy(np.stack([blocks, host], 1)).cuda()
    in_map = torch.from_numpy(np.stack([host, blocks], 1)).cuda()
    block_bytes = dk[0].numel() * dk.element_size()
    moved = 2 * n * block_bytes                       # K and V, one direction
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3   # us

    swap_out = lambda: pkv.swap_blocks(dk, dv, hk, hv, out_map, stream=stream)
    swap_in = lambda: pkv.swap_blocks(hk, hv, dk, dv, in_map, stream=stream)
    for _ in range(warmup):
        swap_out()
        swap_in()
    torch.cuda.synchronize()
    steps = max(1, steps)
    t0 = time.perf_counter()
    out_us = timed(swap_out, steps)
    in_us = timed(swap_in, steps)
    wall = time.perf_counter() - t0
    ok = (torch.equal(hk.view(torch.int16).cuda(), dk.view(torch.int16)[blocks.tolist()]) and
          torch.equal(hv.view(torch.int16).cuda(), dv.view(torch.int16)[blocks.tolist()]))
    if not ok:
        raise SystemExit("swap round trip does not reproduce the blocks")
    flat_d = torch.empty(moved, dtype=torch.uint8, device="cuda")
    flat_h = torch.empty(moved, dtype=torch.uint8).pin_memory()
    d2h_us = timed(lambda: flat_h.copy_(flat_d, non_blocking=True), max(3, steps // 4))
    h2d_us = timed(lambda: flat_d.copy_(flat_h, non_blocking=True), max(3, steps // 4))
    gbps = lambda us: moved / us / 1e3
    value = 2 * moved / (out_us + in_us) / 1e3
    log(f"[swap] {n} blocks of {block_bytes} B (K and V): out {out_us:.0f} us "
        f"({gbps(out_us):.1f} GB/s), in {in_us:.0f} us ({gbps(in_us):.1f} GB/s); "
        f"contiguous DMA d2h {gbps(d2h_us):.1f} GB/s, h2d {gbps(h2d_us):.1f} GB/s")
    rec = {
        "metric": "KV block swap throughput, device <-> pinned host (GB/s)", "value": value,
        "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": (out_us + in_us) / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": DTYPE_NAMES[str(dk.dtype)], "data": "synthetic",
        "config": {"workload": "opt13b_fp16 swap of 16 of 64 sequences", "blocks": n,
                   "block_bytes_per_pool": block_bytes, "bytes_per_direction": moved},
        "swap_out_gbps": gbps(out_us), "swap_in_gbps": gbps(in_us),
        "dma_d2h_gbps": gbps(d2h_us), "dma_h2d_gbps": gbps(h2d_us),
        "roofline": {"bound": "host_link", "achieved": value, "peak": PEAK_HOST_LINK_GBPS,
                     "unit": "GB/s", "frac": value / PEAK_HOST_LINK_GBPS, "traffic": None},
        "timed_wall_s": wall,
    }
    if with_cpu:
        from oracle import pool_after_swap
        kp, vp = w.k_pool.view(torch.int16).numpy(), w.v_pool.view(torch.int16).numpy()
        hkn = np.empty((n,) + kp.shape[1:], dtype=np.int16)
        hvn = np.empty_like(hkn)
        pairs_out = np.stack([blocks, host], 1)
        pairs_in = np.stack([host, blocks], 1)
        trips = 0
        t0 = time.perf_counter()
        while True:                    # round trips for about 10 s of host work
            hkn, hvn = pool_after_swap(kp, vp, hkn, hvn, pairs_out)
            pool_after_swap(hkn, hvn, kp, vp, pairs_in)
            trips += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0:
                break
        rec["cpu_baseline"] = {"value": trips * 2 * moved / dt / 1e9, "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{trips} round trips of the same {n} blocks, numpy "
                                         f"block copies on the host, {dt:.1f} s wall"}
    print(json.dumps(rec), flush=True)


def copy_probe(mib: int, reps: int) -> None:
    """pkv_probe_copy over `mib` MiB, `reps` times: each dispatch reads and
    writes exactly mib MiB, the reference for scaling FETCH_SIZE/WRITE_SIZE."""
    import torch
    import paged_kv_cache_440_amd as pkv
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        pkv.probe_copy(dst, src, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    assert torch.equal(dst[:4096], src[:4096])
    print(json.dumps({"probe": "copy", "bytes_read": n, "bytes_written": n, "dispatches": reps,
                      "us_per_dispatch": us, "gbps_read_plus_write": 2 * n / us / 1e3}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="opt13b_fp16")
    ap.add_argument("--block-size", type=int, default=None)
    ap.add_argument("--partition", type=int, default=None,
                    help="0: one pass per sequence; a multiple of 64: fixed partitions; "
                         "-1: balanced (default: the workload's entry in DEFAULT_SCHEDULE)")
    ap.add_argument("--kv-policy", choices=("auto", "stream", "reuse"), default="auto",
                    help="K/V load policy: streaming (non-temporal) or cached loads; auto = "
                         "cached exactly when the workload's tables share blocks")
    ap.add_argument("--no-grouped", action="store_true",
                    help="time parallel-sampling workloads with the plain decode call instead "
                         "of the grouped one (shared prompt blocks read once per group)")
    ap.add_argument("--walker", choices=("auto", "vector"), default="auto",
                    help="vector: grouped query heads on the vector units instead of the matrix "
                         "cores (PKV_WALKER_VECTOR), for comparison")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--block-manager", action="store_true",
                    help="only time the host block manager's decode-step bookkeeping "
                         "(parallel sampling: 32 prompts x 8 samples, 1032-token prefix) "
                         "against the oracle's, and exit (no GPU)")
    ap.add_argument("--swap", action="store_true",
                    help="only time swapping 16 of the OPT-13B layer's 64 sequences out to "
                         "pinned host memory and back in, and exit")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run the plain copy probe over buffers of this many MiB "
                         "(a transfer of known size for scaling traffic counters) and exit")
    args = ap.parse_args()

    if args.block_manager:
        block_manager_bench(args.steps, args.warmup)
        return
    if args.gpus != 1:
        log(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
            "this library has no multi-GPU path.")
        sys.exit(2)

    import torch
    import paged_kv_cache_440_amd as pkv
    from paged_kv_cache_440_amd import workloads as wl

    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib, args.steps)
        return
    if args.swap:
        swap_bench(min(args.steps, 50), min(args.warmup, 5), not args.no_cpu_baseline)
        return

    if args.partition is None:
        args.partition = DEFAULT_SCHEDULE.get(args.workload, 512)
        if args.partition == "balanced":
            args.partition = pkv_balanced()
    kw = {}
    if args.block_size is not None:
        kw["block_size"] = args.block_size
    t0 = time.perf_counter()
    w = wl.make(args.workload, **kw)
    log(f"[bench] workload {w.name}: B={w.num_seqs} H={w.num_heads} Hkv={w.num_kv_heads} "
        f"D={w.head_dim} bs={w.block_size} dtype={w.dtype} KV={w.kv_bytes() / 1e9:.3f} GB "
        f"pool={w.num_blocks} blocks (generated in {time.perf_counter() - t0:.1f} s)")

    dev = torch.device("cuda:0")
    pkv.library()
    kp, vp = w.k_pool.to(dev), w.v_pool.to(dev)
    q = w.q.to(dev)
    k_new, v_new = w.k_new.to(dev), w.v_new.to(dev)
    tables = torch.from_numpy(w.block_tables).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    pairs = torch.from_numpy(np.ascontiguousarray(w.copy_pairs, np.int32)).to(dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    need = pkv.paged_attention_workspace_size(w.num_seqs, w.num_heads * w.num_queries,
                                              w.num_kv_heads, w.head_dim, w.max_seq_len,
                                              args.partition)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    max_len = w.max_seq_len
    stream = torch.cuda.current_stream()
    grouped = "samples" in w.info and not args.no_grouped and args.partition > 0
    # cached loads where tables share blocks that several waves read; the
    # grouped entry reads shared blocks once, so it streams
    auto_reuse = w.shared_blocks and not grouped
    reuse = auto_reuse if args.kv_policy == "auto" else args.kv_policy == "reuse"

    if w.num_queries > 1 and w.fp8:
        ks, vs = w.k_scales.to(dev), w.v_scales.to(dev)

        def attention(stage="both"):
            pkv.paged_attention_multi_fp8(out, q, kp, vp, ks, vs, tables, lens, max_len, w.scale,
                                          partition_size=args.partition, workspace=ws,
                                          stream=stream, kv_reuse=reuse, stage=stage)

        def append():
            pkv.kv_cache_append_multi_fp8(k_new, v_new, kp, vp, ks, vs, tables, lens,
                                          stream=stream)
    elif w.num_queries > 1:
        def attention(stage="both"):
            pkv.paged_attention_multi(out, q, kp, vp, tables, lens, max_len, w.scale,
                                      partition_size=args.partition, workspace=ws, stream=stream,
                                      kv_reuse=reuse, stage=stage)

        def append():
            pkv.kv_cache_append_multi(k_new, v_new, kp, vp, tables, lens, stream=stream)
    elif grouped and w.fp8:
        ks, vs = w.k_scales.to(dev), w.v_scales.to(dev)
        samples = w.info["samples"]
        shared = torch.from_numpy(wl.shared_tokens(w, samples)).to(dev)

        def attention(stage="both"):
            pkv.paged_attention_decode_grouped_fp8(out, q, kp, vp, ks, vs, tables, lens, max_len,
                                                   w.scale, samples, shared,
                                                   partition_size=args.partition, workspace=ws,
                                                   stream=stream, kv_reuse=reuse, stage=stage)

        def append():
            pkv.kv_cache_append_fp8(k_new, v_new, kp, vp, ks, vs, tables, lens, stream=stream)
    elif w.fp8:
        ks, vs = w.k_scales.to(dev), w.v_scales.to(dev)

        def attention(stage="both"):
            pkv.paged_attention_decode_fp8(out, q, kp, vp, ks, vs, tables, lens, max_len, w.scale,
                                           partition_size=args.partition, workspace=ws,
                                           stream=stream, kv_reuse=reuse, stage=stage)

        def append():
            pkv.kv_cache_append_fp8(k_new, v_new, kp, vp, ks, vs, tables, lens, stream=stream)
    elif grouped:
        samples = w.info["samples"]
        shared = torch.from_numpy(wl.shared_tokens(w, samples)).to(dev)

        def attention(stage="both"):
            pkv.paged_attention_decode_grouped(out, q, kp, vp, tables, lens, max_len, w.scale,
                                               samples, shared, partition_size=args.partition,
                                               workspace=ws, stream=stream, kv_reuse=reuse,
                                               stage=stage)

        def append():
            pkv.kv_cache_append(k_new, v_new, kp, vp, tables, lens, stream=stream)
    else:
        def attention(stage="both"):
            pkv.paged_attention_decode(out, q, kp, vp, tables, lens, max_len, w.scale,
                                       partition_size=args.partition, workspace=ws, stream=stream,
                                       kv_reuse=reuse, stage=stage, walker=args.walker)

        def append():
            pkv.kv_cache_append(k_new, v_new, kp, vp, tables, lens, stream=stream)

    entry = ("paged_attention_multi_fp8" if w.num_queries > 1 and w.fp8 else
             "paged_attention_multi" if w.num_queries > 1 else
             "paged_attention_decode_grouped_fp8" if grouped and w.fp8 else
             "paged_attention_decode_fp8" if w.fp8 else
             "paged_attention_decode_grouped" if grouped else
             "paged_attention_decode")

    def step(ev=None):
        pkv.copy_blocks(kp, vp, pairs, stream=stream)
        append()
        if ev is None:
            attention()
            return
        # the same call as its two launches (walk, then merge), with an event
        # between them, so that the dominant kernel is timed on its own
        ev[0].record(stream)
        attention("walk")
        ev[1].record(stream)
        attention("merge")
        ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole-step wall time over K steps
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3

    # the attention call's two launches, bracketed by events on the stream
    # they are launched on: the walk over the K/V blocks (the dominant
    # kernel) and the merge of split segments
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
           for _ in range(args.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    attn_all = np.array([a.elapsed_time(c) for a, b, c in evs])
    attn_ms = float(np.mean(attn_all))
    walk_all = np.array([a.elapsed_time(b) for a, b, c in evs])
    walk_ms = float(np.mean(walk_all))
    merge_ms = float(np.mean([b.elapsed_time(c) for a, b, c in evs]))

    # practical read ceiling: the probe streams both pools once (contiguous
    # 16-byte loads, no compute), timed the same way on the same stream
    pool_bytes = 2 * kp.numel() * kp.element_size()
    sink = torch.empty(pkv.library().pkv_probe_read_sink_words(kp.numel() * kp.element_size()),
                       dtype=torch.int32, device=dev)
    for _ in range(3):
        pkv.probe_read(kp, sink, stream=stream)
        pkv.probe_read(vp, sink, stream=stream)
    rd = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(20)]
    for a, b in rd:
        a.record(stream)
        pkv.probe_read(kp, sink, stream=stream)
        pkv.probe_read(vp, sink, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    read_ceiling = pool_bytes / (float(np.mean([a.elapsed_time(b) for a, b in rd])) * 1e-3) / 1e9

    # ceiling of the paged access pattern itself: the same rows through the
    # same tables with the same loads and split, no compute (best of a sweep
    # of waves per compute unit and loads per round)
    kv_bytes = w.kv_bytes()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    gsink = torch.empty(16 * cus, dtype=torch.int32, device=dev)
    gather = []
    for per_cu in (4, 8, 16):
        for loads in (2, 4, 8):
            run_g = lambda: pkv.probe_gather(kp, vp, tables, lens, per_cu * cus, loads, gsink,
                                             stream=stream)
            for _ in range(2):
                run_g()
            ge = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(10)]
            for a, b in ge:
                a.record(stream)
                run_g()
                b.record(stream)
            torch.cuda.synchronize()
            g_us = float(np.mean([a.elapsed_time(b) for a, b in ge])) * 1e3
            gather.append((kv_bytes / (g_us * 1e-6) / 1e9, per_cu, loads, g_us))
    gather_gbps, g_per_cu, g_loads, g_us = max(gather)
    log(f"[bench] paged gather probe: {gather_gbps:.0f} GB/s ({g_us:.1f} us; {g_per_cu} waves "
        f"per CU, {g_loads} loads of K and of V per round); sweep "
        + ", ".join(f"{c}/{l}: {x:.0f}" for x, c, l, _ in gather))
    # the same rows read with the matrix-core walker's load shapes (K as
    # 16-row operand tiles: 64 bytes of each row per load)
    gather_mfma = []
    for per_cu in (4, 8, 16):
        for chunks in (1, 2):
            run_m = lambda: pkv.probe_gather_mfma(kp, vp, tables, lens, per_cu * cus, chunks, gsink,
                                                  stream=stream)
            for _ in range(2):
                run_m()
            ge = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(10)]
            for a, b in ge:
                a.record(stream)
                run_m()
                b.record(stream)
            torch.cuda.synchronize()
            m_us = float(np.mean([a.elapsed_time(b) for a, b in ge])) * 1e3
            gather_mfma.append((kv_bytes / (m_us * 1e-6) / 1e9, per_cu, chunks, m_us))
    gm_gbps, gm_per_cu, gm_chunks, gm_us = max(gather_mfma)
    log(f"[bench] paged gather probe, matrix-core load shapes: {gm_gbps:.0f} GB/s ({gm_us:.1f} us; "
        f"{gm_per_cu} waves per CU, {gm_chunks} chunks per round); sweep "
        + ", ".join(f"{c}/{l}: {x:.0f}" for x, c, l, _ in gather_mfma))

    unique_bytes = w.unique_kv_bytes()
    # the roofline counts what HBM must deliver, each distinct K/V row once,
    # over the dominant kernel's own time; the whole call is reported beside it
    achieved = unique_bytes / (walk_ms * 1e-3) / 1e9
    logical = kv_bytes / (walk_ms * 1e-3) / 1e9     # shared rows counted per reader
    call_gbps = unique_bytes / (attn_ms * 1e-3) / 1e9
    tokens_per_s = w.num_seqs * w.num_queries / (ms_per_step * 1e-3)
    shared = f" ({logical:.0f} GB/s counting shared rows per reader)" if w.shared_blocks else ""
    log(f"[bench] step {ms_per_step * 1e3:.1f} us, attention {attn_ms * 1e3:.1f} us "
        f"(walk {walk_ms * 1e3:.1f} + merge {merge_ms * 1e3:.1f}), "
        f"{call_gbps:.0f} GB/s of KV over the call = {100 * call_gbps / PEAK_HBM_GBPS:.1f}% of "
        f"8 TB/s, {achieved:.0f} GB/s over the walk = "
        f"{100 * achieved / PEAK_HBM_GBPS:.1f}%{shared}, {tokens_per_s:.0f} tokens/s; read probe "
        f"{read_ceiling:.0f} GB/s ({100 * achieved / read_ceiling:.1f}% of it)")

    traffic = measured_traffic(w.name, args.partition, "reuse" if reuse else "stream")
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the float64 oracle on the host")
        cpu = cpu_baseline(w)
        log(f"[bench] oracle: {cpu['value']:.2f} tokens/s ({cpu['sample']})")

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[str(w.k_pool.dtype)],
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "num_seqs": w.num_seqs,
            "new_tokens_per_seq": w.num_queries,
            "num_heads": w.num_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "seq_len_total": int(w.seq_lens.sum()),
            "max_seq_len": w.max_seq_len,
            "partition_size": args.partition,
            "kv_policy": "reuse" if reuse else "stream",
            "entry": entry,
            "walker": args.walker,
            "kv_bytes_per_step": kv_bytes,
            "unique_kv_bytes_per_step": unique_bytes,
        },
        "attention_us": attn_ms * 1e3,
        "attention_us_median": float(np.median(attn_all)) * 1e3,
        "attention_us_min": float(np.min(attn_all)) * 1e3,
        "walk_kernel_us": walk_ms * 1e3,
        "walk_kernel_us_median": float(np.median(walk_all)) * 1e3,
        "merge_us": merge_ms * 1e3,
        "kv_gbps_call": call_gbps,
        "kv_frac_of_peak_call": call_gbps / PEAK_HBM_GBPS,
        "kv_gbps": achieved,
        "kv_gbps_logical": logical,
        "kv_frac_of_peak": achieved / PEAK_HBM_GBPS,
        "read_probe_gbps": read_ceiling,
        "kv_frac_of_read_probe": achieved / read_ceiling,
        "gather_probe_gbps": gather_gbps,
        "gather_probe_us": g_us,
        "gather_probe_config": {"waves_per_cu": g_per_cu, "loads_per_round": g_loads},
        "walk_frac_of_gather_probe": g_us / (walk_ms * 1e3),
        "gather_mfma_probe_gbps": gm_gbps,
        "gather_mfma_probe_us": gm_us,
        "gather_mfma_probe_config": {"waves_per_cu": gm_per_cu, "chunks_per_round": gm_chunks},
        "walk_frac_of_gather_mfma_probe": gm_us / (walk_ms * 1e3),
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
