#!/usr/bin/env python3
"""Benchmark: one paged-KV decode step on one MI355X, printed as one JSON line.

A step is the whole hot path over one batch: copy_blocks (copy-on-write pairs, none in the
Llama-7B workload) -> reshape_and_cache (one new token per sequence) -> pa_decode (partition
kernel + log-sum-exp merge).  Inputs are seeded synthetic data drawn on the GPU before timing.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload llama7b_bs16]

The reported value is the step's algorithmic bytes divided by the step time (GB/s).  The
`roofline` object covers the dominant kernel (the decode partition kernel), timed with HIP
events on the stream it runs on; `cpu_baseline` times the float64 CPU oracle on a bounded
sample of the same workload.  `detail` adds the other decode workloads (one over an 8-bit
E4M3 cache: pa_reshape_and_cache_fp8 + pa_decode_fp8), swap_blocks over the host link and
pa_prefill on two chunked-prefill workloads (matrix-core bound: TFLOP/s against
the 2.5 PFLOP/s dense bf16 peak).  `--calibrate-copy` instead times copy_blocks on a known
number of bytes (the reference copy used to scale hardware byte counters).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import pathlib
import sys
import time

import numpy as np

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

from paged_kv_cache_05_amd import ops  # noqa: E402
from paged_kv_cache_05_amd import workloads as W  # noqa: E402

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E, AMD's published peak
METRIC = "paged decode attention achieved HBM GB/s (% of MI355X peak) + seq-heads/s"
TRAFFIC_FILE = ROOT / "profiles" / "decode_traffic.json"
KERNEL_SOURCES = {
    "valu": ["pa_decode_valu.h", "pa_decode_valu_bf16.hip", "pa_common.h"],
    "mfma": ["pa_decode_mfma.h", "pa_decode_mfma.hip", "pa_common.h"],
}


def kernel_source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update((ROOT / "paged_kv_cache_05_amd" / "csrc" / f).read_bytes())
    return h.hexdigest()[:16]


def decode_bytes(case) -> int:
    """Algorithmic HBM bytes of one decode call: every live K and V row once, q in, out, the
    table entries read and the context lengths."""
    sp = case.spec
    e = W.ELEM_BYTES[sp.dtype]
    ekv = W.ELEM_BYTES[sp.kv_dtype or sp.dtype]
    n = case.context_lens.astype(np.int64)
    kv = int(n.sum()) * sp.num_kv_heads * sp.head_dim * ekv * 2
    qo = sp.num_seqs * sp.num_heads * sp.head_dim * e * 2
    tables = int((-(-n // sp.block_size)).sum()) * 4 + 4 * sp.num_seqs
    return kv + qo + tables


def decode_unique_kv_bytes(case) -> int:
    """K/V bytes of the distinct (physical block, slot) rows one decode call reads: a block
    that several sequences share (a common prefix) counts once.  Equal to the K/V part of
    decode_bytes when nothing is shared."""
    sp = case.spec
    bs = sp.block_size
    ekv = W.ELEM_BYTES[sp.kv_dtype or sp.dtype]
    rows = {}
    for s in range(sp.num_seqs):
        n = int(case.context_lens[s])
        for j in range(-(-n // bs)):
            b = int(case.block_tables[s, j])
            rows[b] = max(rows.get(b, 0), min(bs, n - j * bs))
    return sum(rows.values()) * sp.num_kv_heads * sp.head_dim * ekv * 2


def cache_write_bytes(case) -> int:
    sp = case.spec
    e = W.ELEM_BYTES[sp.dtype]
    ekv = W.ELEM_BYTES[sp.kv_dtype or sp.dtype]
    row = sp.num_kv_heads * sp.head_dim
    reshape = len(case.slot_mapping) * (row * (e + ekv) * 2 + 8)       # read new K,V; write both
    block = sp.num_kv_heads * sp.block_size * sp.head_dim * ekv
    copy = len(case.block_mapping) * (block * 2 * 2 + 16)               # read+write K and V blocks
    return reshape + copy


def chosen_kernel(case, requested: str) -> str:
    sp = case.spec
    G = sp.num_heads // sp.num_kv_heads
    grouped = sp.dtype in ("f16", "bf16") and sp.head_dim in (64, 80, 128, 256) and G % 4 == 0
    if sp.kv_dtype == "fp8":
        return "mfma_fp8" if grouped else "valu_fp8"
    if requested != "auto":
        return requested
    return "mfma" if grouped else "valu"


class Step:
    def __init__(self, case, dev, kernel="auto"):
        import torch
        self.case = case
        sp = case.spec
        dt = sp.dtype
        self.kernel = kernel
        self.q = W.to_torch(case.query, dt, dev)
        self.kc, self.vc = case.key_cache, case.value_cache
        self.bt = torch.from_numpy(case.block_tables).to(dev)
        self.cl = torch.from_numpy(case.context_lens).to(dev)
        self.nk = W.to_torch(case.new_key, dt, dev)
        self.nv = W.to_torch(case.new_value, dt, dev)
        self.slots = torch.from_numpy(case.slot_mapping).to(dev)
        self.pairs = torch.from_numpy(case.block_mapping.reshape(-1, 2)).to(dev)
        self.out = torch.empty_like(self.q)
        self.P = sp.partition_size
        self.shared = bool(sp.shared_prefix)   # blocks read by several sequences of the call
        self.fp8 = sp.kv_dtype == "fp8"        # 8-bit cache: pool scales as drawn
        self.k_scale = self.v_scale = W.FP8_DRAW_SCALE
        nbytes = ops.workspace_bytes(sp.num_seqs, sp.num_heads, sp.num_kv_heads, sp.head_dim,
                                     sp.block_size, case.max_blocks_per_seq, self.P)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)

    def run(self, ev=None):
        if len(self.case.block_mapping):
            ops.copy_blocks(self.kc, self.vc, self.pairs)
        if self.fp8:
            ops.reshape_and_cache_fp8(self.nk, self.nv, self.kc, self.vc, self.slots,
                                      self.k_scale, self.v_scale)
        else:
            ops.reshape_and_cache(self.nk, self.nv, self.kc, self.vc, self.slots)
        if ev is not None:
            ev[0].record()
        if self.fp8:
            ops.decode_fp8_partitions(self.out, self.q, self.kc, self.vc, self.bt, self.cl,
                                      float(self.case.scale), self.k_scale, self.v_scale, self.ws,
                                      partition_size=self.P, shared_blocks=self.shared)
        else:
            ops.decode_partitions(self.out, self.q, self.kc, self.vc, self.bt, self.cl,
                                  float(self.case.scale), self.ws, partition_size=self.P,
                                  kernel=self.kernel, shared_blocks=self.shared)
        if ev is not None:
            ev[1].record()
        ops.decode_merge(self.out, self.cl, self.case.spec.num_kv_heads, self.case.spec.block_size,
                         self.case.max_blocks_per_seq, self.ws, partition_size=self.P)
        if ev is not None and len(ev) > 2:
            ev[2].record()


def time_steps(step, steps, warmup):
    import torch
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    # per step: before the decode kernel, between it and the merge, after the merge
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        step.run(evs[i])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    kern = [a.elapsed_time(b) for a, b, _ in evs]
    step.last_kernel_ms = kern
    step.last_merge_ms = [b.elapsed_time(c) for _, b, c in evs]
    return total_ms / steps, float(np.mean(kern)), float(np.min(kern)), wall


MALL_BYTES = 256 << 20   # MI355X Infinity Cache
COLD_WORKLOADS = ("tiny", "gqa_long", "shared_prefix")


def time_steps_cold(step, steps):
    """Steps with cold caches: before each one (untimed) a 1 GiB buffer is written, which
    evicts the L2s and the 256 MiB Infinity Cache.  Returns the median step time and the
    median decode-kernel time (ms)."""
    import torch
    dev = step.q.device
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    ev_step, ev_kern = [], []
    for i in range(steps):
        scratch.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        a.record()
        step.run(ev)
        b.record()
        ev_step.append((a, b))
        ev_kern.append(ev)
    torch.cuda.synchronize()
    del scratch
    return (float(np.median([a.elapsed_time(b) for a, b in ev_step])),
            float(np.median([a.elapsed_time(b) for a, b in ev_kern])))


def snapshot_sequences(case, seqs):
    """Host copies of the blocks each given sequence reads in the step (with the copy-on-write
    sources of its blocks), renumbered 0.., taken before any step runs."""
    import torch
    bs = case.block_size
    pdt = case.spec.kv_dtype or case.dtype
    pairs_all = np.asarray(case.block_mapping).reshape(-1, 2)
    own_slot = case.spec.new_tokens == "next" and len(case.slot_mapping) == case.spec.num_seqs
    out = []
    for s in seqs:
        n = int(case.context_lens[s])
        row = [int(b) for b in case.block_tables[s, : -(-n // bs)]]
        pairs = [(int(a), int(b)) for a, b in pairs_all if int(b) in row]
        blocks = sorted(set(row) | {a for a, _ in pairs})
        remap = {b: i for i, b in enumerate(blocks)}
        idx = torch.tensor(blocks, dtype=torch.int64, device=case.key_cache.device)
        slot = int(case.slot_mapping[s]) if own_slot else -1
        out.append(dict(
            s=s, n=n, table=np.array([[remap[b] for b in row]], np.int32),
            pairs=np.array([[remap[a], remap[b]] for a, b in pairs], np.int64).reshape(-1, 2),
            slot=np.array([remap[slot // bs] * bs + slot % bs] if slot >= 0 else [], np.int64),
            mk=W.from_torch(case.key_cache.index_select(0, idx), pdt),
            mv=W.from_torch(case.value_cache.index_select(0, idx), pdt)))
    return out


def host_threads() -> int:
    """Host cores this process may use (its affinity mask), at most 16 (the share of one GPU)."""
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def oracle_inputs(case, snaps):
    """Per snapshotted sequence, the pools the decode reads: the step's copy-on-write pairs and
    its new token applied by the oracle (untimed), with the sequence's renumbered table."""
    import oracle
    bs = case.block_size
    fp8 = case.spec.kv_dtype == "fp8"
    prepared = []
    for sn in snaps:
        mk, mv = sn["mk"], sn["mv"]
        s = sn["s"]
        if len(sn["pairs"]):
            mk, mv = oracle.copy_blocks_ref(mk, mv, sn["pairs"])
        if len(sn["slot"]):
            if fp8:
                mk, mv = oracle.reshape_and_cache_fp8_ref(
                    case.new_key[s:s + 1], case.new_value[s:s + 1], mk, mv, sn["slot"], bs,
                    case.dtype, W.FP8_DRAW_SCALE, W.FP8_DRAW_SCALE)
            else:
                mk, mv = oracle.reshape_and_cache_ref(case.new_key[s:s + 1], case.new_value[s:s + 1],
                                                      mk, mv, sn["slot"], bs)
        prepared.append((s, sn["n"], mk, mv, sn["table"]))
    return prepared


def cpu_baseline(case, prepared, budget_s, threads=1):
    """The float64 oracle decoding the prepared sequences, one decode_ref call per sequence,
    ``threads`` of them at a time in a thread pool (numpy releases the interpreter lock inside
    its array loops and BLAS calls; BLAS itself is held to one thread per worker).  Sequences
    are taken in order, cycling, until at least ``budget_s`` wall seconds and one decode per
    worker are done.  Rates are per wall second."""
    import concurrent.futures as cf
    import oracle
    from threadpoolctl import threadpool_limits
    sp = case.spec
    e = W.ELEM_BYTES[sp.dtype]
    ekv = W.ELEM_BYTES[sp.kv_dtype or sp.dtype]
    fp8 = sp.kv_dtype == "fp8"
    bs = case.block_size

    def one(item):
        s, n, mk, mv, table = item
        if fp8:
            oracle.decode_fp8_ref(case.query[s:s + 1], mk, mv, table, np.array([n], np.int32), bs,
                                  case.scale, case.dtype, W.FP8_DRAW_SCALE, W.FP8_DRAW_SCALE)
        else:
            oracle.decode_ref(case.query[s:s + 1], mk, mv, table, np.array([n], np.int32), bs,
                              case.scale, case.dtype)
        return n

    done, tokens = 0, 0
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        while True:
            batch = [prepared[(done + k) % len(prepared)] for k in range(threads)]
            for n in ex.map(one, batch):
                tokens += n
            done += len(batch)
            elapsed = time.perf_counter() - t0
            if elapsed >= budget_s:
                break
    nbytes = tokens * sp.num_kv_heads * sp.head_dim * ekv * 2 + done * sp.num_heads * sp.head_dim * e * 2
    heads = done * sp.num_heads
    return {"value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seq_heads_per_s": round(heads / elapsed, 2),
            "s_per_call": float(f"{elapsed * sp.num_seqs / done:.4g}"),
            "seconds": round(elapsed, 2),
            "sample": f"{done} sequence decodes taken in order, cycling over the {len(prepared)} "
                      f"sequences of the step ({tokens} cached tokens read, all {sp.num_heads} "
                      f"heads each), numpy float64, {threads} worker thread"
                      f"{'s' if threads > 1 else ''} with one BLAS thread each"}


# CPU-baseline legs: one per workload family, the one-thread leg where it is asked for
CPU_BASELINE_LEGS = {"tiny": False, "opt13b": True, "llama7b_bs16": True, "gqa_long": False,
                     "shared_prefix": False}


def cpu_baseline_leg(case, snaps, budget_s, one_thread):
    """The oracle on the host's cores, and on one thread when ``one_thread``."""
    prepared = oracle_inputs(case, snaps)
    nt = host_threads()
    rec = cpu_baseline(case, prepared, budget_s, nt)
    if one_thread and nt > 1:
        one = cpu_baseline(case, prepared, budget_s, 1)
        rec["one_thread"] = {k: one[k] for k in ("value", "seq_heads_per_s", "s_per_call", "seconds")}
        rec["speedup_vs_one_thread"] = round(rec["value"] / one["value"], 2)
    return rec


def traffic_for(kernel, workload):
    if not TRAFFIC_FILE.exists():
        return None
    rec = json.loads(TRAFFIC_FILE.read_text())
    entry = rec.get(workload, {})
    if entry.get("kernel") != kernel or entry.get("kernel_source_sha") != kernel_source_sha(kernel):
        return None
    return entry.get("hbm_bytes_per_launch")


def copy_ceiling(dev, steps):
    """copy_blocks over 4096 distinct 128 KiB blocks (K and V): 1 GiB read + 1 GiB written per
    launch.  Returns (ms per launch, bytes read per launch); reported as the GPU's achievable
    copy rate, context for the decode's read bandwidth."""
    import torch
    nb, shape = 8192, (8192, 32, 16, 128)
    kc = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    pairs = torch.stack([torch.arange(0, nb // 2), torch.arange(nb // 2, nb)], 1).to(dev)
    for _ in range(2):
        ops.copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        ops.copy_blocks(kc, vc, pairs)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    moved = 2 * (nb // 2) * 32 * 16 * 128 * 2
    del kc, vc
    return ms, moved


def read_ceiling(dev, steps):
    """pa_read_tiles over a 2 GiB buffer of 4 KiB tiles (one (block, KV head) tile of the
    16-token bf16 workloads): the tiles as one contiguous run, then the same tiles in a seeded
    random order (the decode's pattern: whole tiles scattered over the pool).  Nothing but the
    loads and an XOR per tile, so these are the read rates a decode kernel could reach."""
    import torch
    nbytes, tile = 2 << 30, 4096
    ntiles = nbytes // tile
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    out = torch.empty(ntiles, dtype=torch.int32, device=dev)
    g = torch.Generator(device="cpu")
    g.manual_seed(4096)
    ids = torch.randperm(ntiles, generator=g).to(torch.int32).to(dev)
    res = {"what": "pa_read_tiles, 2 GiB of 4 KiB tiles read per launch (16-byte non-temporal loads)"}
    for name, tid in (("contiguous", None), ("scattered_tiles", ids)):
        for _ in range(3):
            ops.read_tiles(buf, tile, out, tid)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record()
            ops.read_tiles(buf, tile, out, tid)
            b.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        res[name] = {"ms": round(ms, 4), "GBps": round(nbytes / ms / 1e6, 1),
                     "frac_of_peak": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)}
    del buf, out, ids
    return res


def calibrate_copy(dev, steps):
    """The copy of copy_ceiling, printed for the HBM-counter calibration runs."""
    ms, moved = copy_ceiling(dev, steps)
    print(json.dumps({"calibration": "copy_blocks", "read_bytes_per_launch": moved,
                      "write_bytes_per_launch": moved, "ms_per_launch": round(ms, 4),
                      "GBps_read_plus_write": round(2 * moved / ms / 1e6, 1)}), flush=True)


def measure_swap(dev, steps):
    """swap_blocks over the host link: 2048 Llama-7B-shaped blocks (32 heads x 16 x 128 bf16,
    K and V: 256 KiB per block) GPU -> pinned host and back."""
    import torch
    nb, shape = 2048, (2048, 32, 16, 128)
    gk = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    gv = torch.zeros_like(gk)
    hk = torch.zeros(shape, dtype=torch.bfloat16).pin_memory()
    hv = torch.zeros(shape, dtype=torch.bfloat16).pin_memory()
    ident = torch.arange(nb, dtype=torch.int64)
    pairs = torch.stack([ident.flip(0), ident], 1).to(dev)
    moved = nb * 2 * 32 * 16 * 128 * 2
    res = {}
    for name, args in (("gpu_to_host", (gk, gv, hk, hv)), ("host_to_gpu", (hk, hv, gk, gv))):
        ops.swap_blocks(*args, pairs)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            ops.swap_blocks(*args, pairs)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        res[name] = {"ms": round(ms, 4), "GBps": round(moved / ms / 1e6, 2), "bytes": moved}
    return res


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix-core peak


def prefill_flops(case) -> float:
    """4 * head_dim flops (two multiply-adds per dim) per (query row, visible key, query head)."""
    L = case.query_lens.astype(np.int64)
    n = case.context_lens.astype(np.int64)
    pairs = int(np.sum(L * (n - L) + L * (L + 1) // 2))
    return 4.0 * case.spec.head_dim * case.spec.num_heads * pairs


def _lengths_str(spec_lengths) -> str:
    if spec_lengths[0] == "fixed" and len(set(spec_lengths[1])) == 1:
        return f"{spec_lengths[1][0]} tokens each"
    return str(spec_lengths)


def measure_prefill(dev, name, steps, warmup):
    """pa_prefill_ex on a chunked-prefill workload (the library's key-split choice, workspace
    allocated once), both probability precisions, timed with HIP events on the launch
    stream."""
    import torch
    case = W.build_prefill_case(W.PREFILL_CONFIGS[name], device=dev)
    sp = case.spec
    q = W.to_torch(case.query, sp.dtype, dev)
    bt = torch.from_numpy(case.pool.block_tables.astype(np.int32)).to(dev)
    qsl = torch.from_numpy(case.query_start_loc).to(dev)
    cl = torch.from_numpy(case.context_lens).to(dev)
    out = torch.empty_like(q)
    flops = prefill_flops(case)
    need = ops.prefill_workspace_bytes(sp.num_seqs, q.shape[0], sp.num_heads, sp.num_kv_heads,
                                       sp.head_dim, sp.block_size, bt.shape[1], case.max_query_len)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    res = {"flops_per_launch": flops, "num_seqs": sp.num_seqs, "num_heads": sp.num_heads,
           "num_kv_heads": sp.num_kv_heads, "chunk": _lengths_str(sp.chunk_lengths),
           "cached_prefix": str(sp.prefix_lengths), "key_split_workspace_bytes": need}
    if sp.kv_dtype == "fp8":
        res["kv_cache"] = "E4M3, both pool scales 1/64"
    for mode, bf16_p in (("p16", False), ("p_bf16", True)):
        def run():
            if sp.kv_dtype == "fp8":
                ops.prefill_fp8(out, q, case.pool.key_cache, case.pool.value_cache, bt, qsl, cl,
                                float(case.scale), case.max_query_len, W.FP8_DRAW_SCALE,
                                W.FP8_DRAW_SCALE, bf16_p=bf16_p, workspace=ws)
            else:
                ops.prefill(out, q, case.pool.key_cache, case.pool.value_cache, bt, qsl, cl,
                            float(case.scale), case.max_query_len, bf16_p=bf16_p, workspace=ws)
        # warm up for at least `warmup` launches and 0.2 s: the first launches after the pools
        # are drawn run ~10% slow (measured), longer than ten 0.5 ms launches last
        t_end = time.perf_counter() + 0.2
        i = 0
        while i < warmup or time.perf_counter() < t_end:
            run()
            i += 1
            if i % 50 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            run()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        tf = flops / (ms * 1e-3) / 1e12
        res[mode] = {"ms": round(ms, 4), "TFLOPs": round(tf, 1),
                     "frac_of_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    del case
    return res


def measure_device_engine(dev, steps, warmup):
    """The shared-prefix step with its bookkeeping on the GPU: pa_append_slots (one token for
    each of the 64 sequences, copy-on-write where a forked sibling shares the last block) ->
    pa_copy_blocks_counted (device pair count) -> reshape_and_cache at the device-made slots ->
    decode.  Reports the append and counted-copy launches and the whole step."""
    import torch
    case = W.build_case(W.CONFIGS["shared_prefix"], device=dev)
    sp = case.spec
    S, NB, bs = sp.num_seqs, case.num_blocks, sp.block_size
    # engine state before the step: the sequences (lengths without the step's token) and their
    # forked siblings; reference counts = table entries naming each block
    lens = case.context_lens.astype(np.int64) - 1
    tables = np.concatenate([case.block_tables, case.sibling_tables]).astype(np.int32)
    ctx = np.concatenate([lens, case.sibling_lens]).astype(np.int32)
    pre = case.block_tables.copy()
    for s in range(S):                       # undo the step's own copy-on-write / new block
        nb_old = -(-int(lens[s]) // bs)
        pre[s, nb_old:] = -1
        if nb_old:
            pre[s, nb_old - 1] = case.sibling_tables[s, nb_old - 1]
    tables[:S] = pre
    refs = np.zeros(NB, np.int64)
    for row, n in zip(tables, ctx):
        for b in row[: -(-int(n) // bs)]:
            refs[b] += 1
    free = np.flatnonzero(refs == 0).astype(np.int32)
    stack = np.zeros(NB, np.int32)
    stack[: len(free)] = free
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    d0 = [t(tables), t(ctx), t(refs), t(stack), t(np.array([len(free)]))]
    seqs = t(np.arange(S))
    slots = torch.empty(S, dtype=torch.int64, device=dev)
    pairs = torch.empty((S, 2), dtype=torch.int64, device=dev)
    npairs = torch.empty(1, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    nk, nv = W.to_torch(case.new_key, sp.dtype, dev), W.to_torch(case.new_value, sp.dtype, dev)
    q = W.to_torch(case.query, sp.dtype, dev)
    out = torch.empty_like(q)
    maxb = tables.shape[1]
    ws = torch.empty(max(256, ops.workspace_bytes(S, sp.num_heads, sp.num_kv_heads, sp.head_dim, bs,
                                                  maxb, 0)), dtype=torch.uint8, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(warmup + steps):
        d = [x.clone() for x in d0]          # every step starts from the same state
        e = ev[i - warmup] if i >= warmup else None
        if e:
            e[0].record()
        ops.append_slots(*d, seqs, bs, slots, pairs, npairs, status)
        if e:
            e[1].record()
        ops.copy_blocks_counted(case.key_cache, case.value_cache, pairs, npairs, S)
        if e:
            e[2].record()
        ops.reshape_and_cache(nk, nv, case.key_cache, case.value_cache, slots)
        ops.decode(out, q, case.key_cache, case.value_cache, d[0][:S], d[1][:S],
                   float(case.scale), shared_blocks=True, workspace=ws)
        if e:
            e[3].record()
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError(f"device append failed with status {int(status.item())}")
    med = lambda a, b: float(np.median([x[a].elapsed_time(x[b]) for x in ev]))
    return {"append_slots_us": round(1e3 * med(0, 1), 2),
            "copy_blocks_counted_us": round(1e3 * med(1, 2), 2),
            "step_ms": round(med(0, 3), 4), "copy_pairs": int(npairs.item()),
            "sequences": S}


def run_workload(name, dev, steps, warmup, kernel, snap=False):
    """Build the workload on the GPU and time its steps.  With ``snap`` the blocks every
    sequence reads are copied to the host first (for the CPU baseline); returned as case.snaps."""
    import torch
    case = W.build_case(W.CONFIGS[name], device=dev)
    torch.cuda.synchronize()
    case.snaps = snapshot_sequences(case, range(case.spec.num_seqs)) if snap else None
    step = Step(case, dev, kernel)
    ms, kern_ms, kern_min, wall = time_steps(step, steps, warmup)
    return case, step, ms, kern_ms, kern_min, wall


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama7b_bs16", choices=sorted(W.CONFIGS))
    ap.add_argument("--also", default="llama7b_bs32,llama7b_bs8,opt13b,gqa_long,shared_prefix,llama7b_bs16_fp8,gqa_long_fp8,"
                                      "gqa_long_d80,gqa_long_fp8_d80,tiny",
                    help="comma-separated extra workloads timed for the detail field ('' for none)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--cpu-seconds", type=float, default=3.0,
                    help="wall seconds of each CPU-baseline leg (per workload and thread count)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--only", default="",
                    help="time only these detail legs (comma-separated: a decode workload, "
                         "prefill_llama7b, prefill_gqa, prefill_llama7b_fp8, prefill_gptoss_d64, "
                         "prefill_d80, "
                         "swap_blocks, "
                         "device_engine, read_ceiling) "
                         "and print them")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the paged decode step runs on a single MI355X and "
              f"has no multi-GPU path (asked for --gpus {args.gpus}, WORLD_SIZE {world}).",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    ops.load()
    if args.calibrate_copy:
        calibrate_copy(dev, args.steps)
        return 0
    if args.only:
        res = {}
        for leg in [x for x in args.only.split(",") if x]:
            if leg in W.PREFILL_CONFIGS:
                res[leg] = measure_prefill(dev, leg, args.steps, args.warmup)
            elif leg == "swap_blocks":
                res[leg] = measure_swap(dev, args.steps)
            elif leg == "device_engine":
                res[leg] = measure_device_engine(dev, args.steps, args.warmup)
            elif leg == "read_ceiling":
                res[leg] = read_ceiling(dev, args.steps)
            elif leg in W.CONFIGS:
                c2, st2, ms2, k2, _, _ = run_workload(leg, dev, args.steps, args.warmup, args.kernel)
                res[leg] = {"ms_per_step": round(ms2, 4), "decode_kernel_ms": round(k2, 4),
                            "decode_kernel_GBps": round(decode_bytes(c2) / (k2 * 1e-3) / 1e9, 2),
                            "seq_heads_per_s": round(c2.spec.num_seqs * c2.spec.num_heads / (ms2 * 1e-3), 1),
                            "kernel": chosen_kernel(c2, args.kernel)}
                if c2.spec.shared_prefix:
                    ub = decode_unique_kv_bytes(c2)
                    res[leg]["unique_kv_bytes"] = ub
                    res[leg]["decode_kernel_unique_GBps"] = round(ub / (k2 * 1e-3) / 1e9, 2)
                del c2, st2
            else:
                print(f"unknown leg {leg!r}", file=sys.stderr)
                return 2
            torch.cuda.empty_cache()
        print(json.dumps({"only": res}), flush=True)
        return 0

    name = args.workload
    want_cpu = lambda w: not args.no_cpu_baseline and w in CPU_BASELINE_LEGS
    cpu_legs = {}
    case, step, ms, kern_ms, kern_min, wall = run_workload(name, dev, args.steps, args.warmup,
                                                           args.kernel, snap=want_cpu(name))
    sp = case.spec
    dbytes = decode_bytes(case)
    sbytes = dbytes + cache_write_bytes(case)
    kernel = chosen_kernel(case, args.kernel)
    achieved = dbytes / (kern_ms * 1e-3) / 1e9
    value = sbytes / (ms * 1e-3) / 1e9
    P = sp.partition_size or ops.auto_partition(sp.num_seqs, sp.num_heads, sp.num_kv_heads,
                                                sp.head_dim, sp.block_size, case.max_blocks_per_seq)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sp.dtype,
        "data": "synthetic (seeded N(0,1) K/V/q on the GPU; lengths and placement per workload)",
        "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "seq_heads_per_s": round(sp.num_seqs * sp.num_heads / (ms * 1e-3), 1),
        "config": {
            "workload": name, "num_seqs": sp.num_seqs, "num_heads": sp.num_heads,
            "num_kv_heads": sp.num_kv_heads, "head_dim": sp.head_dim, "block_size": sp.block_size,
            "num_blocks": case.num_blocks, "context_lens": str(sp.lengths),
            "mean_context": round(float(case.context_lens.mean()), 1),
            "max_context": int(case.context_lens.max()), "partition": P, "kernel": kernel,
            "step_bytes": sbytes, "decode_bytes": dbytes,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic_for(kernel, name),
            "kernel": f"decode_{kernel}_kernel", "avg_launch_ms": round(kern_ms, 4),
            "min_launch_ms": round(kern_min, 4),
            "median_launch_ms": round(float(np.median(step.last_kernel_ms)), 4),
            "algorithmic_bytes_per_launch": dbytes,
        },
        # the split-KV merge launch that follows the decode kernel in each step (it exits at
        # once for sequences held in one partition)
        "merge_kernel_ms": round(float(np.mean(step.last_merge_ms)), 4),
    }
    if case.snaps is not None:
        cpu_legs[name] = cpu_baseline_leg(case, case.snaps, args.cpu_seconds, CPU_BASELINE_LEGS[name])
        case.snaps = None
    detail = {}
    for extra in [x for x in args.also.split(",") if x and x != name]:
        del step
        torch.cuda.empty_cache()
        c2, step, ms2, k2, k2min, _ = run_workload(extra, dev, args.steps, args.warmup, args.kernel,
                                                   snap=want_cpu(extra))
        b2 = decode_bytes(c2)
        detail[extra] = {"ms_per_step": round(ms2, 4),
                         "GBps_step": round((b2 + cache_write_bytes(c2)) / (ms2 * 1e-3) / 1e9, 2),
                         "decode_kernel_ms": round(k2, 4),
                         "decode_kernel_GBps": round(b2 / (k2 * 1e-3) / 1e9, 2),
                         "seq_heads_per_s": round(c2.spec.num_seqs * c2.spec.num_heads / (ms2 * 1e-3), 1),
                         "kernel": chosen_kernel(c2, args.kernel)}
        detail[extra]["decode_kernel_median_ms"] = round(float(np.median(step.last_kernel_ms)), 4)
        detail[extra]["merge_kernel_ms"] = round(float(np.mean(step.last_merge_ms)), 4)
        ub = decode_unique_kv_bytes(c2)
        if c2.spec.shared_prefix:
            detail[extra]["unique_kv_bytes"] = ub
            detail[extra]["decode_kernel_unique_GBps"] = round(ub / (k2 * 1e-3) / 1e9, 2)
        # workloads that fit the caches, and the small-batch ones (tiny, GQA long, shared
        # prefix), are also timed with cold caches
        if ub < 4 * MALL_BYTES or extra in COLD_WORKLOADS:
            cms, ck = time_steps_cold(step, args.steps)
            detail[extra]["cold"] = {"ms_per_step": round(cms, 4), "decode_kernel_ms": round(ck, 4),
                                     "decode_kernel_GBps": round(b2 / (ck * 1e-3) / 1e9, 2),
                                     "note": "median; 1 GiB written before each step"}
        if c2.snaps is not None:
            cpu_legs[extra] = cpu_baseline_leg(c2, c2.snaps, args.cpu_seconds, CPU_BASELINE_LEGS[extra])
            c2.snaps = None
        del c2
    if detail:
        del step
        torch.cuda.empty_cache()
        detail["swap_blocks"] = measure_swap(dev, max(3, args.steps // 4))
        torch.cuda.empty_cache()
        cms, cmoved = copy_ceiling(dev, max(3, args.steps // 2))
        detail["copy_ceiling"] = {"what": "copy_blocks, 1 GiB read + 1 GiB written per launch",
                                  "ms": round(cms, 4),
                                  "GBps_read_plus_write": round(2 * cmoved / cms / 1e6, 1)}
        torch.cuda.empty_cache()
        detail["read_ceiling"] = read_ceiling(dev, max(5, args.steps // 2))
        torch.cuda.empty_cache()
        for pname in ("prefill_llama7b", "prefill_gqa", "prefill_llama7b_fp8", "prefill_gptoss_d64",
                      "prefill_d80"):
            detail[pname] = measure_prefill(dev, pname, args.steps, args.warmup)
        torch.cuda.empty_cache()
        detail["shared_prefix_device_engine"] = measure_device_engine(dev, args.steps, args.warmup)
        rec["detail"] = detail
    if cpu_legs:
        # the headline workload's leg on top, every workload's leg under per_config
        head = cpu_legs.get(name) or next(iter(cpu_legs.values()))
        rec["cpu_baseline"] = dict(head)
        rec["cpu_baseline"]["workload"] = name if name in cpu_legs else next(iter(cpu_legs))
        rec["cpu_baseline"]["per_config"] = cpu_legs
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
