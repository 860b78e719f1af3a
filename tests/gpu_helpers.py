"""Shared pieces of the GPU parity tests: uploading generated cases, running the library
through its binding, the oracle side of a decode step, and the attention tolerance.

Tolerance (for fp16/bf16 inputs with fp32 accumulation): against the float64 oracle rounded
once (nearest-even) to the output type, max |err| <= 2e-3 * max|V| over the V entries the call
reads, and ||err||_2 / ||ref||_2 <= 1e-3 over the whole output.  Rounding a correct result to
bfloat16 alone already moves it by ~1.6e-3 in relative L2, so the comparison is made against
the rounded oracle; the error against the unrounded oracle is reported, not gated.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from paged_kv_cache_05_amd import ops
from paged_kv_cache_05_amd import workloads as W

MAX_ABS_FACTOR = 2e-3
REL_L2_BOUND = 1e-3


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


class Uploaded:
    def __init__(self, case: W.DecodeCase, dev):
        import torch
        dt = case.dtype
        self.case = case
        self.q = W.to_torch(case.query, dt, dev)
        if isinstance(case.key_cache, np.ndarray):
            self.kc = W.to_torch(case.key_cache, dt, dev)
            self.vc = W.to_torch(case.value_cache, dt, dev)
        else:
            self.kc, self.vc = case.key_cache, case.value_cache
        self.bt = torch.from_numpy(np.ascontiguousarray(case.block_tables, np.int32)).to(dev)
        self.cl = torch.from_numpy(np.ascontiguousarray(case.context_lens, np.int32)).to(dev)
        self.nk = W.to_torch(case.new_key, dt, dev)
        self.nv = W.to_torch(case.new_value, dt, dev)
        self.slots = torch.from_numpy(np.ascontiguousarray(case.slot_mapping, np.int64)).to(dev)
        self.pairs = torch.from_numpy(np.ascontiguousarray(case.block_mapping, np.int64).reshape(-1, 2)).to(dev)
        self.out = torch.empty_like(self.q)

    def decode(self, kernel="auto", partition_size=0, shared_blocks=None):
        import torch
        if shared_blocks is None:
            shared_blocks = bool(self.case.spec.shared_prefix)
        ops.decode(self.out, self.q, self.kc, self.vc, self.bt, self.cl, float(self.case.scale),
                   partition_size=partition_size, kernel=kernel, shared_blocks=shared_blocks)
        torch.cuda.synchronize()
        return W.from_torch(self.out, self.case.dtype)

    def step(self, kernel="auto", partition_size=0):
        """copy_blocks -> reshape_and_cache -> decode on one stream."""
        if len(self.case.block_mapping):
            ops.copy_blocks(self.kc, self.vc, self.pairs)
        if len(self.case.slot_mapping):
            ops.reshape_and_cache(self.nk, self.nv, self.kc, self.vc, self.slots)
        return self.decode(kernel, partition_size)


def oracle_decode(case: W.DecodeCase, key_cache=None, value_cache=None, context_lens=None):
    return oracle.decode_ref(case.query, case.key_cache if key_cache is None else key_cache,
                             case.value_cache if value_cache is None else value_cache,
                             case.block_tables,
                             case.context_lens if context_lens is None else context_lens,
                             case.block_size, case.scale, case.dtype)


def oracle_step(case: W.DecodeCase):
    """Oracle for copy_blocks -> reshape_and_cache -> decode on a host-generated case."""
    kc, vc = case.key_cache, case.value_cache
    if len(case.block_mapping):
        kc, vc = oracle.copy_blocks_ref(kc, vc, case.block_mapping)
    if len(case.slot_mapping):
        kc, vc = oracle.reshape_and_cache_ref(case.new_key, case.new_value, kc, vc,
                                              case.slot_mapping, case.block_size)
    return oracle_decode(case, kc, vc), kc, vc


def live_vmax(case: W.DecodeCase, value_cache=None) -> float:
    vc = case.value_cache if value_cache is None else value_cache
    m = 0.0
    for s in range(case.spec.num_seqs):
        n = int(case.context_lens[s])
        if n > 0:
            V = oracle.resolve_sequence(vc, case.block_tables[s], n, case.block_size, case.dtype)
            m = max(m, float(np.max(np.abs(V))))
    return m


def attention_errors(gpu_storage, ref64, dtype):
    ref_r = oracle.storage_to_f64(oracle.f64_to_storage(ref64, dtype), dtype)
    got = oracle.storage_to_f64(gpu_storage, dtype)
    err = got - ref_r
    max_abs = float(np.max(np.abs(err))) if err.size else 0.0
    denom = float(np.linalg.norm(ref_r))
    rel = float(np.linalg.norm(err)) / denom if denom > 0 else float(np.linalg.norm(err))
    rel_unrounded = float(np.linalg.norm(got - ref64)) / max(float(np.linalg.norm(ref64)), 1e-300)
    return max_abs, rel, rel_unrounded


def assert_attention_close(gpu_storage, ref64, dtype, vmax, what=""):
    got = oracle.storage_to_f64(gpu_storage, dtype)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    max_abs, rel, rel_u = attention_errors(gpu_storage, ref64, dtype)
    tol = MAX_ABS_FACTOR * vmax
    say(f"  {what}: max_abs={max_abs:.3e} (tol {tol:.3e}) rel_l2={rel:.3e} (tol {REL_L2_BOUND}) "
        f"rel_l2_vs_unrounded={rel_u:.3e}")
    assert max_abs <= tol, f"{what}: max abs error {max_abs} > {tol}"
    assert rel <= REL_L2_BOUND, f"{what}: relative L2 error {rel} > {REL_L2_BOUND}"
    return max_abs, rel


def bits(storage, dtype):
    a = np.ascontiguousarray(storage)
    return a.view(np.uint32) if dtype == "f32" else a.view(np.uint16)


# ---------------------------------------------------------------------------------------
# full-size parity: every sequence of a GPU-drawn workload against the oracle
# ---------------------------------------------------------------------------------------
def host_threads() -> int:
    """Host cores this process may use (its affinity mask), at most 16 (one GPU's share)."""
    import os
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def snapshot_seq(case: W.DecodeCase, s: int, kc, vc, pool_dtype=None) -> dict:
    """Host copies of every block sequence s reads in this step (and the copy-on-write sources
    of its blocks), renumbered 0.., with the step's table row, copy pairs and slot in that
    numbering.  Taken from the GPU pools ``kc``/``vc``."""
    import torch
    pdt = pool_dtype or case.dtype
    bs = case.block_size
    n = int(case.context_lens[s])
    nb = -(-n // bs)
    row = [int(b) for b in case.block_tables[s, :nb]]
    pairs = [(int(a), int(b)) for a, b in np.asarray(case.block_mapping).reshape(-1, 2) if int(b) in row]
    blocks = sorted(set(row) | {a for a, _ in pairs})
    remap = {b: i for i, b in enumerate(blocks)}
    idx = torch.tensor(blocks, dtype=torch.int64, device=kc.device)
    mk = W.from_torch(kc.index_select(0, idx), pdt)
    mv = W.from_torch(vc.index_select(0, idx), pdt)
    table = np.array([[remap[b] for b in row]], dtype=np.int32)
    mpairs = np.array([[remap[a], remap[b]] for a, b in pairs], dtype=np.int64).reshape(-1, 2)
    # with one appended token per sequence, slot_mapping[s] is sequence s's new token
    own = case.spec.new_tokens == "next" and len(case.slot_mapping) == case.spec.num_seqs
    slot = int(case.slot_mapping[s]) if own else -1
    mslot = np.array([remap[slot // bs] * bs + slot % bs], dtype=np.int64) if slot >= 0 else \
        np.zeros(0, np.int64)
    return dict(s=s, blocks=blocks, mk=mk, mv=mv, table=table, pairs=mpairs, slot=mslot, n=n)


def compare_every_sequence(case: W.DecodeCase, got, kc, vc, snaps, oracle_seq, what,
                           pool_dtype=None, batch=32):
    """The whole GPU output ``got`` ([S, Hq, d] storage) against the oracle, sequence by
    sequence (``oracle_seq(snap) -> (out [Hq, d] float64, pool_k, pool_v, max|V| of the
    sequence)``, run in a thread pool), checked at the attention bar over the whole tensor;
    and, for every sequence, the blocks it reads after the step bit for bit against the
    oracle's pools (every block the step wrote is among them)."""
    import concurrent.futures as cf
    import torch
    from threadpoolctl import threadpool_limits
    pdt = pool_dtype or case.dtype
    S = case.spec.num_seqs
    ref = np.zeros(got.shape, dtype=np.float64)
    vmax = 0.0
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(max_workers=host_threads()) as ex:
        for b0 in range(0, S, batch):
            seqs = range(b0, min(S, b0 + batch))
            futs = {s: ex.submit(oracle_seq, snaps[s]) for s in seqs}
            after = {}
            for s in seqs:      # the GPU pools after the step, the same blocks
                idx = torch.tensor(snaps[s]["blocks"], dtype=torch.int64, device=kc.device)
                after[s] = (W.from_torch(kc.index_select(0, idx), pdt),
                            W.from_torch(vc.index_select(0, idx), pdt))
            for s in seqs:
                out_s, rk, rv, vm = futs[s].result()
                ref[s] = out_s
                vmax = max(vmax, vm)
                ak, av = after[s]
                assert np.array_equal(ak.view(np.uint8), np.ascontiguousarray(rk).view(np.uint8)), \
                    f"{what}: key blocks of sequence {s} differ from the oracle's"
                assert np.array_equal(av.view(np.uint8), np.ascontiguousarray(rv).view(np.uint8)), \
                    f"{what}: value blocks of sequence {s} differ from the oracle's"
            del futs, after
    out_dt = case.dtype
    worst = max(range(S), key=lambda s: float(np.max(np.abs(
        oracle.storage_to_f64(got[s], out_dt) -
        oracle.storage_to_f64(oracle.f64_to_storage(ref[s], out_dt), out_dt)))))
    say(f"  {what}: {S} sequences compared; largest error in sequence {worst} "
        f"(n={int(case.context_lens[worst])})")
    return assert_attention_close(got, ref, out_dt, vmax, f"{what} (all {S} sequences)")


def prefill_every_row(case, got, dev, what, pool_dtype, ref_fn, vmax_fn):
    """Every row of every sequence of a prefill run against the oracle.  Each sequence's blocks
    are copied to the host (``pool_dtype`` storage) and given to ``ref_fn(query rows, keys,
    values, table, query_start_loc, context_lens)`` as a sequence of its own (table 0 .. nb-1);
    sequences run in a pool of host threads.  ``vmax_fn(values)`` gives max|V| for the bar."""
    import concurrent.futures as cf
    import torch
    from threadpoolctl import threadpool_limits
    bs = case.block_size
    ref = np.zeros(got.shape, dtype=np.float64)
    vmax = 0.0

    def one(s, kc, vc):
        n, L = int(case.context_lens[s]), int(case.query_lens[s])
        q0 = int(case.query_start_loc[s])
        table = np.arange(kc.shape[0], dtype=np.int32)[None]
        out = ref_fn(case.query[q0:q0 + L], kc, vc, table, np.array([0, L], np.int32),
                     np.array([n], np.int32))
        return q0, L, out, vmax_fn(vc)

    S = case.spec.num_seqs
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(max_workers=host_threads()) as ex:
        futs = []
        for s in range(S):
            nb = -(-int(case.context_lens[s]) // bs)
            ids = torch.from_numpy(case.pool.block_tables[s, :nb].astype(np.int64)).to(dev)
            kc = W.from_torch(case.pool.key_cache.index_select(0, ids), pool_dtype)
            vc = W.from_torch(case.pool.value_cache.index_select(0, ids), pool_dtype)
            futs.append(ex.submit(one, s, kc, vc))
        for f in futs:
            q0, L, out, vm = f.result()
            ref[q0:q0 + L] = out
            vmax = max(vmax, vm)
    say(f"  {what}: every row of {S} sequences compared")
    return assert_attention_close(got, ref, case.dtype, vmax, f"{what}: every row of {S} sequences")
