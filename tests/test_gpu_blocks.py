"""GPU parity of the device block engine (pa_append_slots, pa_fork_seqs, pa_free_seqs,
pa_copy_blocks_counted) and of pa_block_hashes, through the C ABI.

Appends run in parallel with atomics, so which free block a sequence receives and which sharer
keeps a shared block may differ from the oracle's one-at-a-time order.  What is unique is
compared exactly (status, lengths, the free-stack top and the set of blocks taken, reference
counts of every block not taken, the number of copies of each shared block); the rest is
checked for validity (counts equal table references, free list and used blocks partition the
pool, every sequence reads its old tokens plus its new one in a block it alone holds).  Fork,
free (as sets) and the hashes are deterministic and compared exactly.  The end-to-end step
(fork -> append -> counted copy -> reshape_and_cache -> decode) is compared on its decode
output, which does not depend on placement."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle_pins
from gpu_helpers import assert_attention_close, need_gpu, say
from paged_kv_cache_05_amd import ops
from paged_kv_cache_05_amd import workloads as W

pytestmark = pytest.mark.gpu


def _dev_state(state, dev):
    import torch
    tables, ctx, refs, stack, top = state
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    return [t(tables), t(ctx), t(refs), t(stack), t(np.array([top], np.int32))]


def _host(ts):
    return [x.cpu().numpy() for x in ts]


def _validate_append(before, after, slots, pairs, seqs, bs, want):
    """Compare a parallel append with the oracle's sequential one (see module docstring)."""
    tables, ctx, refs, stack, top = before
    gt, gc, gr, gs, gtop = after
    wt, wc, wr, ws, wtop, wslots, wpairs, wstatus = want
    assert np.array_equal(gc, wc), "lengths"
    assert int(gtop) == int(wtop), "free-stack top"
    assert np.array_equal(gs, stack), "the stack array is only read"
    taken = set(stack[int(wtop):int(top)].tolist())
    oracle_pins._check_engine(gt, gc, gr, gs, int(gtop), bs)
    for b in range(len(refs)):
        if b not in taken:
            assert gr[b] == wr[b], f"refs[{b}]"
    assert len(pairs) == len(wpairs)
    for b in set(wpairs[:, 0].tolist()) if len(wpairs) else set():
        assert np.sum(pairs[:, 0] == b) == np.sum(wpairs[:, 0] == b), f"copies of {b}"
    new_blocks = [int(b) for b in pairs[:, 1]]
    label = {}
    for s in range(len(ctx)):
        for t in range(int(ctx[s])):
            k = (int(tables[s, t // bs]), t % bs)
            label[k] = k
    model = dict(label)
    for a, b in pairs:
        for o in range(bs):
            if (int(a), o) in label:
                model[(int(b), o)] = label[(int(a), o)]
    for i, s in enumerate(seqs):
        n = int(ctx[s])
        if slots[i] < 0:
            assert gc[s] == n
            continue
        blk = int(gt[s, n // bs])
        assert slots[i] == blk * bs + n % bs, "slot"
        assert gr[blk] == 1, "the written block is private"
        if n % bs == 0 or blk != int(tables[s, n // bs]):
            assert blk in taken, "a fresh block comes from the free stack"
        old = [label[(int(tables[s, t // bs]), t % bs)] for t in range(n)]
        got = [model.get((int(gt[s, t // bs]), t % bs)) for t in range(n)]
        assert got == old, f"sequence {s} lost a token"
    assert len(set(new_blocks)) == len(new_blocks) and set(new_blocks) <= taken


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_append_slots_parallel_matches_sequential(seed):
    import torch
    dev = need_gpu()
    bs = 4
    state = oracle_pins._engine_state(oracle, seed=seed)
    tables, ctx, refs, stack, top = state
    rng = np.random.default_rng(50 + seed)
    seqs = rng.permutation(len(ctx))[: len(ctx) - 1].astype(np.int32)
    say(f"append seed={seed}: {len(seqs)} sequences, free {top}")
    want = oracle.append_slots_ref(tables, ctx, refs, stack, top, seqs, bs)
    d = _dev_state(state, dev)
    slots = torch.full((len(seqs),), -7, dtype=torch.int64, device=dev)
    pairs = torch.full((len(seqs), 2), -7, dtype=torch.int64, device=dev)
    npairs = torch.full((1,), -7, dtype=torch.int32, device=dev)
    status = torch.full((1,), -7, dtype=torch.int32, device=dev)
    ops.append_slots(*d, torch.from_numpy(seqs).to(dev), bs, slots, pairs, npairs, status)
    torch.cuda.synchronize()
    gt, gc, gr, gs, gtop = _host(d)
    k = int(npairs.item())
    assert int(status.item()) == want[7] == 0
    _validate_append(state, (gt, gc, gr, gs, int(gtop[0])), slots.cpu().numpy(),
                     pairs.cpu().numpy()[:k], seqs, bs, want)


def test_append_slots_out_of_blocks_and_full_tables():
    """Three free blocks for five sequences that each need one: exactly three append, two keep
    their state with slot -1, status 1; a full table gives status 2."""
    import torch
    dev = need_gpu()
    bs = 4
    tables = np.array([[0, -1], [1, -1], [2, -1], [3, -1], [4, -1], [5, 6]], np.int32)
    ctx = np.array([4, 4, 4, 4, 4, 8], np.int32)
    refs = np.zeros(12, np.int32)
    refs[:7] = 1
    stack = np.array([9, 11, 10, 7, 8, 0, 0, 0, 0, 0, 0, 0], np.int32)
    top = 3
    d = _dev_state((tables, ctx, refs, stack, top), dev)
    seqs = np.arange(5, dtype=np.int32)
    slots = torch.empty(5, dtype=torch.int64, device=dev)
    pairs = torch.empty((5, 2), dtype=torch.int64, device=dev)
    npairs = torch.empty(1, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    ops.append_slots(*d, torch.from_numpy(seqs).to(dev), bs, slots, pairs, npairs, status)
    torch.cuda.synchronize()
    gt, gc, gr, gs, gtop = _host(d)
    sl = slots.cpu().numpy()
    assert int(status.item()) == 1 and int(gtop[0]) == 0 and int(npairs.item()) == 0
    ok = sl >= 0
    assert ok.sum() == 3
    assert sorted(gt[seqs[ok], 1].tolist()) == [9, 10, 11]
    assert np.all(gc[seqs[ok]] == 5) and np.all(gc[seqs[~ok]] == 4)
    assert np.all(gt[seqs[~ok], 1] == -1)
    ops.append_slots(*d, torch.tensor([5], dtype=torch.int32, device=dev), bs, slots, pairs,
                     npairs, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 2 and int(slots[0].item()) == -1


def test_fork_and_free_match_oracle():
    import torch
    dev = need_gpu()
    bs = 4
    state = oracle_pins._engine_state(oracle, seed=11)
    tables, ctx, refs, stack, top = state
    d = _dev_state(state, dev)
    # fork sequence 2 into row 9 (rows 5..8 already hold forks)
    assert ctx[9] == 0
    pc = np.array([[2, 9]], np.int32)
    ops.fork_seqs(d[0], d[1], d[2], torch.from_numpy(pc).to(dev), bs)
    torch.cuda.synchronize()
    wt, wc, wr = oracle.fork_ref(tables, ctx, refs, pc, bs)
    gt, gc, gr, _, _ = _host(d)
    assert np.array_equal(gc, wc) and np.array_equal(gr, wr)
    for s in range(len(ctx)):
        nb = -(-int(wc[s]) // bs)
        assert np.array_equal(gt[s, :nb], wt[s, :nb])
    # free a forked child and two originals
    ids = np.array([9, 0, 3], np.int32)
    ops.free_seqs(*d, torch.from_numpy(ids).to(dev), bs)
    torch.cuda.synchronize()
    ft, fc, fr, fs, ftop = oracle.free_seqs_ref(wt, wc, wr, stack, top, ids, bs)
    gt, gc, gr, gs, gtop = _host(d)
    assert np.array_equal(gc, fc) and np.array_equal(gr, fr) and int(gtop[0]) == ftop
    assert np.array_equal(gs[:top], fs[:top])
    assert sorted(gs[top:ftop].tolist()) == sorted(fs[top:ftop].tolist())
    assert all(np.all(gt[s, : -(-int(wc[s]) // bs)] == -1) for s in ids)
    oracle_pins._check_engine(gt, gc, gr, gs, int(gtop[0]), bs)


def test_block_hashes_match_oracle():
    import torch
    dev = need_gpu()
    rng = np.random.default_rng(3)
    for bs, T in ((16, 1000), (4, 64), (128, 2048)):
        S = 7
        tok = rng.integers(-2**31, 2**31 - 1, size=(S, T), dtype=np.int64).astype(np.int32)
        tok[1, :T // 2] = tok[0, :T // 2]                      # a shared prefix
        lens = np.array([T, T, T - 1, 0, bs - 1, bs, 3 * bs + 1], np.int32)
        want = oracle.block_hashes_ref(tok, lens, bs)
        h = torch.full((S, T // bs), -1, dtype=torch.int64, device=dev)
        ops.block_hashes(torch.from_numpy(tok).to(dev), torch.from_numpy(lens).to(dev), bs, h)
        torch.cuda.synchronize()
        got = h.cpu().numpy().view(np.uint64)
        say(f"hashes bs={bs} T={T}")
        assert np.array_equal(got, want)
        shared = (T // 2) // bs
        assert np.array_equal(got[0, :shared], got[1, :shared])


def test_device_step_fork_append_copy_decode():
    """A parallel-sampling step kept on the GPU: fork every sequence, append one token to each
    original through pa_append_slots, copy the recorded pairs with the device count, write the
    new tokens at the device-made slots, decode.  The decode output equals the oracle's chain
    (its own placement), since decode does not depend on where blocks sit."""
    import torch
    dev = need_gpu()
    S, Hq, Hkv, D, bs, NB, maxb = 6, 8, 2, 128, 16, 64, 8
    rng = np.random.default_rng(21)
    lens = np.array([1, 15, 16, 17, 40, 100], np.int32)
    tables = np.full((2 * S, maxb), -1, np.int32)
    ctx = np.zeros(2 * S, np.int32)
    refs = np.zeros(NB, np.int32)
    stack = rng.permutation(NB).astype(np.int32)
    top = NB
    for s in range(S):                                     # grow the originals on the host oracle
        for _ in range(int(lens[s])):
            tables, ctx, refs, stack, top, _, _, _ = oracle.append_slots_ref(
                tables, ctx, refs, stack, top, [s], bs)
    pc = np.stack([np.arange(S), np.arange(S) + S], 1).astype(np.int32)
    kc = W.round_to_storage(rng.standard_normal((NB, Hkv, bs, D)).astype(np.float32), "bf16")
    vc = W.round_to_storage(rng.standard_normal((NB, Hkv, bs, D)).astype(np.float32), "bf16")
    q = W.round_to_storage(rng.standard_normal((S, Hq, D)).astype(np.float32), "bf16")
    nk = W.round_to_storage(rng.standard_normal((S, Hkv, D)).astype(np.float32), "bf16")
    nv = W.round_to_storage(rng.standard_normal((S, Hkv, D)).astype(np.float32), "bf16")
    seqs = np.arange(S, dtype=np.int32)
    # oracle chain
    t1, c1, r1 = oracle.fork_ref(tables, ctx, refs, pc, bs)
    t2, c2, r2, s2, top2, oslots, opairs, st = oracle.append_slots_ref(t1, c1, r1, stack, top, seqs, bs)
    k2, v2 = oracle.copy_blocks_ref(kc, vc, opairs)
    k3, v3 = oracle.reshape_and_cache_ref(nk, nv, k2, v2, oslots, bs)
    want = oracle.decode_ref(q, k3, v3, t2[:S], c2[:S], bs, np.float32(D ** -0.5), "bf16")
    # device chain
    d = _dev_state((tables, ctx, refs, stack, top), dev)
    ops.fork_seqs(d[0], d[1], d[2], torch.from_numpy(pc).to(dev), bs)
    slots = torch.empty(S, dtype=torch.int64, device=dev)
    pairs = torch.empty((S, 2), dtype=torch.int64, device=dev)
    npairs = torch.empty(1, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    ops.append_slots(*d, torch.from_numpy(seqs).to(dev), bs, slots, pairs, npairs, status)
    gk, gv = W.to_torch(kc, "bf16", dev), W.to_torch(vc, "bf16", dev)
    ops.copy_blocks_counted(gk, gv, pairs, npairs, S)
    ops.reshape_and_cache(W.to_torch(nk, "bf16", dev), W.to_torch(nv, "bf16", dev), gk, gv, slots)
    gq = W.to_torch(q, "bf16", dev)
    out = torch.empty_like(gq)
    ops.decode(out, gq, gk, gv, d[0][:S].contiguous(), d[1][:S].contiguous(), D ** -0.5)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and int(npairs.item()) == len(opairs)
    vmax = float(np.max(np.abs(oracle.storage_to_f64(v3, "bf16"))))
    assert_attention_close(W.from_torch(out, "bf16"), want, "bf16", vmax, "device step")
    # the forked siblings still read their old tokens only
    sib = oracle.decode_ref(q, k3, v3, t2[S:], c2[S:], bs, np.float32(D ** -0.5), "bf16")
    ops.decode(out, gq, gk, gv, d[0][S:].contiguous(), d[1][S:].contiguous(), D ** -0.5)
    torch.cuda.synchronize()
    assert_attention_close(W.from_torch(out, "bf16"), sib, "bf16", vmax, "siblings")


def _outcome(ctx_before, tables_before, slots, ctx_after, refs_after, status, seqs, bs, shared):
    """What a parallel or sequential append decided, independent of which free block each
    copy received: per appender 'fail', 'in place' or 'copy'; the lengths; the status; the
    reference counts of the shared blocks."""
    kinds = []
    for i, s in enumerate(seqs):
        n = int(ctx_before[s])
        if slots[i] < 0:
            kinds.append("fail")
        elif int(slots[i]) // bs == int(tables_before[s, n // bs]):
            kinds.append("in place")
        else:
            kinds.append("copy")
    return (tuple(kinds), tuple(int(x) for x in ctx_after), int(status),
            tuple(int(refs_after[b]) for b in shared))


# (sharers of each shared partial block, free blocks): a block shared by k sequences that all
# append is copied min(k - 1, free) times in any one-at-a-time order, and its last holder writes
# in place only when every other sharer got a copy
EXHAUSTED = [((2,), 0), ((2,), 1), ((4,), 1), ((4,), 2), ((3, 2), 1), ((3, 2), 2), ((2, 2, 2), 2)]


@pytest.mark.parametrize("sharers,free", EXHAUSTED)
def test_append_shared_blocks_with_too_few_free(sharers, free):
    """Sequences sharing partly filled last blocks (as after parallel-sampling forks) all append
    while the free stack holds fewer blocks than the copies would need.  Repeated 100 times from
    the same state, every parallel outcome must be one that appending the sequences one at a
    time, in some order, produces (all orders are enumerated with the oracle): a sequence may
    write in place only once no other sequence still holds its block."""
    import itertools
    import torch
    dev = need_gpu()
    bs = 4
    tables, ctx, shared = [], [], []
    NB = len(sharers) + free                   # the shared blocks and the free ones
    for b, k in enumerate(sharers):
        shared.append(b)
        for _ in range(k):
            tables.append([b, -1])
            ctx.append(2)                     # two tokens in the shared block
    tables = np.array(tables, np.int32)
    ctx = np.array(ctx, np.int32)
    refs = np.zeros(NB, np.int32)
    for b, k in enumerate(sharers):
        refs[b] = k
    stack = np.zeros(NB, np.int32)
    stack[:free] = np.arange(len(sharers), NB, dtype=np.int32)
    top = free
    S = len(ctx)
    seqs = np.arange(S, dtype=np.int32)
    allowed = set()
    for order in itertools.permutations(range(S)):
        w = oracle.append_slots_ref(tables, ctx, refs, stack, top, np.array(order, np.int32), bs)
        wslots = np.full(S, -1, np.int64)
        for pos, s in enumerate(order):
            wslots[s] = w[5][pos]
        allowed.add(_outcome(ctx, tables, wslots, w[1], w[2], w[7], seqs, bs, shared))
    say(f"shared {sharers}, free {free}: {len(allowed)} sequential outcomes")
    seen = set()
    for rep in range(100):
        d = _dev_state((tables, ctx, refs, stack, top), dev)
        slots = torch.full((S,), -7, dtype=torch.int64, device=dev)
        pairs = torch.full((S, 2), -7, dtype=torch.int64, device=dev)
        npairs = torch.zeros(1, dtype=torch.int32, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        ops.append_slots(*d, torch.from_numpy(seqs).to(dev), bs, slots, pairs, npairs, status)
        torch.cuda.synchronize()
        gt, gc, gr, gs, gtop = _host(d)
        got = _outcome(ctx, tables, slots.cpu().numpy(), gc, gr, int(status.item()), seqs, bs, shared)
        assert got in allowed, (rep, got, allowed)
        seen.add(got)
        k = int(npairs.item())
        assert k == sum(1 for x in got[0] if x == "copy")
        assert int(gtop[0]) == top - k
    say(f"  parallel outcomes seen: {len(seen)}")
