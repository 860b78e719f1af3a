"""Host-side KV-cache block engine: free list, reference counts, block tables, copy-on-write.

This is the bookkeeping half of the paged KV cache; the GPU library only ever sees what it
produces (``block_tables``, ``context_lens``, ``slot_mapping`` and copy-on-write pairs).

Behaviour, from the pages:
* The cache is a pool of fixed-size physical blocks shared by all requests; each sequence
  owns a table that maps its logical blocks, in order, to arbitrary physical blocks
  (PyTorch-CUDA-v2.9 PagedAttention page (jsqmd.com), section on giving the KV cache
  paged memory; "GPT-OSS显存管理技巧" (yongjin360.com) §2.2; UltraLAB summary of Kwon et al.
  (xasun.com) §一).
* Blocks are taken on demand and returned when a request ends (xasun.com summary §二, block
  engine item; jsqmd.com page, serving workflow list).
* Sharing between sequences (parallel sampling, beam search, a common prompt prefix) is by
  reference count, with copy-on-write before a shared block is written (xasun.com summary
  §一 and §二, sharing item).

Readings where the pages are loose:
* A decode step appends one token into the next free slot of the sequence's last block and
  takes a new block only when that block is full.  (The jsqmd.com workflow list says each
  new token gets a new page; that contradicts the 16-token page it describes earlier.)
* Copy-on-write copies the whole shared last block into a fresh block; the new token is
  then written into the copy.  Shared blocks that are full are never copied, since appends
  never write into them.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


class PoolExhausted(RuntimeError):
    """No free physical block is left (the trigger for preemption in a serving system)."""


@dataclass
class _Seq:
    table: list = field(default_factory=list)
    length: int = 0


class BlockManager:
    """Free list + reference counts + per-sequence block tables for one KV-cache pool.

    ``seed`` shuffles the free list so that logical blocks land on scattered physical
    blocks, as they do in a pool that has served many requests.
    """

    def __init__(self, num_blocks: int, block_size: int, seed=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = np.arange(self.num_blocks, dtype=np.int64)
        if seed is not None:
            order = np.random.default_rng(seed).permutation(order)
        # pop() takes from the end, so reverse to hand out order[0] first
        self._free = [int(b) for b in order[::-1]]
        self.ref = np.zeros(self.num_blocks, dtype=np.int64)
        self._seqs: dict[int, _Seq] = {}
        self._next_id = 0

    # ---- pool ---------------------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    def _alloc(self) -> int:
        if not self._free:
            raise PoolExhausted(f"all {self.num_blocks} blocks are in use")
        b = self._free.pop()
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        if self.ref[b] <= 0:
            raise RuntimeError(f"block {b} released more often than it was referenced")
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self._free.append(b)

    # ---- sequences ----------------------------------------------------------------------
    def new_sequence(self) -> int:
        sid = self._next_id
        self._next_id += 1
        self._seqs[sid] = _Seq()
        return sid

    def length(self, sid: int) -> int:
        return self._seqs[sid].length

    def table(self, sid: int) -> list:
        return list(self._seqs[sid].table)

    def fork(self, parent: int) -> int:
        """A child that shares every block of ``parent`` (reference counts go up by one)."""
        p = self._seqs[parent]
        sid = self.new_sequence()
        c = self._seqs[sid]
        c.table = list(p.table)
        c.length = p.length
        for b in c.table:
            self.ref[b] += 1
        return sid

    def append_token(self, sid: int):
        """Reserve the slot for one new token of ``sid``.

        Returns ``(slot, cow)`` where ``slot = physical_block * block_size + offset`` and
        ``cow`` is ``(src, dst)`` when the shared last block had to be copied first, else
        ``None``.
        """
        s = self._seqs[sid]
        bs = self.block_size
        off = s.length % bs
        cow = None
        if off == 0:
            b = self._alloc()
            s.table.append(b)
        else:
            b = s.table[-1]
            if self.ref[b] > 1:
                nb = self._alloc()
                self.ref[b] -= 1
                s.table[-1] = nb
                cow = (b, nb)
                b = nb
        s.length += 1
        return b * bs + off, cow

    def append_tokens(self, sid: int, count: int):
        """Append ``count`` tokens; returns the list of slots and copy-on-write pairs."""
        slots, pairs = [], []
        for _ in range(int(count)):
            slot, cow = self.append_token(sid)
            slots.append(slot)
            if cow is not None:
                pairs.append(cow)
        return slots, pairs

    def free_sequence(self, sid: int) -> None:
        s = self._seqs.pop(sid)
        for b in s.table:
            self._release(b)

    # ---- export -------------------------------------------------------------------------
    def block_tables(self, sids, width=None, fill=-1) -> np.ndarray:
        """int32 ``[len(sids), width]``; entries past a sequence's last block hold ``fill``."""
        rows = [self._seqs[s].table for s in sids]
        w = max((len(r) for r in rows), default=0) if width is None else int(width)
        out = np.full((len(rows), max(w, 1)), fill, dtype=np.int64)
        for i, r in enumerate(rows):
            if len(r) > w:
                raise ValueError("table wider than requested width")
            out[i, : len(r)] = r
        return out.astype(np.int32)

    def context_lens(self, sids) -> np.ndarray:
        return np.array([self._seqs[s].length for s in sids], dtype=np.int32)

    def live_blocks(self) -> np.ndarray:
        return np.flatnonzero(self.ref > 0)
