"""CPU oracle for the paged KV-cache block manager -- TEST INFRASTRUCTURE ONLY.

Only the test suite may import this module; the product path never does, and
this module imports nothing from the product package.

What it models, in plain Python:

* a pool of ``num_blocks`` fixed-size physical blocks handed out on demand
  from a free list and returned when no sequence uses them any more (page
  "KV Cache与PagedAttention内存管理", section 分页机制 and its block-pool
  demo; page "vLLM 的 PagedAttention：KV cache 为什么要分页", §4 and §4.1:
  logical blocks of a request map to physical blocks anywhere in the pool,
  and a sequence grows one block at a time);
* per-sequence block tables (logical block index -> physical block id) and
  token counts; a token at logical position t lives in slot
  ``table[t // B] * B + t % B`` (page "读 vLLM 的 PagedAttention kernel", §3.2:
  the flat physical slot of the cache write);
* sharing with reference counts: a forked sequence starts with its parent's
  table and every block's count goes up by one (memory page, the
  prefix-sharing paragraph after 分页机制; blog page §4.2, parallel
  sampling: identical prefixes, including a last block that has not
  diverged yet, reuse the same physical blocks);
* copy-on-write: a write into a shared block whose count is above one first
  copies the block to a fresh one and redirects the writer's table entry;
  with a count of one the write goes in place (blog page §4.2).

Readings of points the pages leave open:
* the free list is a stack: it starts as ids num_blocks-1 .. 0 (so the first
  allocations return 0, 1, 2, ...), and released blocks are pushed in the
  order of the releasing table, so the last one released is reused first;
* a decode step appends exactly one token to each listed sequence, in list
  order; a sequence may appear once per step;
* a new token at a position that is a multiple of B opens a new block and
  never copies (the full block before it is not written);
* an operation that would need more free blocks than there are fails as a
  whole and changes nothing;
* a copy duplicates the whole block (all of its slots, for every KV head).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Sequence, Tuple

import numpy as np


class BlockManagerError(Exception):
    pass


@dataclass
class _Seq:
    table: List[int] = field(default_factory=list)
    num_tokens: int = 0


class BlockManager:
    """Reference block manager (see the module docstring for the rules)."""

    def __init__(self, num_blocks: int, block_size: int):
        if num_blocks <= 0 or block_size <= 0:
            raise BlockManagerError("sizes must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: List[int] = list(range(num_blocks - 1, -1, -1))   # top of stack = end
        self.refcount = [0] * num_blocks
        self.seqs: Dict[int, _Seq] = {}

    # -- helpers -----------------------------------------------------------
    def _take(self) -> int:
        b = self.free.pop()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def _slot(self, seq: _Seq, t: int) -> int:
        B = self.block_size
        return seq.table[t // B] * B + t % B

    # -- operations --------------------------------------------------------
    def add_sequence(self, seq_id: int, num_tokens: int) -> List[int]:
        """A new sequence holding ``num_tokens`` tokens (its prompt): allocates
        ceil(num_tokens / B) blocks and returns the slot of every token."""
        if seq_id in self.seqs or num_tokens < 0:
            raise BlockManagerError("bad sequence")
        need = -(-num_tokens // self.block_size)
        if need > len(self.free):
            raise BlockManagerError("out of blocks")
        seq = _Seq([self._take() for _ in range(need)], num_tokens)
        self.seqs[seq_id] = seq
        return [self._slot(seq, t) for t in range(num_tokens)]

    def fork(self, parent: int, child: int) -> None:
        """``child`` shares every block of ``parent``."""
        if parent not in self.seqs or child in self.seqs:
            raise BlockManagerError("bad fork")
        p = self.seqs[parent]
        for b in p.table:
            self.refcount[b] += 1
        self.seqs[child] = _Seq(list(p.table), p.num_tokens)

    def free_sequence(self, seq_id: int) -> None:
        if seq_id not in self.seqs:
            raise BlockManagerError("no such sequence")
        for b in self.seqs.pop(seq_id).table:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)

    def _blocks_needed(self, seq_ids: Sequence[int]) -> int:
        B = self.block_size
        pending = {}            # block -> count after the earlier appends of this step
        need = 0
        for sid in seq_ids:
            seq = self.seqs[sid]
            L = seq.num_tokens
            if L % B == 0:
                need += 1
                continue
            last = seq.table[L // B]
            rc = pending.get(last, self.refcount[last])
            if rc > 1:
                need += 1
                pending[last] = rc - 1
        return need

    def append_slots(self, seq_ids: Sequence[int]) -> Tuple[List[int], List[Tuple[int, int]]]:
        """One new token for each listed sequence (a decode step).  Returns the
        slot of every new token and the (source, destination) block copies
        the step's copy-on-writes need, in order."""
        if len(set(seq_ids)) != len(seq_ids) or any(s not in self.seqs for s in seq_ids):
            raise BlockManagerError("bad batch")
        if self._blocks_needed(seq_ids) > len(self.free):
            raise BlockManagerError("out of blocks")
        B = self.block_size
        slots, copies = [], []
        for sid in seq_ids:
            seq = self.seqs[sid]
            L = seq.num_tokens
            if L % B == 0:
                seq.table.append(self._take())
            else:
                last = seq.table[L // B]
                if self.refcount[last] > 1:          # shared: copy, then write the copy
                    new = self._take()
                    self.refcount[last] -= 1
                    seq.table[L // B] = new
                    copies.append((last, new))
            slots.append(self._slot(seq, L))
            seq.num_tokens = L + 1
        return slots, copies

    # -- queries -----------------------------------------------------------
    def num_free_blocks(self) -> int:
        return len(self.free)

    def seq_len(self, seq_id: int) -> int:
        return self.seqs[seq_id].num_tokens

    def table(self, seq_id: int) -> List[int]:
        return list(self.seqs[seq_id].table)

    def block_tables(self, seq_ids: Sequence[int], width: int, pad: int = -1) -> np.ndarray:
        out = np.full((len(seq_ids), width), pad, dtype=np.int32)
        for i, sid in enumerate(seq_ids):
            t = self.seqs[sid].table
            if len(t) > width:
                raise BlockManagerError("table wider than the output")
            out[i, :len(t)] = t
        return out


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs) -> None:
    """Apply (source, destination) block copies to the pools in place: every
    slot of every KV head of the destination becomes the source's.  Pairs
    are applied in order; a pair with an id outside the pool is skipped."""
    NB = k_cache.shape[0]
    for src, dst in pairs:
        if 0 <= src < NB and 0 <= dst < NB:
            k_cache[dst] = k_cache[src]
            v_cache[dst] = v_cache[src]
