"""Pins of the block-manager oracle (CPU).

* The hand-worked copy-on-write scenario in tests/golden/cow_scenario.json
  (parallel sampling, blog page §4.2; allocation on demand, memory page
  分页机制), step by step: slots, copies, tables, reference counts, free
  blocks, and the all-or-nothing failures.
* On seeded random operation sequences: reference counts equal the number of
  table entries naming each block, the free list holds exactly the unused
  blocks, and -- the point of paging -- every sequence's tokens read back
  through its table in logical order, after every fork, copy-on-write and
  release (a pool of token ids stands in for the K/V contents).
* Planted mistakes (always copy, never copy, wrong slot, leaked release)
  fail one of the above.
"""
import copy
import json
import os

import numpy as np
import pytest

import oracle
from oracle import BlockManager, BlockManagerError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cow_scenario.json")


def run_golden(make, error=BlockManagerError):
    d = json.load(open(GOLDEN))
    bm = make(d["num_blocks"], d["block_size"])
    for i, st in enumerate(d["steps"]):
        op = st["op"]
        got = {}
        try:
            if op == "add":
                got["slots"] = list(bm.add_sequence(st["seq"], st["tokens"]))
            elif op == "fork":
                bm.fork(st["parent"], st["child"])
            elif op == "free":
                bm.free_sequence(st["seq"])
            elif op == "append":
                s, c = bm.append_slots(st["seqs"])
                got["slots"], got["copies"] = list(s), [list(x) for x in c]
            err = False
        except error:
            err = True
        where = f"step {i} ({op})"
        assert err == st.get("error", False), where
        for k in ("slots", "copies"):
            if k in st:
                assert got[k] == st[k], where
        for sid, t in st.get("tables", {}).items():
            assert list(bm.table(int(sid))) == t, where
        for b, r in st.get("refcount", {}).items():
            assert bm.refcount[int(b)] == r, where
        for sid, n in st.get("lens", {}).items():
            assert bm.seq_len(int(sid)) == n, where
        assert bm.num_free_blocks() == st["free"], where


def test_golden_cow_scenario():
    run_golden(BlockManager)


class ContentModel:
    """Token ids stand in for K/V: pool[b][o] holds the id written to slot
    b*B + o.  Each sequence keeps the list of ids it should read back."""

    def __init__(self, num_blocks, B):
        self.B = B
        self.pool = np.full((num_blocks, B), -1, dtype=np.int64)
        self.hist = {}
        self.next_id = 0

    def write(self, slots):
        ids = list(range(self.next_id, self.next_id + len(slots)))
        self.next_id += len(slots)
        for s, t in zip(slots, ids):
            self.pool[s // self.B, s % self.B] = t
        return ids

    def check(self, bm):
        for sid, h in self.hist.items():
            t = bm.table(sid)
            got = [int(self.pool[t[i // self.B], i % self.B]) for i in range(len(h))]
            assert got == h, f"sequence {sid} reads back other tokens"


def random_ops(bm, seed, n_ops=400, check_every=True):
    rng = np.random.default_rng(seed)
    B = bm.block_size
    cm = ContentModel(bm.num_blocks, B)
    live = []
    next_sid = 0
    for _ in range(n_ops):
        r = rng.random()
        try:
            if r < 0.15 or not live:
                n = int(rng.integers(0, 5 * B))
                slots = bm.add_sequence(next_sid, n)
                cm.hist[next_sid] = cm.write(slots)
                live.append(next_sid)
                next_sid += 1
            elif r < 0.30:
                p = int(rng.choice(live))
                bm.fork(p, next_sid)
                cm.hist[next_sid] = list(cm.hist[p])
                live.append(next_sid)
                next_sid += 1
            elif r < 0.40 and len(live) > 1:
                sid = int(rng.choice(live))
                bm.free_sequence(sid)
                live.remove(sid)
                del cm.hist[sid]
            else:
                k = int(rng.integers(1, min(len(live), 6) + 1))
                batch = [int(x) for x in rng.choice(live, size=k, replace=False)]
                slots, copies = bm.append_slots(batch)
                for src, dst in copies:          # copies first, then the step's writes
                    cm.pool[dst] = cm.pool[src]
                ids = cm.write(slots)
                for sid, t in zip(batch, ids):
                    cm.hist[sid].append(t)
        except BlockManagerError:
            pass
        if check_every:
            check_invariants(bm)
            cm.check(bm)
    return cm


def check_invariants(bm):
    count = np.zeros(bm.num_blocks, dtype=np.int64)
    for sid in bm.seqs:
        for b in bm.table(sid):
            count[b] += 1
    assert list(count) == list(bm.refcount)
    free = list(bm.free)
    assert len(set(free)) == len(free)
    assert set(free) == {b for b in range(bm.num_blocks) if count[b] == 0}
    for sid in bm.seqs:
        n = bm.seq_len(sid)
        assert len(bm.table(sid)) == -(-n // bm.block_size)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
@pytest.mark.parametrize("nb,B", [(24, 4), (64, 16), (9, 2)])
def test_random_sequences_keep_content_and_counts(seed, nb, B):
    random_ops(BlockManager(nb, B), seed)


def snapshot(bm):
    return copy.deepcopy((bm.free, bm.refcount,
                          {k: (bm.table(k), bm.seq_len(k)) for k in bm.seqs}))


def test_failed_operations_change_nothing():
    bm = BlockManager(4, 4)
    bm.add_sequence(0, 7)           # blocks 0, 1; 2 free
    for child in (1, 2, 3):
        bm.fork(0, child)           # block 1 (partly filled) shared four ways
    before = snapshot(bm)
    with pytest.raises(BlockManagerError):
        bm.add_sequence(9, 9)       # 3 blocks, 2 free
    with pytest.raises(BlockManagerError):
        bm.append_slots([0, 1, 2, 3])   # three copy-on-writes, 2 free
    with pytest.raises(BlockManagerError):
        bm.append_slots([0, 0])     # a sequence twice in one step
    with pytest.raises(BlockManagerError):
        bm.fork(5, 6)
    with pytest.raises(BlockManagerError):
        bm.fork(0, 1)
    assert snapshot(bm) == before
    bm.free_sequence(3)             # block 1 now shared three ways
    slots, copies = bm.append_slots([0, 1, 2])     # two copies, the last writes in place
    assert copies == [(1, 2), (1, 3)] and slots == [2 * 4 + 3, 3 * 4 + 3, 1 * 4 + 3]


def test_copy_blocks_oracle():
    rng = np.random.default_rng(0)
    k = rng.standard_normal((6, 2, 4, 16, 8)).astype(np.float16)
    v = rng.standard_normal((6, 2, 32, 16)).astype(np.float16)
    k0, v0 = k.copy(), v.copy()
    oracle.copy_blocks(k, v, [(1, 4), (1, 5), (9, 0), (2, -1)])
    assert np.array_equal(k[4], k0[1]) and np.array_equal(v[5], v0[1])
    for b in (0, 1, 2, 3):
        assert np.array_equal(k[b], k0[b]) and np.array_equal(v[b], v0[b])


# -- planted mistakes ------------------------------------------------------

class AlwaysCopy(BlockManager):
    """Treats every partly filled last block as shared (copies it on each write)."""

    def append_slots(self, seq_ids):
        for sid in seq_ids:
            if self.seqs[sid].table:
                self.refcount[self.seqs[sid].table[-1]] += 1
        return super().append_slots(seq_ids)


class NeverCopy(BlockManager):
    """Writes shared blocks in place."""

    def append_slots(self, seq_ids):
        B = self.block_size
        slots = []
        for sid in seq_ids:
            seq = self.seqs[sid]
            L = seq.num_tokens
            if L % B == 0:
                seq.table.append(self._take())
            slots.append(self._slot(seq, L))
            seq.num_tokens = L + 1
        return slots, []


class OffByOneSlot(BlockManager):
    def _slot(self, seq, t):
        B = self.block_size
        return seq.table[t // B] * B + (t + 1) % B


class LeakyFree(BlockManager):
    """Returns only the first block of a released table."""

    def free_sequence(self, seq_id):
        seq = self.seqs.pop(seq_id)
        for i, b in enumerate(seq.table):
            self.refcount[b] -= 1
            if self.refcount[b] == 0 and i == 0:
                self.free.append(b)


@pytest.mark.parametrize("bad", [NeverCopy, OffByOneSlot, LeakyFree, AlwaysCopy])
def test_planted_mistakes_are_caught(bad):
    caught = False
    try:
        run_golden(bad)
    except AssertionError:
        caught = True
    if not caught:
        try:
            for seed in range(3):
                random_ops(bad(24, 4), seed)
        except AssertionError:
            caught = True
    assert caught, bad.__name__
