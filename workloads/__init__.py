"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays them into arrays of the shapes
the paged KV cache uses (page "读 vLLM 的 PagedAttention kernel", §3.1):

    q        [num_seqs, num_heads, head_size]                       fp16
    k_cache  [num_blocks, num_kv_heads, head_size // x, block_size, x]  fp16
    v_cache  [num_blocks, num_kv_heads, head_size, block_size]       fp16
    block_tables [num_seqs, max_blocks_per_seq]  int32, padding = -1
    seq_lens [num_seqs]                                              int32

It holds none of the attention arithmetic and none of the layout decoding:
the pools are filled wholesale with N(0, sigma) values, and the block tables
are a seeded random placement of logical blocks onto physical ids.  Both the
CPU oracle (via the tests) and the HIP path consume what it returns.

Draw order for one (config, seed), one ``numpy.random.default_rng`` stream:
  1. seq_lens (uniform integers, inclusive bounds)
  2. physical placement: a permutation of the pool ids; the first
     sum(ceil(L_s / block_size)) ids are handed out seq-major in logical order
     (shared-prefix workloads hand out each group's prefix ids once)
  3. q
  4. K pool, 5. V pool (each from its own child SeedSequence, chunked and
     threaded; the chunking is fixed, so the values do not depend on the
     thread count)
  6. new key / value tokens for the cache-write step
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

FP16_NAN_BITS = 0x7E00


@dataclass(frozen=True)
class Workload:
    """One synthetic paged-decode workload (shapes and value distribution)."""

    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_size: int
    seq_len_lo: int
    seq_len_hi: int
    block_size: int = 16
    sigma: float = 1.0
    # fixed pool size in blocks; None = ceil(pool_slack * blocks needed)
    num_blocks: Optional[int] = None
    pool_slack: float = 1.1
    partition_size: int = 512
    # shared-prefix parallel sampling: groups of `group_size` sequences share
    # a `prefix_len`-token prefix (same physical ids), then a private tail of
    # U[seq_len_lo, seq_len_hi] cached tokens, then one new token written by
    # the cache-write step (so L_s = prefix_len + tail + 1)
    group_size: int = 0
    prefix_len: int = 0
    # multi-token queries: the last `query_len` tokens of every sequence have
    # queries (a prefill chunk / speculative verify); 0 = one decode query
    query_len: int = 0
    kernels: tuple = ("v1",)
    note: str = ""

    @property
    def x(self) -> int:
        return 16 // 2  # fp16 elements per 16-byte chunk

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_size)

    @property
    def max_seq_len(self) -> int:
        if self.group_size:
            return self.prefix_len + self.seq_len_hi + 1
        return self.seq_len_hi

    @property
    def max_blocks_per_seq(self) -> int:
        return -(-self.max_seq_len // self.block_size)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five synthetic workloads (shapes and distributions of the pages'
# decode setting: 7B-class GQA, one LLaMA-7B layer, 32K-128K contexts,
# parallel sampling with a shared prefix).
WORKLOADS = {
    "tiny": Workload("tiny", 4, 4, 4, 64, 1, 128, num_blocks=64,
                     kernels=("v1",), note="launch-bound; v1 only"),
    "gqa7b": Workload("gqa7b", 64, 28, 4, 128, 512, 4096,
                      kernels=("v1", "v2")),
    "mha7b": Workload("mha7b", 16, 32, 32, 128, 2048, 2048,
                      kernels=("v1", "v2")),
    "long_gqa": Workload("long_gqa", 8, 32, 8, 128, 32768, 131072,
                         sigma=0.5, num_blocks=65536, kernels=("v2",)),
    "shared_prefix": Workload("shared_prefix", 256, 32, 8, 128, 1, 256,
                              group_size=8, prefix_len=1024,
                              kernels=("cache", "v2")),
    # prefill-side shapes (multi-token queries over the paged cache)
    "prefill": Workload("prefill", 8, 32, 8, 128, 2048, 2048, query_len=2048,
                        kernels=("prefill",), note="full causal prefill of 2K-token prompts"),
    "chunked_prefill": Workload("chunked_prefill", 16, 32, 8, 128, 4096, 8192, query_len=512,
                                kernels=("prefill",),
                                note="512-token chunks at the end of 4K-8K contexts"),
}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill_normal_fp16(out: np.ndarray, seed_seq: np.random.SeedSequence,
                     sigma: float, chunk: int = 1 << 22) -> None:
    """Fill a float16 array with N(0, sigma) draws rounded to nearest-even.

    The array is cut into fixed chunks, each drawn from its own child of
    ``seed_seq``, so the result is the same for any thread count.
    """
    flat = out.reshape(-1)
    n = flat.size
    nchunks = max(1, -(-n // chunk))
    kids = seed_seq.spawn(nchunks)

    def work(i: int) -> None:
        lo = i * chunk
        hi = min(n, lo + chunk)
        rng = np.random.default_rng(kids[i])
        a = rng.standard_normal(hi - lo, dtype=np.float32)
        if sigma != 1.0:
            a *= np.float32(sigma)
        flat[lo:hi] = a  # float32 -> float16, round to nearest even

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))


def draw_seq_lens(w: Workload, rng: np.random.Generator) -> np.ndarray:
    if w.group_size:
        tails = rng.integers(w.seq_len_lo, w.seq_len_hi, size=w.num_seqs,
                             endpoint=True)
        return (w.prefix_len + tails + 1).astype(np.int32)
    return rng.integers(w.seq_len_lo, w.seq_len_hi, size=w.num_seqs,
                        endpoint=True).astype(np.int32)


def place_blocks(w: Workload, seq_lens: np.ndarray, rng: np.random.Generator):
    """Random physical placement -> (block_tables int32 padded with -1, num_blocks)."""
    B = w.block_size
    nblk = -(-seq_lens.astype(np.int64) // B)
    if w.group_size:
        n_groups = w.num_seqs // w.group_size
        pre = w.prefix_len // B
        need = n_groups * pre + int((nblk - pre).sum())
    else:
        need = int(nblk.sum())
    NB = w.num_blocks if w.num_blocks is not None else int(math.ceil(w.pool_slack * need))
    if NB < need:
        raise ValueError(f"pool of {NB} blocks cannot hold {need}")
    perm = rng.permutation(NB).astype(np.int32)
    bt = np.full((w.num_seqs, w.max_blocks_per_seq), -1, dtype=np.int32)
    pos = 0
    if w.group_size:
        pre = w.prefix_len // B
        for gidx in range(w.num_seqs // w.group_size):
            shared = perm[pos:pos + pre]
            pos += pre
            for s in range(gidx * w.group_size, (gidx + 1) * w.group_size):
                bt[s, :pre] = shared
                k = int(nblk[s]) - pre
                bt[s, pre:pre + k] = perm[pos:pos + k]
                pos += k
    else:
        for s in range(w.num_seqs):
            k = int(nblk[s])
            bt[s, :k] = perm[pos:pos + k]
            pos += k
    return bt, NB


@dataclass
class DecodeInputs:
    workload: Workload
    seed: int
    seq_lens: np.ndarray
    block_tables: np.ndarray
    num_blocks: int
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    # cache-write step: one new token per sequence
    key: Optional[np.ndarray] = None
    value: Optional[np.ndarray] = None
    new_pos: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return self.workload.scale

    @property
    def kv_bytes(self) -> int:
        """Bytes of K and V one decode call must read: sum_s L_s * 2 * KVH * D * 2."""
        w = self.workload
        return int(self.seq_lens.astype(np.int64).sum()) * 2 * w.num_kv_heads * w.head_size * 2

    @property
    def unique_kv_bytes(self) -> int:
        """Bytes of distinct (block, kv_head) tiles touched (shared blocks once)."""
        w = self.workload
        used = {}
        B = w.block_size
        for s in range(w.num_seqs):
            L = int(self.seq_lens[s])
            nb = -(-L // B)
            for i in range(nb):
                b = int(self.block_tables[s, i])
                fill = min(B, L - i * B)
                used[b] = max(used.get(b, 0), fill)
        return sum(used.values()) * 2 * w.num_kv_heads * w.head_size * 2


def make_inputs(w: Workload, seed: int, fill_values: bool = True) -> DecodeInputs:
    """Draw one seeded instance of a workload (host numpy arrays).

    ``fill_values=False`` leaves the pools uninitialised (structure only)."""
    rng = np.random.default_rng(seed)
    seq_lens = draw_seq_lens(w, rng)
    bt, NB = place_blocks(w, seq_lens, rng)
    q = np.empty((w.num_seqs, w.num_heads, w.head_size), dtype=np.float16)
    q[...] = (rng.standard_normal(q.shape, dtype=np.float32) * np.float32(w.sigma))
    x = w.x
    k_cache = np.empty((NB, w.num_kv_heads, w.head_size // x, w.block_size, x), dtype=np.float16)
    v_cache = np.empty((NB, w.num_kv_heads, w.head_size, w.block_size), dtype=np.float16)
    ss_k, ss_v, ss_new = np.random.SeedSequence(seed).spawn(3)
    if fill_values:
        fill_normal_fp16(k_cache, ss_k, w.sigma)
        fill_normal_fp16(v_cache, ss_v, w.sigma)
    inp = DecodeInputs(w, seed, seq_lens, bt, NB, q, k_cache, v_cache)
    # the decode step's new token per sequence: written to the cache at
    # logical position L_s - 1, then attended (append, then attend)
    rng_new = np.random.default_rng(ss_new)
    shape = (w.num_seqs, w.num_kv_heads, w.head_size)
    inp.key = (rng_new.standard_normal(shape, dtype=np.float32) * np.float32(w.sigma)).astype(np.float16)
    inp.value = (rng_new.standard_normal(shape, dtype=np.float32) * np.float32(w.sigma)).astype(np.float16)
    inp.new_pos = np.maximum(seq_lens.astype(np.int64) - 1, 0)
    return inp


def slot_of(block_tables: np.ndarray, seq: int, pos: int, block_size: int) -> int:
    """Flat physical slot of logical position `pos` of sequence `seq`:
    physical block id * block_size + offset in block (page "读 vLLM 的
    PagedAttention kernel", §3.2).  Index bookkeeping for building inputs."""
    return int(block_tables[seq, pos // block_size]) * block_size + pos % block_size


def new_token_slots(inp: DecodeInputs) -> np.ndarray:
    """slot_mapping (int64) for the cache-write step's new tokens (-1, i.e.
    skip, for an empty sequence)."""
    B = inp.workload.block_size
    return np.array([slot_of(inp.block_tables, s, int(p), B) if inp.seq_lens[s] > 0 else -1
                     for s, p in enumerate(inp.new_pos)], dtype=np.int64)


def small_workload(name: str = "small", *, num_seqs=3, num_heads=8, num_kv_heads=2,
                   head_size=128, seq_len_lo=1, seq_len_hi=200, sigma=1.0,
                   num_blocks=None, partition_size=64, block_size=16) -> Workload:
    """An ad-hoc workload for parity cases (any G, D, length mix)."""
    return Workload(name, num_seqs, num_heads, num_kv_heads, head_size, seq_len_lo,
                    seq_len_hi, block_size=block_size, sigma=sigma, num_blocks=num_blocks,
                    partition_size=partition_size, kernels=("v1", "v2"))


# -- parallel sampling (fork) ------------------------------------------------

@dataclass(frozen=True)
class ForkWorkload:
    """Parallel sampling: `groups` prompts of `prompt_len` tokens, each forked
    into `samples` sequences that share the prompt's blocks (blog page §4.2).
    The first decode step after the fork splits every shared, partly filled
    last prompt block by copy-on-write.  Only the values are drawn here; the
    slots, tables and copies come from whichever block manager is under test."""
    name: str = "fork"
    groups: int = 32
    samples: int = 8
    prompt_len: int = 1000           # not a multiple of the block size
    num_heads: int = 32
    num_kv_heads: int = 8
    head_size: int = 128
    block_size: int = 16
    partition_size: int = 512
    sigma: float = 1.0

    @property
    def num_seqs(self) -> int:
        return self.groups * self.samples

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_size)

    @property
    def pool_blocks(self) -> int:
        """Prompt blocks plus one new block per sequence, with 10% slack."""
        need = self.groups * -(-self.prompt_len // self.block_size) + self.num_seqs
        return int(math.ceil(1.1 * need))


@dataclass
class ForkInputs:
    workload: ForkWorkload
    seed: int
    prompt_k: np.ndarray     # [groups, prompt_len, KVH, D] fp16
    prompt_v: np.ndarray
    q: np.ndarray            # [num_seqs, H, D] fp16 (sequence g*samples + c)
    key: np.ndarray          # [num_seqs, KVH, D] fp16: the step's new token
    value: np.ndarray


FORK = ForkWorkload()


def make_fork_inputs(w: ForkWorkload, seed: int) -> ForkInputs:
    """One rng stream, drawn in order: prompt K, prompt V, q, new key, new value."""
    rng = np.random.default_rng(seed)

    def normal(shape):
        return (w.sigma * rng.standard_normal(shape)).astype(np.float16)

    KVH, D = w.num_kv_heads, w.head_size
    pk = normal((w.groups, w.prompt_len, KVH, D))
    pv = normal((w.groups, w.prompt_len, KVH, D))
    q = normal((w.num_seqs, w.num_heads, D))
    key = normal((w.num_seqs, KVH, D))
    value = normal((w.num_seqs, KVH, D))
    return ForkInputs(w, seed, pk, pv, q, key, value)


def make_chunk(w: Workload, inp: "DecodeInputs", seed: int):
    """Queries and the new K/V of the last `query_len` tokens of every
    sequence, with their slots: q [T, H, D], key/value [T, KVH, D] fp16,
    slots [T] int64, query_start_loc [S + 1] int32 (T = S * query_len).
    Drawn from their own stream (seed, 1) so the pools stay as make_inputs
    drew them."""
    rng = np.random.default_rng([seed, 1])
    n = w.query_len
    S, H, KVH, D, B = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_size, w.block_size
    T = S * n
    q = (w.sigma * rng.standard_normal((T, H, D))).astype(np.float16)
    key = (w.sigma * rng.standard_normal((T, KVH, D))).astype(np.float16)
    value = (w.sigma * rng.standard_normal((T, KVH, D))).astype(np.float16)
    slots = np.empty(T, np.int64)
    for s in range(S):
        L = int(inp.seq_lens[s])
        t = np.arange(L - n, L)
        slots[s * n:(s + 1) * n] = inp.block_tables[s, t // B].astype(np.int64) * B + t % B
    qsl = (np.arange(S + 1) * n).astype(np.int32)
    return q, key, value, slots, qsl
