"""CPU oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check of ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never does, and this
module imports nothing from the product package.

What it computes, in float64, from inputs widened exactly from fp16:

* the paged layout decode (page "读 vLLM 的 PagedAttention kernel", §3.1:
  ``k_cache[num_blocks, num_kv_heads, head_size/x, block_size, x]`` and
  ``v_cache[num_blocks, num_kv_heads, head_size, block_size]``, with the
  block table mapping logical block -> physical block, §2 and §3.4);
* plain scaled dot-product attention with a two-pass softmax (page
  "KV Cache与PagedAttention内存管理", section 自回归推理, the formula
  softmax(QK^T / sqrt(d_k)) V; page "读 vLLM 的 PagedAttention kernel", §4,
  ``dense_attention`` as "the truth");
* the per-partition partial results of the partitioned ("v2") variant and
  their log-sum-exp merge (§3.3 of the kernel page says the partitions are
  computed in parallel and merged afterwards but prints no merge formula; the
  reading used here is the standard exact merge, written out below);
* the cache-write scatter through ``slot_mapping`` (§3.2) and the inverse
  gather in logical order.

The paging changes where K/V live, never what attention computes (§4 and §6
of the kernel page), so the oracle's attention is the plain definition applied
to the gathered, contiguous K/V.  It does not use the online-softmax
recurrence; ``online_block_attention`` below writes that recurrence out
separately, only to cross-check this oracle.

Readings of points the pages leave open:
* query head h reads KV head h // (num_heads // num_kv_heads);
* ``scale`` is an explicit argument (the configs use 1/sqrt(head_size));
* ``seq_len == 0`` gives an all-zero output row;
* partition p covers tokens [p*PS, min((p+1)*PS, L)); partials are stored
  normalised (o_p = acc/l) with m_p and l_p in natural-log units;
* ``slot < 0`` in slot_mapping means "skip this token".
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# Layout decode (kernel page §3.1, §2 "block table is the page table of KV")
# ---------------------------------------------------------------------------

def key_vector(k_cache: np.ndarray, block: int, kv_head: int, slot: int) -> np.ndarray:
    """K of the token in slot `slot` of physical block `block`.

    k_cache[b, h, c, o, j] holds dimension d = c*x + j of the token in slot o
    (head_size cut into runs of x contiguous elements, §3.1).
    """
    tile = k_cache[block, kv_head]          # [D/x, B, x]
    return tile[:, slot, :].reshape(-1)     # d = c*x + j


def value_vector(v_cache: np.ndarray, block: int, kv_head: int, slot: int) -> np.ndarray:
    """V of the token in slot `slot`: v_cache[b, h, d, o] (no packing, §3.1)."""
    return v_cache[block, kv_head, :, slot]


def gather_sequence(k_cache, v_cache, block_table_row, seq_len: int, kv_head: int,
                    block_size: int):
    """Walk one sequence's block table in logical order and return its K, V as
    contiguous [seq_len, head_size] arrays in the storage dtype.

    Logical token t lives in physical block block_table_row[t // block_size],
    slot t % block_size (page map l_i -> p_i of page "KV Cache与PagedAttention
    内存管理", section 分页机制; kernel page §3.4 steps 1-2).  Entries past
    ceil(seq_len / block_size) and slots past seq_len in the last block are
    never read (kernel page §4: the last block may be partly filled).
    """
    D = k_cache.shape[2] * k_cache.shape[4]
    K = np.empty((seq_len, D), dtype=k_cache.dtype)
    V = np.empty((seq_len, D), dtype=v_cache.dtype)
    for t in range(seq_len):
        b = int(block_table_row[t // block_size])
        o = t % block_size
        K[t] = key_vector(k_cache, b, kv_head, o)
        V[t] = value_vector(v_cache, b, kv_head, o)
    return K, V


def gather_sequence_fast(k_cache, v_cache, block_table_row, seq_len: int, kv_head: int,
                         block_size: int):
    """Same as gather_sequence, by whole blocks (numpy fancy indexing), for
    large sequences.  The per-token version above pins it in the tests."""
    nb = -(-seq_len // block_size)
    D = k_cache.shape[2] * k_cache.shape[4]
    if nb == 0:
        return (np.empty((0, D), dtype=k_cache.dtype), np.empty((0, D), dtype=v_cache.dtype))
    ids = np.asarray(block_table_row[:nb], dtype=np.int64)
    kt = k_cache[ids, kv_head]                       # [nb, D/x, B, x]
    K = kt.transpose(0, 2, 1, 3).reshape(nb * block_size, -1)[:seq_len]
    vt = v_cache[ids, kv_head]                       # [nb, D, B]
    V = vt.transpose(0, 2, 1).reshape(nb * block_size, -1)[:seq_len]
    return K, V


def kv_head_of(h: int, num_heads: int, num_kv_heads: int) -> int:
    """Query head -> KV head: contiguous groups of G = num_heads/num_kv_heads
    query heads share one KV head (reading; the pages only name num_kv_heads)."""
    return h // (num_heads // num_kv_heads)


# ---------------------------------------------------------------------------
# Attention (page "KV Cache与PagedAttention内存管理", 自回归推理 formula)
# ---------------------------------------------------------------------------

def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V for queries q [n, D] over keys/values [L, D], fp64.

    Two passes: scores, their maximum M, weights exp(z - M) and their sum Z,
    then the weighted sum of V divided by Z.  L == 0 gives zeros.
    """
    q64 = np.asarray(q, dtype=F64).reshape(-1, q.shape[-1])
    if K.shape[0] == 0:
        return np.zeros((q64.shape[0], V.shape[1]), dtype=F64)
    K64 = np.asarray(K, dtype=F64)
    V64 = np.asarray(V, dtype=F64)
    z = scale * (q64 @ K64.T)                    # [n, L]
    M = z.max(axis=1, keepdims=True)
    w = np.exp(z - M)
    Z = w.sum(axis=1, keepdims=True)
    return (w @ V64) / Z


def paged_decode(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                 block_size: int, fast: bool = True, heads=None) -> np.ndarray:
    """Decode attention over the paged cache -> out [S, H, D] float64.

    For each sequence s and query head h: gather K/V of KV head h // G through
    the block table, then plain attention.  `heads` optionally restricts the
    computation to a list of (s, h) pairs (other rows are NaN).
    """
    S, H, D = q.shape
    KVH = k_cache.shape[1]
    out = np.full((S, H, D), np.nan, dtype=F64)
    gather = gather_sequence_fast if fast else gather_sequence
    wanted = None
    if heads is not None:
        wanted = {}
        for s, h in heads:
            wanted.setdefault(int(s), set()).add(int(h))
    for s in range(S):
        if wanted is not None and s not in wanted:
            continue
        L = max(0, int(seq_lens[s]))
        by_kv = {}
        for h in range(H):
            if wanted is None or h in wanted[s]:
                by_kv.setdefault(kv_head_of(h, H, KVH), []).append(h)
        for kvh, hs in by_kv.items():
            K, V = gather(k_cache, v_cache, block_tables[s], L, kvh, block_size)
            out[s, hs] = attention(q[s, hs], K, V, scale)
    return out


def paged_prefill(q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, scale: float,
                  block_size: int) -> np.ndarray:
    """Multi-token queries with a causal mask -> out [total_q, H, D] float64.

    Sequence s holds L = seq_lens[s] tokens; its last n = query_start_loc[s+1]
    - query_start_loc[s] tokens have queries (rows query_start_loc[s] + j).
    Query j sits at position p = L - n + j and attends keys 0..p: the plain
    definition over the gathered K/V prefix (prefill writes the prompt's K/V
    and attends causally -- blog page §2; memory page, 自回归推理).  n = 1 is
    a decode step; n = L a full prefill.
    """
    T, H, D = q.shape
    KVH = k_cache.shape[1]
    out = np.full((T, H, D), np.nan, dtype=F64)
    for s in range(len(seq_lens)):
        L = int(seq_lens[s])
        q0, q1 = int(query_start_loc[s]), int(query_start_loc[s + 1])
        n = q1 - q0
        for kvh in range(KVH):
            K, V = gather_sequence_fast(k_cache, v_cache, block_tables[s], L, kvh, block_size)
            hs = [h for h in range(H) if kv_head_of(h, H, KVH) == kvh]
            for j in range(n):
                m = visible_keys(L - n + j)
                out[q0 + j, hs] = attention(q[q0 + j, hs], K[:m], V[:m], scale)
    return out


def visible_keys(p: int) -> int:
    """Keys a query at position p attends to under the causal mask: 0..p."""
    return p + 1


# ---------------------------------------------------------------------------
# Partitioned variant and its merge (kernel page §3.3: PARTITION_SIZE)
# ---------------------------------------------------------------------------

def num_partitions(seq_len: int, partition_size: int) -> int:
    return -(-max(0, seq_len) // partition_size)


def partition_partials(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                       block_size: int, partition_size: int, max_num_partitions: int):
    """Per-partition partial results of the partitioned decode.

    Partition p of sequence s covers tokens [p*PS, min((p+1)*PS, L_s)).  For
    each query head: m_p = max of its scores, l_p = sum exp(z - m_p), and the
    normalised partial output o_p = sum exp(z - m_p) V / l_p.  Partitions
    p >= ceil(L_s / PS) are left NaN (never written, never read).
    Returns (tmp_out [S,H,P,D], exp_sums [S,H,P], max_logits [S,H,P]).
    """
    S, H, D = q.shape
    KVH = k_cache.shape[1]
    G = H // KVH
    P = max_num_partitions
    tmp_out = np.full((S, H, P, D), np.nan, dtype=F64)
    exp_sums = np.full((S, H, P), np.nan, dtype=F64)
    max_logits = np.full((S, H, P), np.nan, dtype=F64)
    for s in range(S):
        L = max(0, int(seq_lens[s]))
        for kvh in range(KVH):
            K, V = gather_sequence_fast(k_cache, v_cache, block_tables[s], L, kvh, block_size)
            K64 = K.astype(F64)
            V64 = V.astype(F64)
            q64 = q[s, kvh * G:(kvh + 1) * G].astype(F64)
            for p in range(num_partitions(L, partition_size)):
                lo, hi = p * partition_size, min((p + 1) * partition_size, L)
                z = scale * (q64 @ K64[lo:hi].T)             # [G, n]
                m = z.max(axis=1)
                e = np.exp(z - m[:, None])
                l = e.sum(axis=1)
                hs = slice(kvh * G, (kvh + 1) * G)
                max_logits[s, hs, p] = m
                exp_sums[s, hs, p] = l
                tmp_out[s, hs, p] = (e @ V64[lo:hi]) / l[:, None]
    return tmp_out, exp_sums, max_logits


def lse_merge(tmp_out, exp_sums, max_logits, seq_lens, partition_size: int) -> np.ndarray:
    """Merge per-partition partials into the final output (log-sum-exp merge).

    With M = max_p m_p and w_p = l_p * exp(m_p - M):
        out = sum_p w_p * o_p / sum_p w_p      over p < ceil(L_s / PS).
    Because o_p = acc_p / l_p and acc_p = sum_{t in p} exp(z_t - m_p) v_t, the
    numerator is exp(-M) * sum_t exp(z_t) v_t and the denominator
    exp(-M) * sum_t exp(z_t): exactly the unpartitioned softmax.  A sequence
    with no partition (L_s <= 0) gives zeros.
    """
    S, H, P, D = tmp_out.shape
    out = np.zeros((S, H, D), dtype=F64)
    for s in range(S):
        n = min(P, num_partitions(int(seq_lens[s]), partition_size))
        if n == 0:
            continue
        m = np.asarray(max_logits[s, :, :n], dtype=F64)       # [H, n]
        l = np.asarray(exp_sums[s, :, :n], dtype=F64)
        o = np.asarray(tmp_out[s, :, :n], dtype=F64)          # [H, n, D]
        M = m.max(axis=1, keepdims=True)
        w = l * np.exp(m - M)
        out[s] = (w[:, :, None] * o).sum(axis=1) / w.sum(axis=1)[:, None]
    return out


# ---------------------------------------------------------------------------
# Online-softmax block loop (kernel page §2 flowchart and §3.3), cross-check
# ---------------------------------------------------------------------------

def online_block_attention(q, K, V, scale: float, block_size: int) -> np.ndarray:
    """The block-at-a-time online-softmax recurrence, fp64, for one query row
    set q [n, D] over contiguous K, V [L, D].

    Running state per query: maximum m (start -inf), normaliser l (start 0)
    and accumulator acc (start 0).  For each block of keys: scores z, new
    maximum m' = max(m, max z), correction c = exp(m - m') (0 while m is
    -inf), weights p = exp(z - m'), then l = l*c + sum p, acc = acc*c + p V,
    m = m'.  At the end out = acc / l.  Written only to cross-check
    ``attention`` (the two must agree to rounding).
    """
    q64 = np.asarray(q, dtype=F64).reshape(-1, q.shape[-1])
    n, D = q64.shape
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, V.shape[1]))
    for lo in range(0, K.shape[0], block_size):
        Kb = np.asarray(K[lo:lo + block_size], dtype=F64)
        Vb = np.asarray(V[lo:lo + block_size], dtype=F64)
        z = scale * (q64 @ Kb.T)
        m_new = np.maximum(m, z.max(axis=1))
        c = np.where(np.isneginf(m), 0.0, np.exp(m - m_new))
        p = np.exp(z - m_new[:, None])
        l = l * c + p.sum(axis=1)
        acc = acc * c[:, None] + p @ Vb
        m = m_new
    return acc / l[:, None]


# ---------------------------------------------------------------------------
# Cache write and logical-order gather (kernel page §3.2)
# ---------------------------------------------------------------------------

def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, block_size: int,
                      inplace: bool = False):
    """Scatter new tokens into the pools, token by token.

    Token i goes to flat physical slot s = slot_mapping[i]: block s // B, offset
    s % B.  Its K lands in k_cache[b, h, d // x, o, d % x] and its V in
    v_cache[b, h, d, o] for every KV head h.  slot < 0 skips the token.
    Returns the new (k_cache, v_cache): copies, unless inplace=True.
    """
    kc = k_cache if inplace else k_cache.copy()
    vc = v_cache if inplace else v_cache.copy()
    T, KVH, D = key.shape
    x = kc.shape[4]
    for i in range(T):
        slot = int(slot_mapping[i])
        if slot < 0:
            continue
        b, o = divmod(slot, block_size)
        for h in range(KVH):
            for d in range(D):
                kc[b, h, d // x, o, d % x] = key[i, h, d]
                vc[b, h, d, o] = value[i, h, d]
    return kc, vc


def gather_kv(k_cache, v_cache, block_tables, seq_lens, block_size: int):
    """All sequences' K and V in logical order, storage dtype (bit-exact):
    returns (k_out, v_out) of shape [sum_s L_s, num_kv_heads, head_size]."""
    S = block_tables.shape[0]
    KVH = k_cache.shape[1]
    D = k_cache.shape[2] * k_cache.shape[4]
    total = int(sum(max(0, int(L)) for L in seq_lens))
    k_out = np.empty((total, KVH, D), dtype=k_cache.dtype)
    v_out = np.empty((total, KVH, D), dtype=v_cache.dtype)
    pos = 0
    for s in range(S):
        L = max(0, int(seq_lens[s]))
        for h in range(KVH):
            K, V = gather_sequence_fast(k_cache, v_cache, block_tables[s], L, h, block_size)
            k_out[pos:pos + L, h] = K
            v_out[pos:pos + L, h] = V
        pos += L
    return k_out, v_out


# ---------------------------------------------------------------------------
# Helpers for test inputs (index facts only)
# ---------------------------------------------------------------------------

def used_fill(block_tables, seq_lens, block_size: int) -> dict:
    """Physical block id -> number of leading slots some sequence attends
    (the largest fill over every sequence whose table names the block)."""
    fill = {}
    for s in range(block_tables.shape[0]):
        L = max(0, int(seq_lens[s]))
        nb = -(-L // block_size)
        for i in range(nb):
            b = int(block_tables[s, i])
            fill[b] = max(fill.get(b, 0), min(block_size, L - i * block_size))
    return fill


def poison_unused(k_cache, v_cache, block_tables, seq_lens, block_size: int,
                  nan_bits: int = 0x7E00):
    """In place: NaN into every slot no sequence attends -- unreferenced blocks
    and the tail slots of partly filled last blocks -- to show the kernels
    never read them."""
    NB = k_cache.shape[0]
    fill = used_fill(block_tables, seq_lens, block_size)
    kv = k_cache.view(np.uint16)
    vv = v_cache.view(np.uint16)
    unref = sorted(set(range(NB)) - set(fill))
    if unref:
        kv[unref] = nan_bits
        vv[unref] = nan_bits
    for b, f in fill.items():
        if f < block_size:
            kv[b, :, :, f:, :] = nan_bits
            vv[b, :, :, f:] = nan_bits

