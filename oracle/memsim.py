"""CPU oracle of the KV-cache memory model -- TEST INFRASTRUCTURE ONLY.

Page "KV Cache与PagedAttention内存管理": the KV cache of a batch takes
2 (K and V) x layers x d_model x sequence length x batch x 2 bytes (fp16),
section 内存占用模型 (LLaMA-7B: 2*32*4096*2048*16*2 B ~ 17.2 GB); a reserving
allocator gives every request s_max cells, so its utilisation is
eta = sum_i s_i / (N * s_max), section 碎片化问题; a paged allocator hands
out fixed-size blocks on demand (section 分页机制), wasting at most the
unfilled tail of each request's last block (blog page "vLLM 的
PagedAttention：KV cache 为什么要分页", §5.1).

Admission is written in closed form: requests are admitted in arrival order
and the first one that does not fit stops admission, so the admitted set is
the longest prefix of the arrival order whose cost fits the pool.
"""
from __future__ import annotations

import numpy as np


def kv_cache_bytes(layers: int, d_model: int, seq_len: int, batch: int, elem_bytes: int = 2) -> int:
    return 2 * layers * d_model * seq_len * batch * elem_bytes


def reservation_utilization(lengths, s_max: int) -> float:
    return sum(lengths) / (len(lengths) * s_max)


def paged_utilization(lengths, block_size: int) -> float:
    blocks = sum(-(-s // block_size) for s in lengths)
    return sum(lengths) / (blocks * block_size)


def serve_reserved(lengths, total_cells: int, s_max: int):
    """Whole-length reservation: each admitted request costs s_max cells
    whatever its length, so the admitted prefix has min(N, total // s_max)
    requests.  Returns (served, cells holding tokens, cells reserved)."""
    served = min(len(lengths), total_cells // s_max)
    return served, int(sum(int(s) for s in lengths[:served])), served * s_max


def serve_paged(lengths, total_cells: int, block_size: int):
    """Paged blocks: request i costs ceil(s_i / B) blocks of a pool of
    total // B; the admitted prefix is the longest one whose running block
    count stays within the pool.  Returns (served, cells holding tokens,
    cells held in blocks)."""
    need = np.array([-(-int(s) // block_size) for s in lengths], dtype=np.int64)
    running = np.cumsum(need)
    served = int(np.searchsorted(running, total_cells // block_size, side="right"))
    held = int(running[served - 1]) * block_size if served else 0
    return served, int(sum(int(s) for s in lengths[:served])), held
