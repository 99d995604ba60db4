"""KV-cache memory model and an allocation simulator: how many requests a
pool serves, and how much of it holds tokens, under whole-length reservation
versus paged blocks handed out by the native block manager (libpa.so).

Page "KV Cache与PagedAttention内存管理": sections 内存占用模型 (2 x layers x
d_model x S x B x 2 bytes), 碎片化问题 (utilisation eta = sum s_i / (N s_max)
under reservation) and 分页机制 (fixed-size blocks on demand); blog page
"vLLM 的 PagedAttention：KV cache 为什么要分页", §3 (reservation waste) and
§5.1 (paging leaves only each request's last block partly empty).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence

from ._lib import BlockManager, BlockManagerError


def kv_cache_bytes(layers: int, d_model: int, seq_len: int, batch: int, elem_bytes: int = 2) -> int:
    """K and V of every layer for `batch` sequences of `seq_len` tokens."""
    return 2 * layers * d_model * seq_len * batch * elem_bytes


@dataclass
class ServeResult:
    served: int          # requests admitted before the pool ran out
    token_cells: int     # cells holding tokens
    held_cells: int      # cells taken from the pool (reserved, or in blocks)

    @property
    def utilization(self) -> float:
        return self.token_cells / self.held_cells if self.held_cells else 0.0


def serve_reserved(lengths: Sequence[int], total_cells: int, s_max: int) -> ServeResult:
    """Whole-length reservation on the native block manager: the pool is cut
    into total_cells // s_max regions of s_max cells and every request takes
    one whole region however short it is (one block of s_max tokens); admit
    in order until a region cannot be had."""
    regions = total_cells // s_max
    if regions <= 0:
        return ServeResult(0, 0, 0)
    bm = BlockManager(regions, s_max)
    served = used = 0
    for i, s in enumerate(lengths):
        try:
            bm.add_sequence(i, s_max)
        except BlockManagerError:
            break
        used += int(s)
        served += 1
    return ServeResult(served, used, (regions - bm.num_free_blocks()) * s_max)


def serve_paged(lengths: Sequence[int], total_cells: int, block_size: int) -> ServeResult:
    """Every request takes ceil(s / block_size) blocks from the native block
    manager (a pool of total_cells // block_size blocks); admit in order
    until an allocation fails."""
    bm = BlockManager(total_cells // block_size, block_size)
    served = used = 0
    for i, s in enumerate(lengths):
        try:
            bm.add_sequence(i, int(s))
        except BlockManagerError:
            break
        used += int(s)
        served += 1
    held = (total_cells // block_size - bm.num_free_blocks()) * block_size
    return ServeResult(served, used, held)
