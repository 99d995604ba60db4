"""CPU oracle of the KV-cache memory model -- TEST INFRASTRUCTURE ONLY.

Page "KV Cache与PagedAttention内存管理": the KV cache of a batch takes
2 (K and V) x layers x d_model x sequence length x batch x 2 bytes (fp16),
section 内存占用模型 (LLaMA-7B: 2*32*4096*2048*16*2 B ~ 17.2 GB); a reserving
allocator gives every request s_max cells, so its utilisation is
eta = sum_i s_i / (N * s_max), section 碎片化问题; a paged allocator hands
out fixed-size blocks on demand (section 分页机制 and its block-pool demo),
wasting at most the unfilled tail of each request's last block (blog page
"vLLM 的 PagedAttention：KV cache 为什么要分页", §5.1).
"""
from __future__ import annotations


def kv_cache_bytes(layers: int, d_model: int, seq_len: int, batch: int, elem_bytes: int = 2) -> int:
    return 2 * layers * d_model * seq_len * batch * elem_bytes


def reservation_utilization(lengths, s_max: int) -> float:
    return sum(lengths) / (len(lengths) * s_max)


def paged_utilization(lengths, block_size: int) -> float:
    blocks = sum(-(-s // block_size) for s in lengths)
    return sum(lengths) / (blocks * block_size)


def serve_reserved(lengths, total_cells: int, s_max: int):
    """Admit requests in order while a full s_max reservation still fits.
    Returns (served, cells used by tokens, cells reserved)."""
    served = used = reserved = 0
    for s in lengths:
        if reserved + s_max > total_cells:
            break
        reserved += s_max
        used += s
        served += 1
    return served, used, reserved


def serve_paged(lengths, total_cells: int, block_size: int):
    """Admit requests in order while their ceil(s / block_size) blocks fit.
    Returns (served, cells used by tokens, cells held in blocks)."""
    free = total_cells // block_size
    served = used = held = 0
    for s in lengths:
        need = -(-s // block_size)
        if need > free:
            break
        free -= need
        used += s
        held += need * block_size
        served += 1
    return served, used, held
