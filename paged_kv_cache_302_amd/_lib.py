"""ctypes binding over libpa.so.

Argument marshalling only: every function checks dtypes, devices, shapes and
contiguity of the torch tensors it is given, passes their device pointers and
sizes to the C entry point of the same name on the current HIP stream, and
raises on a non-zero status.  All arithmetic happens in the HIP kernels; if
the library is missing, loading fails with an error instead of falling back
to anything.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY names another build of the same library (e.g. one with host-side
# sanitizers); by default the in-tree libpa.so
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_HERE, "libpa.so")

_c_int = ctypes.c_int
_c_float = ctypes.c_float
_c_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p

_SIGNATURES = {
    "pa_abi_version": ([], _c_int),
    "pa_status_str": ([_c_int], ctypes.c_char_p),
    "pa_decode_v1": ([_ptr] * 6 + [_c_int] * 7 + [_c_float, _c_int, _c_float, _c_float, _ptr], _c_int),
    "pa_v2_max_partitions": ([_c_int, _c_int], _c_int),
    "pa_decode_v2": ([_ptr] * 8 + [_c_int] * 9 + [_c_float, _c_int, _c_float, _c_float, _ptr], _c_int),
    "pa_decode_v2_shared": ([_ptr] * 8 + [_c_int] * 9 + [_c_float, _c_int, _c_float, _c_float, _ptr],
                            _c_int),
    "pa_reduce": ([_ptr] * 5 + [_c_int] * 5 + [_ptr], _c_int),
    "pa_decode_v2_noalloc": ([_ptr] * 6 + [_c_int] * 9 + [_c_float, _c_int, _c_float, _c_float, _ptr],
                             _c_int),
    "pa_prefill": ([_ptr] * 7 + [_c_int] * 9 + [_c_float, _c_int, _c_float, _c_float, _ptr], _c_int),
    "pa_reshape_and_cache": ([_ptr] * 5 + [_c_int] * 5 + [_c_i64, _c_i64, _c_int, _c_float, _c_float,
                                                         _ptr], _c_int),
    "pa_gather_kv": ([_ptr] * 7 + [_c_int] * 7 + [_ptr], _c_int),
    # block manager (host) and its device block copy -- include/pa_blocks.h
    "pa_bm_create": ([_c_int, _c_int], _ptr),
    "pa_bm_destroy": ([_ptr], None),
    "pa_bm_add_sequence": ([_ptr, _c_i64, _c_int, _ptr], _c_int),
    "pa_bm_fork": ([_ptr, _c_i64, _c_i64], _c_int),
    "pa_bm_free_sequence": ([_ptr, _c_i64], _c_int),
    "pa_bm_append_slots": ([_ptr, _ptr, _c_int, _ptr, _ptr, _c_int, _ptr], _c_int),
    "pa_bm_block_tables": ([_ptr, _ptr, _c_int, _ptr, _c_int, ctypes.c_int32, _ptr], _c_int),
    "pa_bm_num_free_blocks": ([_ptr], _c_int),
    "pa_bm_num_sequences": ([_ptr], _c_int),
    "pa_bm_seq_len": ([_ptr, _c_i64], _c_int),
    "pa_bm_refcount": ([_ptr, _c_int], _c_int),
    "pa_copy_blocks": ([_ptr] * 3 + [_c_int] * 6 + [_ptr], _c_int),
}

_lib = None


class PagedAttentionError(RuntimeError):
    pass


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise PagedAttentionError(
                f"{path} is missing: build it with `python -m paged_kv_cache_302_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def exported_symbols() -> list:
    return list(_SIGNATURES)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        msg = load_library().pa_status_str(rc).decode()
        raise PagedAttentionError(f"{what}: status {rc} ({msg})")


def _stream(t: torch.Tensor, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(handle)


def _want(t: torch.Tensor, name: str, dtype, ndim: Optional[int] = None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _p(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


# kv_cache_dtype codes of include/pa.h
PA_KV_FP16 = 0
PA_KV_FP8_E4M3 = 1
_FP8_STORAGE = (torch.uint8, torch.float8_e4m3fn)


def kv_dtype_of(k_cache: torch.Tensor) -> int:
    """PA_KV_FP16 for fp16 pools, PA_KV_FP8_E4M3 for uint8 / float8_e4m3fn pools."""
    if k_cache.dtype == torch.float16:
        return PA_KV_FP16
    if k_cache.dtype in _FP8_STORAGE:
        return PA_KV_FP8_E4M3
    raise TypeError(f"unsupported cache dtype {k_cache.dtype} (fp16, or fp8 E4M3 as uint8/float8_e4m3fn)")


def _cache_dims(k_cache: torch.Tensor, v_cache: torch.Tensor):
    kvd = kv_dtype_of(k_cache)
    _want(k_cache, "k_cache", k_cache.dtype, 5)
    _want(v_cache, "v_cache", k_cache.dtype, 4, k_cache.device)
    NB, KVH, Dx, B, x = k_cache.shape
    D = Dx * x
    want_x = 8 if kvd == PA_KV_FP16 else 16
    if x != want_x:
        raise ValueError(f"k_cache last dim must be x = {want_x} for this dtype")
    if tuple(v_cache.shape) != (NB, KVH, D, B):
        raise ValueError(f"v_cache shape {tuple(v_cache.shape)} does not match k_cache {tuple(k_cache.shape)}")
    return NB, KVH, D, B


def _decode_common(q, k_cache, v_cache, block_tables, seq_lens):
    NB, KVH, D, B = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _want(q, "q", torch.float16, 3, dev)
    _want(block_tables, "block_tables", torch.int32, 2, dev)
    _want(seq_lens, "seq_lens", torch.int32, 1, dev)
    S, H, Dq = q.shape
    if Dq != D:
        raise ValueError(f"q head_size {Dq} != cache head_size {D}")
    if block_tables.shape[0] != S or seq_lens.shape[0] != S:
        raise ValueError("block_tables / seq_lens must have num_seqs rows")
    return S, H, KVH, D, B, NB, block_tables.shape[1]


def pa_abi_version() -> int:
    return load_library().pa_abi_version()


def pa_v2_max_partitions(max_seq_len: int, partition_size: int) -> int:
    return load_library().pa_v2_max_partitions(int(max_seq_len), int(partition_size))


def pa_decode_v1(out, q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                 k_scale: float = 1.0, v_scale: float = 1.0, stream=None):
    """out[S,H,D] fp32 <- paged decode attention (no partitioning).  The
    scales apply to fp8 pools only."""
    S, H, KVH, D, B, NB, MB = _decode_common(q, k_cache, v_cache, block_tables, seq_lens)
    _want(out, "out", torch.float32, 3, q.device)
    if tuple(out.shape) != (S, H, D):
        raise ValueError("out must be [num_seqs, num_heads, head_size]")
    lib = load_library()
    rc = lib.pa_decode_v1(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables), _p(seq_lens),
                          S, H, KVH, D, B, MB, NB, float(scale), kv_dtype_of(k_cache),
                          float(k_scale), float(v_scale), _stream(q, stream))
    _check(rc, "pa_decode_v1")
    return out


def pa_decode_v2(tmp_out, exp_sums, max_logits, q, k_cache, v_cache, block_tables, seq_lens,
                 scale: float, partition_size: int, k_scale: float = 1.0, v_scale: float = 1.0,
                 stream=None, shared_blocks: bool = False):
    """Per-partition partials (tmp_out[S,P,H,D], exp_sums/max_logits[S,P,H]).
    shared_blocks=True calls pa_decode_v2_shared (same results, for batches
    whose block tables share physical blocks)."""
    S, H, KVH, D, B, NB, MB = _decode_common(q, k_cache, v_cache, block_tables, seq_lens)
    _want(tmp_out, "tmp_out", torch.float32, 4, q.device)
    _want(exp_sums, "exp_sums", torch.float32, 3, q.device)
    _want(max_logits, "max_logits", torch.float32, 3, q.device)
    P = tmp_out.shape[1]
    if tuple(tmp_out.shape) != (S, P, H, D) or tuple(exp_sums.shape) != (S, P, H) or \
            tuple(max_logits.shape) != (S, P, H):
        raise ValueError("v2 scratch shapes must be [S,P,H,D] and [S,P,H]")
    lib = load_library()
    name = "pa_decode_v2_shared" if shared_blocks else "pa_decode_v2"
    rc = getattr(lib, name)(_p(tmp_out), _p(exp_sums), _p(max_logits), _p(q), _p(k_cache),
                            _p(v_cache), _p(block_tables), _p(seq_lens), S, H, KVH, D, B, MB, NB,
                            P, int(partition_size), float(scale), kv_dtype_of(k_cache),
                            float(k_scale), float(v_scale), _stream(q, stream))
    _check(rc, name)


def pa_decode_v2_shared(tmp_out, exp_sums, max_logits, q, k_cache, v_cache, block_tables,
                        seq_lens, scale: float, partition_size: int, k_scale: float = 1.0,
                        v_scale: float = 1.0, stream=None):
    """pa_decode_v2 for batches whose sequences share K/V blocks (include/pa.h)."""
    pa_decode_v2(tmp_out, exp_sums, max_logits, q, k_cache, v_cache, block_tables, seq_lens,
                 scale, partition_size, k_scale, v_scale, stream, shared_blocks=True)


def pa_decode_v2_noalloc(out, q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                         partition_size: int, max_num_partitions: int, k_scale: float = 1.0,
                         v_scale: float = 1.0, stream=None):
    """out[S,H,D] fp32 <- pa_decode_v2 + pa_reduce with the partials in the
    library's fixed device scratch (no allocation; include/pa.h)."""
    S, H, KVH, D, B, NB, MB = _decode_common(q, k_cache, v_cache, block_tables, seq_lens)
    _want(out, "out", torch.float32, 3, q.device)
    if tuple(out.shape) != (S, H, D):
        raise ValueError("out must be [num_seqs, num_heads, head_size]")
    lib = load_library()
    rc = lib.pa_decode_v2_noalloc(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables),
                                  _p(seq_lens), S, H, KVH, D, B, MB, NB, int(max_num_partitions),
                                  int(partition_size), float(scale), kv_dtype_of(k_cache),
                                  float(k_scale), float(v_scale), _stream(q, stream))
    _check(rc, "pa_decode_v2_noalloc")
    return out


def pa_prefill(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
               max_query_len: int, scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
               stream=None):
    """out[T,H,D] fp32 <- causal attention of the last n_s tokens of every
    sequence (rows query_start_loc[s] ..) over its paged K/V."""
    NB, KVH, D, B = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _want(q, "q", torch.float16, 3, dev)
    _want(out, "out", torch.float32, 3, dev)
    _want(block_tables, "block_tables", torch.int32, 2, dev)
    _want(seq_lens, "seq_lens", torch.int32, 1, dev)
    _want(query_start_loc, "query_start_loc", torch.int32, 1, dev)
    T, H, Dq = q.shape
    S = seq_lens.shape[0]
    if Dq != D or tuple(out.shape) != (T, H, D):
        raise ValueError("q and out must be [total_q, num_heads, head_size] of the cache's head_size")
    if block_tables.shape[0] != S or query_start_loc.shape[0] != S + 1:
        raise ValueError("block_tables [S, ...] and query_start_loc [S + 1] must match seq_lens [S]")
    lib = load_library()
    rc = lib.pa_prefill(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables), _p(seq_lens),
                        _p(query_start_loc), S, T, H, KVH, D, B, block_tables.shape[1], NB,
                        int(max_query_len), float(scale), kv_dtype_of(k_cache), float(k_scale),
                        float(v_scale), _stream(q, stream))
    _check(rc, "pa_prefill")
    return out


def pa_reduce(out, tmp_out, exp_sums, max_logits, seq_lens, partition_size: int, stream=None):
    """out[S,H,D] <- log-sum-exp merge of the v2 partials."""
    dev = tmp_out.device
    _want(tmp_out, "tmp_out", torch.float32, 4, dev)
    _want(exp_sums, "exp_sums", torch.float32, 3, dev)
    _want(max_logits, "max_logits", torch.float32, 3, dev)
    _want(seq_lens, "seq_lens", torch.int32, 1, dev)
    _want(out, "out", torch.float32, 3, dev)
    S, P, H, D = tmp_out.shape
    if tuple(out.shape) != (S, H, D) or seq_lens.shape[0] != S or \
            tuple(exp_sums.shape) != (S, P, H) or tuple(max_logits.shape) != (S, P, H):
        raise ValueError("out must be [S,H,D], partials [S,P,H,D] / [S,P,H], seq_lens [S]")
    lib = load_library()
    rc = lib.pa_reduce(_p(out), _p(tmp_out), _p(exp_sums), _p(max_logits), _p(seq_lens), S, H, D,
                       P, int(partition_size), _stream(out, stream))
    _check(rc, "pa_reduce")
    return out


def pa_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, k_scale: float = 1.0,
                         v_scale: float = 1.0, stream=None):
    """Scatter key/value [T,KVH,D] into the pools at slot_mapping[T] (int64);
    into fp8 pools as E4M3 codes of key / k_scale and value / v_scale."""
    NB, KVH, D, B = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    for name, t in (("key", key), ("value", value)):
        if t.dtype != torch.float16 or t.dim() != 3 or t.device != dev:
            raise ValueError(f"{name} must be fp16 [T, KVH, D] on {dev}")
        if t.stride(2) != 1 or t.stride(1) != D:
            raise ValueError(f"{name} must have contiguous heads (token stride may differ)")
    _want(slot_mapping, "slot_mapping", torch.int64, 1, dev)
    T = key.shape[0]
    if tuple(key.shape) != (T, KVH, D) or tuple(value.shape) != (T, KVH, D) or slot_mapping.shape[0] != T:
        raise ValueError("key/value must be [T, num_kv_heads, head_size], slot_mapping [T]")
    lib = load_library()
    rc = lib.pa_reshape_and_cache(_p(key), _p(value), _p(k_cache), _p(v_cache), _p(slot_mapping), T, KVH,
                               D, B, NB, key.stride(0) if T else KVH * D,
                               value.stride(0) if T else KVH * D, kv_dtype_of(k_cache),
                               float(k_scale), float(v_scale), _stream(key, stream))
    _check(rc, "pa_reshape_and_cache")


# the pages' name of the operation
reshape_and_cache = pa_reshape_and_cache


def pa_gather_kv(k_out, v_out, k_cache, v_cache, block_tables, seq_lens, cu_seq_lens, stream=None):
    """k_out/v_out [sum L, KVH, D] <- every sequence's K/V in logical order."""
    NB, KVH, D, B = _cache_dims(k_cache, v_cache)
    dev = k_cache.device
    _want(block_tables, "block_tables", torch.int32, 2, dev)
    _want(seq_lens, "seq_lens", torch.int32, 1, dev)
    _want(cu_seq_lens, "cu_seq_lens", torch.int64, 1, dev)
    _want(k_out, "k_out", k_cache.dtype, 3, dev)
    _want(v_out, "v_out", k_cache.dtype, 3, dev)
    S, MB = block_tables.shape
    lib = load_library()
    rc = lib.pa_gather_kv(_p(k_out), _p(v_out), _p(k_cache), _p(v_cache), _p(block_tables),
                          _p(seq_lens), _p(cu_seq_lens), S, KVH, D, B, MB, NB,
                          kv_dtype_of(k_cache), _stream(k_cache, stream))
    _check(rc, "pa_gather_kv")


# --------------------------------------------------------------------------
# Conveniences that allocate their outputs with torch (plumbing only)
# --------------------------------------------------------------------------

def paged_attention_v1(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                       k_scale: float = 1.0, v_scale: float = 1.0):
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    return pa_decode_v1(out, q, k_cache, v_cache, block_tables, seq_lens, scale, k_scale, v_scale)


def v2_scratch(num_seqs: int, num_heads: int, head_size: int, max_num_partitions: int, device):
    tmp = torch.empty((num_seqs, max_num_partitions, num_heads, head_size), dtype=torch.float32,
                      device=device)
    es = torch.empty((num_seqs, max_num_partitions, num_heads), dtype=torch.float32, device=device)
    ml = torch.empty_like(es)
    return tmp, es, ml


def paged_attention_v2(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                       partition_size: int = 512, max_seq_len: Optional[int] = None,
                       k_scale: float = 1.0, v_scale: float = 1.0, shared_blocks: bool = False):
    S, H, D = q.shape
    if max_seq_len is None:
        max_seq_len = block_tables.shape[1] * k_cache.shape[3]
    P = pa_v2_max_partitions(max_seq_len, partition_size)
    tmp, es, ml = v2_scratch(S, H, D, P, q.device)
    pa_decode_v2(tmp, es, ml, q, k_cache, v_cache, block_tables, seq_lens, scale, partition_size,
                 k_scale, v_scale, shared_blocks=shared_blocks)
    out = torch.empty((S, H, D), dtype=torch.float32, device=q.device)
    return pa_reduce(out, tmp, es, ml, seq_lens, partition_size)


def split_kv_cache(kv_cache: torch.Tensor, num_kv_heads: int, head_size: int):
    """Views of a [2, num_blocks, num_kv_heads * head_size * block_size] fp16
    buffer as the x-packed K pool and the V pool (the split_kv_cache view of
    page "读 vLLM 的 PagedAttention kernel", §4)."""
    x = 16 // kv_cache.element_size()
    nb = kv_cache.shape[1]
    k = kv_cache[0].view(nb, num_kv_heads, head_size // x, -1, x)
    v = kv_cache[1].view(nb, num_kv_heads, head_size, -1)
    return k, v


# -- block manager and copy-on-write -----------------------------------------

PA_ERR_NO_SPACE = -5


class BlockManagerError(PagedAttentionError):
    pass


class BlockManager:
    """Host block manager of libpa.so (include/pa_blocks.h): allocation on
    demand, fork with reference counts, copy-on-write, release.  Marshalling
    only -- every rule is applied by the native code."""

    def __init__(self, num_blocks: int, block_size: int = 16):
        self._lib = load_library()
        self._h = self._lib.pa_bm_create(int(num_blocks), int(block_size))
        if not self._h:
            raise BlockManagerError("pa_bm_create failed (bad sizes or out of host memory)")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._lib.pa_bm_destroy(h)

    def _rc(self, rc: int, what: str) -> None:
        if rc != 0:
            msg = self._lib.pa_status_str(rc).decode()
            raise BlockManagerError(f"{what}: status {rc} ({msg})")

    def add_sequence(self, seq_id: int, num_tokens: int):
        """Allocate a new sequence's blocks; returns the slots of its tokens (int64 array)."""
        import numpy as np
        slots = np.empty(max(int(num_tokens), 0), dtype=np.int64)
        self._rc(self._lib.pa_bm_add_sequence(self._h, int(seq_id), int(num_tokens),
                                              slots.ctypes.data if slots.size else None),
                 "add_sequence")
        return slots

    def fork(self, parent: int, child: int) -> None:
        self._rc(self._lib.pa_bm_fork(self._h, int(parent), int(child)), "fork")

    def free_sequence(self, seq_id: int) -> None:
        self._rc(self._lib.pa_bm_free_sequence(self._h, int(seq_id)), "free_sequence")

    def append_slots(self, seq_ids):
        """One decode step: returns (slots int64 [n], copies int32 [k, 2])."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.size
        slots = np.empty(n, dtype=np.int64)
        copies = np.empty((max(n, 1), 2), dtype=np.int32)
        nc = ctypes.c_int(0)
        self._rc(self._lib.pa_bm_append_slots(self._h, ids.ctypes.data if n else None, n,
                                              slots.ctypes.data if n else None,
                                              copies.ctypes.data, n, ctypes.byref(nc)),
                 "append_slots")
        return slots, copies[:nc.value].copy()

    def block_tables(self, seq_ids, width: int, pad: int = -1):
        """(tables int32 [n, width], seq_lens int32 [n]) for a batch."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.size
        tables = np.empty((n, width), dtype=np.int32)
        lens = np.empty(n, dtype=np.int32)
        self._rc(self._lib.pa_bm_block_tables(self._h, ids.ctypes.data if n else None, n,
                                              tables.ctypes.data if n else None, int(width),
                                              int(pad), lens.ctypes.data if n else None),
                 "block_tables")
        return tables, lens

    def table(self, seq_id: int):
        n = self.seq_len(seq_id)
        if n < 0:
            raise BlockManagerError(f"no sequence {seq_id}")
        width = max(-(-n // self.block_size), 1)
        t, _ = self.block_tables([seq_id], width)
        return [int(x) for x in t[0, :-(-n // self.block_size)]]

    def num_free_blocks(self) -> int:
        return self._lib.pa_bm_num_free_blocks(self._h)

    def num_sequences(self) -> int:
        return self._lib.pa_bm_num_sequences(self._h)

    def seq_len(self, seq_id: int) -> int:
        return self._lib.pa_bm_seq_len(self._h, int(seq_id))

    def refcount_of(self, block: int) -> int:
        return self._lib.pa_bm_refcount(self._h, int(block))

    @property
    def refcount(self):
        return [self.refcount_of(b) for b in range(self.num_blocks)]


def pa_copy_blocks(k_cache, v_cache, block_pairs, stream=None):
    """Copy-on-write on the device: block_pairs int32 [n, 2] (source, destination)."""
    NB, KVH, D, B = _cache_dims(k_cache, v_cache)
    _want(block_pairs, "block_pairs", torch.int32, 2, k_cache.device)
    if block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [num_pairs, 2]")
    rc = load_library().pa_copy_blocks(_p(k_cache), _p(v_cache), _p(block_pairs),
                                    block_pairs.shape[0], KVH, D, B, NB, kv_dtype_of(k_cache),
                                    _stream(k_cache, stream))
    _check(rc, "pa_copy_blocks")


copy_blocks = pa_copy_blocks
