"""CPU oracle for the fp8 KV cache -- TEST INFRASTRUCTURE ONLY.

Only the test suite and the ``cpu_baseline`` leg of ``bench.py`` may import
this module; it imports nothing from the product package.

The kernel page ("读 vLLM 的 PagedAttention kernel", §3.2) shows the cache
write taking ``kv_cache_dtype, k_scale, v_scale`` but defines no scheme.
The scheme taken here (each point is a reading, not the pages'):

* the code is 8-bit OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits; exponent field 0 is subnormal (m * 2**-9); there
  is no infinity; S.1111.111 is NaN; the largest finite magnitude is 448;
* one fp32 scale per pool and per call (``k_scale`` for K, ``v_scale`` for
  V): the stored code of an fp16 element x is encode(fp32(x) / fp32(scale)),
  the division correctly rounded in fp32 (the kernel's precision, since that
  quotient decides the code), and an element reads back as decode(code) *
  scale;
* encode rounds to the nearest representable value, ties to the even
  mantissa, and saturates finite values beyond 448 to +-448 (the fp8 cache
  stays finite); NaN encodes to 0x7F;
* the pools keep their layouts with 1-byte elements: K
  ``[num_blocks, num_kv_heads, head_size/16, block_size, 16]`` (x = 16
  elements per 16 bytes) and V ``[num_blocks, num_kv_heads, head_size,
  block_size]``;
* attention over an fp8 cache is the plain definition over the decoded,
  scaled K and V (fp64 here).
"""
from __future__ import annotations

import numpy as np

F64 = np.float64
E4M3_MAX = 448.0
NAN_CODE = 0x7F


def decode_e4m3(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8 array) as float64, from the bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(F64) - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# all 256 values, and the finite non-negative ones sorted (codes 0x00..0x7E are
# already increasing in value)
_TABLE = decode_e4m3(np.arange(256, dtype=np.uint8))
_POS = _TABLE[:0x7F]


def encode_e4m3(x) -> np.ndarray:
    """Nearest E4M3 code of each float (float32/float64 array), ties to the
    even mantissa (even code), saturating at +-448; NaN -> 0x7F.  -0.0 encodes
    to 0x80."""
    v = np.asarray(x, dtype=F64)
    out = np.empty(v.shape, dtype=np.uint8)
    flat_v = v.reshape(-1)
    flat_o = out.reshape(-1)
    nan = np.isnan(flat_v)
    a = np.minimum(np.abs(np.where(nan, 0.0, flat_v)), E4M3_MAX)
    # index of the largest representable magnitude <= a, and the next one up
    lo = np.searchsorted(_POS, a, side="right") - 1
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi != lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    neg = np.signbit(flat_v) & ~nan
    code = np.where(neg, code | 0x80, code)
    code = np.where(nan, NAN_CODE, code)
    flat_o[:] = code.astype(np.uint8)
    return out


def quantize(x_fp16, scale: float) -> np.ndarray:
    """Codes of fp16 values under a per-tensor scale: encode(fp32(x) / fp32(scale))."""
    q = np.asarray(x_fp16, dtype=np.float16).astype(np.float32) / np.float32(scale)
    return encode_e4m3(q)


def dequantize(codes, scale: float) -> np.ndarray:
    """float64 values decode(code) * scale."""
    return decode_e4m3(codes) * F64(np.float32(scale))


def reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping, block_size: int,
                          k_scale: float, v_scale: float):
    """The fp8 cache write, token by token: token i with slot s >= 0 stores
    quantize(key[i, h, d], k_scale) at k_cache[s // B, h, d // 16, s % B, d % 16]
    and quantize(value[i, h, d], v_scale) at v_cache[s // B, h, d, s % B].
    Updates the uint8 pools in place."""
    T, KVH, D = key.shape
    x = k_cache.shape[4]
    assert x == 16 and k_cache.dtype == np.uint8 and v_cache.dtype == np.uint8
    qk = quantize(key, k_scale)
    qv = quantize(value, v_scale)
    for i in range(T):
        s = int(slot_mapping[i])
        if s < 0:
            continue
        b, o = s // block_size, s % block_size
        for h in range(KVH):
            k_cache[b, h, :, o, :] = qk[i, h].reshape(D // x, x)
            v_cache[b, h, :, o] = qv[i, h]


def dequantize_pools(k_cache, v_cache, k_scale: float, v_scale: float):
    """float64 pools with the same shapes (K keeps x = 16 in its last
    dimension, which is where the layout decoding of the fp16 oracle reads x
    from), so paged_decode / partition_partials apply unchanged."""
    return dequantize(k_cache, k_scale), dequantize(v_cache, v_scale)
