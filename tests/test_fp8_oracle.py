"""Pins of the fp8 (OCP E4M3) cache oracle (CPU).

* decode: the fixed points of the OCP 8-bit format (1.0, the largest finite
  448, the smallest normal 2**-6 and subnormal 2**-9, +-0, the two NaNs), a
  strictly increasing magnitude order, and every one of the 256 codes against
  torch's own float8_e4m3fn conversion (an independent implementation);
* encode: every finite fp16 value, divided by several scales, against torch's
  float32 -> float8_e4m3fn conversion (round to nearest even) wherever the
  quotient is in range, saturation to +-448 beyond it, and a brute-force
  nearest-code check on random values;
* the cache write and the decode over an fp8 pool: token-by-token scatter of
  the codes, and values that are exactly representable come back exactly, so
  attention over the fp8 pool equals attention over the fp16 pool.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8

ALL_FP16 = np.arange(65536, dtype=np.uint16).view(np.float16)
FINITE_FP16 = ALL_FP16[np.isfinite(ALL_FP16)]


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_encode(x32):
    return torch.from_numpy(np.asarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_decode_fixed_points_of_the_format():
    d = fp8.decode_e4m3(np.array([0x38, 0x7E, 0x08, 0x01, 0x00, 0x80, 0x7F, 0xFF, 0xFE, 0x40],
                                 dtype=np.uint8))
    assert d[0] == 1.0 and d[1] == 448.0 and d[2] == 2.0 ** -6 and d[3] == 2.0 ** -9
    assert d[4] == 0.0 and d[5] == 0.0 and np.signbit(d[5])
    assert np.isnan(d[6]) and np.isnan(d[7]) and d[8] == -448.0 and d[9] == 2.0


def test_decode_all_codes_against_torch_and_order():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = fp8.decode_e4m3(codes), torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert (np.diff(ours[:0x7F]) > 0).all()


@pytest.mark.parametrize("scale", [1.0, 0.5, 1 / 3, 0.0123, 7.0, 2.0 ** -8])
def test_encode_every_fp16_against_torch(scale):
    q32 = FINITE_FP16.astype(np.float32) / np.float32(scale)
    ours = fp8.quantize(FINITE_FP16, scale)
    inr = np.abs(q32) <= 448.0
    assert np.array_equal(ours[inr], torch_encode(q32[inr]))
    big = ~inr
    assert (ours[big & (q32 > 0)] == 0x7E).all() and (ours[big & (q32 < 0)] == 0xFE).all()


def test_encode_is_the_nearest_code_ties_to_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 30, rng.standard_normal(5000) * 1e-3,
                        fp8.decode_e4m3(np.arange(0x7F, dtype=np.uint8))])       # exact codes
    # midpoints between neighbours: ties
    pos = fp8.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([x, mids, -mids])
    c = fp8.encode_e4m3(x)
    got = fp8.decode_e4m3(c)
    err = np.abs(got - np.clip(x, -448, 448))
    table = pos
    best = np.min(np.abs(np.abs(np.clip(x, -448, 448))[:, None] - table[None, :]), axis=1)
    assert np.array_equal(err, best)
    tie = np.isin(np.abs(x), mids)
    assert ((c[tie] & 1) == 0).all()                 # even mantissa on ties
    assert np.array_equal(np.signbit(got[x != 0]), np.signbit(x[x != 0]))
    assert fp8.encode_e4m3(np.array([np.nan]))[0] == 0x7F


def test_cache_write_scatter():
    rng = np.random.default_rng(1)
    T, KVH, D, B, NB = 5, 2, 32, 16, 6
    key = rng.standard_normal((T, KVH, D)).astype(np.float16)
    val = rng.standard_normal((T, KVH, D)).astype(np.float16)
    kc = np.zeros((NB, KVH, D // 16, B, 16), np.uint8)
    vc = np.zeros((NB, KVH, D, B), np.uint8)
    slots = np.array([3, 17, -1, 95, 40])
    fp8.reshape_and_cache_fp8(key, val, kc, vc, slots, B, 0.25, 0.5)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        b, o = s // B, s % B
        for h in range(KVH):
            for d in range(D):
                assert kc[b, h, d // 16, o, d % 16] == fp8.quantize(key[i, h, d], 0.25)
                assert vc[b, h, d, o] == fp8.quantize(val[i, h, d], 0.5)
    assert (kc[3:5] == 0).all() and (vc[3:5] == 0).all()      # untouched blocks


def test_exactly_representable_values_make_fp8_attention_equal_fp16():
    rng = np.random.default_rng(2)
    NB, KVH, D, B, H = 12, 2, 64, 16, 4
    codes_k = rng.integers(0, 0x7F, (NB, KVH, D // 16, B, 16)).astype(np.uint8) | \
        (rng.integers(0, 2, (NB, KVH, D // 16, B, 16)).astype(np.uint8) << 7)
    codes_k[(codes_k & 0x7F) > 0x60] &= 0xB7      # keep magnitudes moderate
    codes_v = rng.integers(0, 0x60, (NB, KVH, D, B)).astype(np.uint8)
    ks, vs = 0.125, 0.25
    dk, dv = fp8.dequantize_pools(codes_k, codes_v, ks, vs)
    # the same values as fp16 in the fp16 layout (x = 8)
    k16 = dk.transpose(0, 1, 2, 4, 3).reshape(NB, KVH, D, B).reshape(NB, KVH, D // 8, 8, B) \
        .transpose(0, 1, 2, 4, 3).astype(np.float16)
    assert np.array_equal(k16.astype(np.float64).transpose(0, 1, 2, 4, 3).reshape(NB, KVH, D, B),
                          dk.transpose(0, 1, 2, 4, 3).reshape(NB, KVH, D, B))
    v16 = dv.astype(np.float16)
    q = rng.standard_normal((2, H, D)).astype(np.float16)
    bt = np.array([[3, 7, 1], [0, 5, -1]], np.int32)
    sl = np.array([40, 20], np.int32)
    a = oracle.paged_decode(q, dk, dv, bt, sl, 0.1, B)
    b = oracle.paged_decode(q, k16, v16, bt, sl, 0.1, B)
    assert np.array_equal(a, b)
    # and re-quantizing the exact values gives the codes back
    assert np.array_equal(fp8.quantize(v16, vs), codes_v)
