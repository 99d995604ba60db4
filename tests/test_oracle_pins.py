"""Pins for the CPU oracle: values the pages print, closed forms, invariants,
library special cases and brute force on tiny inputs.  CPU only.

Each pin is chosen so that a plausible mistake in the oracle (a dropped scale,
a transposed layout index, a wrong head mapping, an off-by-one at the partly
filled last block, a wrong merge weight) fails at least one of them; the
mutation tests at the end plant such mistakes in the oracle and check that.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from oracle import paged_attention as opa

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------------------
# Building paged layouts independently of the oracle: the pages define the
# pools by their shapes (kernel page §3.1); here they are built with numpy
# reshapes/transposes of contiguous data, not with the oracle's index helpers.
# ---------------------------------------------------------------------------

def build_paged(Ks, Vs, block_tables, num_blocks, block_size, x, fill=0.0, dtype=np.float64):
    """Ks/Vs: per sequence arrays [KVH, L_s, D].  Returns k_cache, v_cache."""
    KVH, _, D = Ks[0].shape
    kc = np.full((num_blocks, KVH, D // x, block_size, x), fill, dtype=dtype)
    vc = np.full((num_blocks, KVH, D, block_size), fill, dtype=dtype)
    for s, (K, V) in enumerate(zip(Ks, Vs)):
        L = K.shape[1]
        nb = -(-L // block_size)
        pad = nb * block_size - L
        Kp = np.concatenate([K, np.full((KVH, pad, D), fill)], axis=1)
        Vp = np.concatenate([V, np.full((KVH, pad, D), fill)], axis=1)
        # [KVH, nb, B, D/x, x] -> [nb, KVH, D/x, B, x]
        kb = Kp.reshape(KVH, nb, block_size, D // x, x).transpose(1, 0, 3, 2, 4)
        vb = Vp.reshape(KVH, nb, block_size, D).transpose(1, 0, 3, 2)
        for i in range(nb):
            b = block_tables[s][i]
            if i == nb - 1 and pad:
                f = block_size - pad
                kc[b, :, :, :f, :] = kb[i][:, :, :f, :]
                vc[b, :, :, :f] = vb[i][:, :, :f]
            else:
                kc[b] = kb[i]
                vc[b] = vb[i]
    return kc, vc


def random_case(rng, S, H, KVH, D, B, x, lens, num_blocks=None, dtype=np.float64):
    Ks = [rng.standard_normal((KVH, L, D)) for L in lens]
    Vs = [rng.standard_normal((KVH, L, D)) for L in lens]
    need = sum(-(-L // B) for L in lens)
    NB = num_blocks or need + 3
    perm = rng.permutation(NB)
    mb = max(1, max(-(-L // B) for L in lens))
    bt = np.full((S, mb), -1, dtype=np.int32)
    pos = 0
    for s, L in enumerate(lens):
        nb = -(-L // B)
        bt[s, :nb] = perm[pos:pos + nb]
        pos += nb
    kc, vc = build_paged(Ks, Vs, bt, NB, B, x, dtype=dtype)
    q = rng.standard_normal((S, H, D))
    return q, Ks, Vs, bt, kc, vc


def sdpa(q_row, K, V, scale):
    """Library attention (torch SDPA, fp64, grouped-query mapping built in):
    q_row [H, D], K/V [KVH, L, D] -> [H, D]."""
    qt = torch.from_numpy(np.ascontiguousarray(q_row, dtype=np.float64))[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(K, dtype=np.float64))[None]
    vt = torch.from_numpy(np.ascontiguousarray(V, dtype=np.float64))[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
    return o[0, :, 0, :].numpy()


# ---------------------------------------------------------------------------
# P1: the pages' worked example
# ---------------------------------------------------------------------------

def load_worked_example():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        return json.load(f)


def worked_example_case(x):
    ex = load_worked_example()
    D, B, L = ex["head_size"], ex["block_size"], ex["seq_len"]
    K = np.array(ex["K"])[None]
    V = np.array(ex["V"])[None]
    bt = np.array([ex["block_table"]], dtype=np.int32)
    kc, vc = build_paged([K], [V], bt, 5, B, x, fill=np.nan)
    q = np.array(ex["q"])[None, None, :]
    return ex, q, kc, vc, bt, np.array([L], dtype=np.int32)


@pytest.mark.parametrize("x", [1, 2, 4])
@pytest.mark.parametrize("fast", [False, True])
def test_worked_example_matches_page(x, fast):
    ex, q, kc, vc, bt, lens = worked_example_case(x)
    out = oracle.paged_decode(q, kc, vc, bt, lens, ex["scale"], ex["block_size"], fast=fast)
    got = np.round(out[0, 0], ex["expected_decimals"])
    np.testing.assert_allclose(got, ex["expected_out"], rtol=0, atol=1e-12)
    assert np.isfinite(out).all()  # NaN in the half-empty block's unused slots is never read


def test_worked_example_online_and_partitions():
    ex, q, kc, vc, bt, lens = worked_example_case(2)
    K, V = oracle.gather_sequence(kc, vc, bt[0], 6, 0, ex["block_size"])
    on = oracle.online_block_attention(q[0], K, V, ex["scale"], ex["block_size"])
    np.testing.assert_allclose(np.round(on[0], 6), ex["expected_out"], atol=1e-12)
    for ps in (4, 8):
        t, e, m = oracle.partition_partials(q, kc, vc, bt, lens, ex["scale"], ex["block_size"], ps, 2)
        out = oracle.lse_merge(t, e, m, lens, ps)
        np.testing.assert_allclose(np.round(out[0, 0], 6), ex["expected_out"], atol=1e-12)


# ---------------------------------------------------------------------------
# P2: brute force -- oracle(paged) == library dense attention(contiguous)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,KVH,D,B,x", [
    (4, 4, 8, 4, 2), (8, 2, 16, 4, 8), (7, 1, 8, 16, 4), (6, 3, 64, 16, 8), (16, 4, 32, 16, 1),
])
def test_oracle_equals_dense_library_attention(H, KVH, D, B, x):
    rng = np.random.default_rng(100 + H * 7 + D)
    lens = [1, B - 1, B, B + 1, 3 * B + 5]
    S = len(lens)
    q, Ks, Vs, bt, kc, vc = random_case(rng, S, H, KVH, D, B, x, lens)
    scale = 1.0 / math.sqrt(D)
    for fast in (False, True):
        out = oracle.paged_decode(q, kc, vc, bt, np.array(lens), scale, B, fast=fast)
        for s in range(S):
            ref = sdpa(q[s], Ks[s], Vs[s], scale)
            np.testing.assert_allclose(out[s], ref, rtol=0, atol=1e-12)


def test_gather_sequence_forms_agree_and_restore_order():
    rng = np.random.default_rng(7)
    lens = [37, 16, 1]
    q, Ks, Vs, bt, kc, vc = random_case(rng, 3, 4, 2, 16, 16, 8, lens)
    for s, L in enumerate(lens):
        for h in range(2):
            K1, V1 = oracle.gather_sequence(kc, vc, bt[s], L, h, 16)
            K2, V2 = oracle.gather_sequence_fast(kc, vc, bt[s], L, h, 16)
            np.testing.assert_array_equal(K1, Ks[s][h])
            np.testing.assert_array_equal(V1, Vs[s][h])
            np.testing.assert_array_equal(K2, Ks[s][h])
            np.testing.assert_array_equal(V2, Vs[s][h])


def test_k_layout_matches_split_kv_cache_view():
    """The x-split K layout is the view key_cache.view(NB, KVH, D//x, -1, x)
    of a flat per-(block, head) buffer of D*B elements (kernel page §4,
    split_kv_cache); for the token in slot o, dimension d sits at flat offset
    (d // x) * B * x + o * x + d % x."""
    NB, KVH, D, B, x = 3, 2, 16, 4, 8
    flat = np.arange(NB * KVH * D * B, dtype=np.float64).reshape(NB, KVH, D * B)
    view = torch.from_numpy(flat).view(NB, KVH, D // x, -1, x).numpy()
    for b in range(NB):
        for h in range(KVH):
            for o in range(B):
                kv = oracle.key_vector(view, b, h, o)
                expect = [flat[b, h, (d // x) * B * x + o * x + d % x] for d in range(D)]
                np.testing.assert_array_equal(kv, expect)


# ---------------------------------------------------------------------------
# P3: the online recurrence == the two-pass definition
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("L,B", [(1, 16), (15, 16), (16, 16), (100, 16), (257, 4)])
def test_online_recurrence_equals_two_pass(L, B):
    rng = np.random.default_rng(L)
    q = rng.standard_normal((5, 32)) * 2
    K = rng.standard_normal((L, 32))
    V = rng.standard_normal((L, 32))
    a = oracle.attention(q, K, V, 0.3)
    b = oracle.online_block_attention(q, K, V, 0.3, B)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# P4-P9: closed forms and invariants
# ---------------------------------------------------------------------------

def test_seq_len_one_returns_v_exactly():
    rng = np.random.default_rng(3)
    q, Ks, Vs, bt, kc, vc = random_case(rng, 2, 4, 2, 16, 16, 8, [1, 1])
    out = oracle.paged_decode(q, kc, vc, bt, np.array([1, 1]), 0.25, 16)
    for s in range(2):
        for h in range(4):
            np.testing.assert_array_equal(out[s, h], Vs[s][h // 2][0])


def test_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(4)
    L, D = 45, 16
    k = rng.standard_normal(D)
    K = np.tile(k, (L, 1))[None]
    V = rng.standard_normal((1, L, D))
    bt = np.array([[4, 0, 2]], dtype=np.int32)
    kc, vc = build_paged([K], [V], bt, 5, 16, 8, fill=np.nan)
    q = rng.standard_normal((1, 3, D)) * 3
    out = oracle.paged_decode(q, kc, vc, bt, np.array([L]), 0.7, 16)
    for h in range(3):
        np.testing.assert_allclose(out[0, h], V[0].mean(axis=0), rtol=0, atol=1e-13)


def test_permuting_physical_ids_leaves_output_unchanged():
    rng = np.random.default_rng(5)
    lens = [50, 17, 33]
    q, Ks, Vs, bt, kc, vc = random_case(rng, 3, 4, 2, 16, 16, 8, lens, num_blocks=12)
    out = oracle.paged_decode(q, kc, vc, bt, np.array(lens), 0.3, 16)
    perm = rng.permutation(12)             # new id of old block b is perm[b]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    out2 = oracle.paged_decode(q, kc2, vc2, bt2, np.array(lens), 0.3, 16)
    np.testing.assert_array_equal(out, out2)


def test_partial_block_and_poison_are_never_read():
    rng = np.random.default_rng(6)
    lens = [19, 1, 32, 47]
    q, Ks, Vs, bt, kc, vc = random_case(rng, 4, 8, 2, 32, 16, 8, lens)
    lens = np.array(lens)
    clean = oracle.paged_decode(q, kc, vc, bt, lens, 0.2, 16)
    kp, vp = kc.copy(), vc.copy()
    # float64 pools here: poison with NaN directly
    fill = oracle.used_fill(bt, lens, 16)
    for b in range(kp.shape[0]):
        f = fill.get(b, 0)
        kp[b, :, :, f:, :] = np.nan
        vp[b, :, :, f:] = np.nan
    for fast in (False, True):
        out = oracle.paged_decode(q, kp, vp, bt, lens, 0.2, 16, fast=fast)
        assert np.isfinite(out).all()
        np.testing.assert_array_equal(out, clean)


def test_fp16_poison_helper_marks_exactly_unattended_slots():
    rng = np.random.default_rng(8)
    lens = np.array([19, 33], dtype=np.int32)
    q, Ks, Vs, bt, kc, vc = random_case(rng, 2, 2, 1, 16, 16, 8, list(lens), num_blocks=8,
                                        dtype=np.float16)
    kc = kc.astype(np.float16)
    vc = vc.astype(np.float16)
    before = oracle.paged_decode(q, kc, vc, bt, lens, 0.25, 16)
    oracle.poison_unused(kc, vc, bt, lens, 16)
    assert np.isnan(kc.astype(np.float32)).any()
    after = oracle.paged_decode(q, kc, vc, bt, lens, 0.25, 16)
    np.testing.assert_array_equal(before, after)
    n_nan_v = np.isnan(vc.astype(np.float32)).sum()
    used = sum(int(L) for L in lens)
    assert n_nan_v == vc.size - used * 1 * 16


def test_shift_and_linearity_in_v():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((4, 16))
    K = rng.standard_normal((70, 16))
    V = rng.standard_normal((70, 16))
    V2 = rng.standard_normal((70, 16))
    base = oracle.attention(q, K, V, 0.5)
    np.testing.assert_allclose(oracle.attention(q, K, V + 2.5, 0.5), base + 2.5, atol=1e-12)
    np.testing.assert_allclose(oracle.attention(q, K, 3 * V - V2, 0.5),
                               3 * base - oracle.attention(q, K, V2, 0.5), atol=1e-12)


def test_needle_closed_form():
    """All keys zero except one needle k* = alpha q/|q|: every other score is
    exactly 0, the needle's is z* = scale*alpha*|q|, so
    out = (e^{z*} v* + sum_{t != *} v_t) / (e^{z*} + L - 1)."""
    rng = np.random.default_rng(10)
    L, D, star = 300, 64, 123
    q = rng.standard_normal(D)
    alpha = 8.0
    K = np.zeros((L, D))
    K[star] = alpha * q / np.linalg.norm(q)
    V = rng.standard_normal((L, D))
    bt = np.array([rng.permutation(40)[:19]], dtype=np.int32)
    kc, vc = build_paged([K[None]], [V[None]], bt, 40, 16, 8, fill=np.nan)
    scale = 1 / math.sqrt(D)
    out = oracle.paged_decode(q[None, None], kc, vc, bt, np.array([L]), scale, 16)[0, 0]
    zs = scale * alpha * np.linalg.norm(q)
    expect = (math.exp(zs) * V[star] + (V.sum(0) - V[star])) / (math.exp(zs) + L - 1)
    np.testing.assert_allclose(out, expect, rtol=1e-12, atol=1e-13)


def test_zero_length_sequence_gives_zeros():
    rng = np.random.default_rng(11)
    q, Ks, Vs, bt, kc, vc = random_case(rng, 2, 2, 1, 16, 16, 8, [5, 3])
    out = oracle.paged_decode(q, kc, vc, bt, np.array([0, 3]), 0.25, 16)
    np.testing.assert_array_equal(out[0], 0.0)
    t, e, m = oracle.partition_partials(q, kc, vc, bt, np.array([0, 3]), 0.25, 16, 16, 1)
    merged = oracle.lse_merge(t, e, m, np.array([0, 3]), 16)
    np.testing.assert_array_equal(merged[0], 0.0)


# ---------------------------------------------------------------------------
# P10: partitions and the log-sum-exp merge
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ps", [16, 32, 64, 512])
def test_partition_merge_equals_unpartitioned(ps):
    rng = np.random.default_rng(ps)
    lens = [1, 16, 17, 100, 513, 640]
    S = len(lens)
    q, Ks, Vs, bt, kc, vc = random_case(rng, S, 8, 2, 32, 16, 8, lens)
    lens = np.array(lens)
    P = max(oracle.num_partitions(L, ps) for L in lens)
    t, e, m = oracle.partition_partials(q, kc, vc, bt, lens, 0.2, 16, ps, P)
    merged = oracle.lse_merge(t, e, m, lens, ps)
    full = oracle.paged_decode(q, kc, vc, bt, lens, 0.2, 16)
    np.testing.assert_allclose(merged, full, rtol=0, atol=1e-12)


def test_partials_match_library_on_each_slice():
    """Each partial o_p is library attention over that partition's tokens; and
    m_p + log(l_p) is the library log-sum-exp of those scaled scores."""
    rng = np.random.default_rng(12)
    L, ps, D = 200, 64, 16
    q, Ks, Vs, bt, kc, vc = random_case(rng, 1, 4, 1, D, 16, 8, [L])
    t, e, m = oracle.partition_partials(q, kc, vc, bt, np.array([L]), 0.4, 16, ps, 4)
    qt = torch.from_numpy(q[0])
    for p in range(4):
        lo, hi = p * ps, min((p + 1) * ps, L)
        ref = sdpa(q[0], Ks[0][:, lo:hi], Vs[0][:, lo:hi], 0.4)
        np.testing.assert_allclose(t[0, :, p], ref, atol=1e-12)
        z = 0.4 * (qt @ torch.from_numpy(Ks[0][0, lo:hi]).T).numpy()   # [H, n]
        np.testing.assert_allclose(m[0, :, p] + np.log(e[0, :, p]),
                                   scipy.special.logsumexp(z, axis=1), atol=1e-12)
        assert (e[0, :, p] >= 1.0).all() and (e[0, :, p] <= hi - lo).all()


def test_merge_is_order_free_associative_and_ignores_empty_partitions():
    rng = np.random.default_rng(13)
    P, D = 6, 8
    o = rng.standard_normal((1, 1, P, D))
    m = rng.standard_normal((1, 1, P)) * 5
    l = rng.uniform(1, 30, size=(1, 1, P))
    ref = oracle.lse_merge(o, l, m, np.array([P * 16]), 16)
    perm = rng.permutation(P)
    np.testing.assert_allclose(oracle.lse_merge(o[:, :, perm], l[:, :, perm], m[:, :, perm],
                                                np.array([P * 16]), 16), ref, atol=1e-13)
    # merge (0..2) and (3..5) first, then merge the two results
    parts = []
    for a, b in ((0, 3), (3, 6)):
        sub = oracle.lse_merge(o[:, :, a:b], l[:, :, a:b], m[:, :, a:b], np.array([(b - a) * 16]), 16)
        M = m[0, 0, a:b].max()
        ls = (l[0, 0, a:b] * np.exp(m[0, 0, a:b] - M)).sum()
        parts.append((sub[0, 0], M, ls))
    o2 = np.array([[[p[0] for p in parts]]])
    m2 = np.array([[[p[1] for p in parts]]])
    l2 = np.array([[[p[2] for p in parts]]])
    np.testing.assert_allclose(oracle.lse_merge(o2, l2, m2, np.array([32]), 16), ref, atol=1e-13)
    # an empty partition (l = 0, m = -inf) contributes nothing
    o3 = np.concatenate([o, np.zeros((1, 1, 1, D))], axis=2)
    l3 = np.concatenate([l, np.zeros((1, 1, 1))], axis=2)
    m3 = np.concatenate([m, np.full((1, 1, 1), -np.inf)], axis=2)
    np.testing.assert_allclose(oracle.lse_merge(o3, l3, m3, np.array([(P + 1) * 16]), 16), ref,
                               atol=1e-13)


# ---------------------------------------------------------------------------
# P11: cache write (scatter) and gather
# ---------------------------------------------------------------------------

def test_reshape_and_cache_then_gather_roundtrip_bit_exact():
    rng = np.random.default_rng(14)
    T, KVH, D, B, NB = 37, 2, 16, 16, 8
    key = rng.standard_normal((T, KVH, D)).astype(np.float16)
    value = rng.standard_normal((T, KVH, D)).astype(np.float16)
    kc = np.full((NB, KVH, D // 8, B, 8), np.nan, dtype=np.float16)
    vc = np.full((NB, KVH, D, B), np.nan, dtype=np.float16)
    # one sequence of T tokens over blocks [5, 2, 7]
    bt = np.array([[5, 2, 7]], dtype=np.int32)
    slots = np.array([bt[0, t // B] * B + t % B for t in range(T)], dtype=np.int64)
    kc2, vc2 = oracle.reshape_and_cache(key, value, kc, vc, slots, B)
    k_out, v_out = oracle.gather_kv(kc2, vc2, bt, np.array([T]), B)
    assert k_out.tobytes() == key.tobytes()
    assert v_out.tobytes() == value.tobytes()
    # untouched blocks and slots keep their bits
    touched = np.zeros(NB * B, dtype=bool)
    touched[slots] = True
    for b in range(NB):
        for o in range(B):
            if not touched[b * B + o]:
                assert np.isnan(kc2[b, :, :, o, :].astype(np.float32)).all()
                assert np.isnan(vc2[b, :, :, o].astype(np.float32)).all()
    # the pools read back through the page's split view agree with the input
    for t in range(T):
        b, o = divmod(int(slots[t]), B)
        flat = kc2[b].reshape(KVH, -1)
        view = torch.from_numpy(flat.view(np.int16)).view(KVH, D // 8, -1, 8).numpy().view(np.float16)
        np.testing.assert_array_equal(view[:, :, o, :].reshape(KVH, D), key[t])


def test_reshape_and_cache_skips_negative_slots():
    rng = np.random.default_rng(15)
    key = rng.standard_normal((3, 1, 8)).astype(np.float16)
    kc = np.zeros((2, 1, 1, 4, 8), dtype=np.float16)
    vc = np.zeros((2, 1, 8, 4), dtype=np.float16)
    kc2, vc2 = oracle.reshape_and_cache(key, key, kc, vc, np.array([-1, 6, -5]), 4)
    np.testing.assert_array_equal(kc2[1, 0, 0, 2], key[1, 0])
    np.testing.assert_array_equal(vc2[1, 0, :, 2], key[1, 0])
    assert np.count_nonzero(kc2) == np.count_nonzero(key[1]) and np.count_nonzero(vc2) == np.count_nonzero(key[1])


# ---------------------------------------------------------------------------
# Mutation checks: a planted oracle mistake must fail a pin
# ---------------------------------------------------------------------------

def _transposed_key_vector(k_cache, block, kv_head, slot):
    tile = k_cache[block, kv_head]
    return tile[:, slot, :].T.reshape(-1)     # wrong order of (d // x, d % x)


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_pins_catch_planted_mistakes(monkeypatch):
    # 1. transposed x-packing
    with monkeypatch.context() as mp:
        mp.setattr(opa, "key_vector", _transposed_key_vector)
        assert _fails(lambda: test_worked_example_matches_page(2, False))
    # 2. dropped scale
    orig_attention = opa.attention
    with monkeypatch.context() as mp:
        mp.setattr(opa, "attention", lambda q, K, V, scale: orig_attention(q, K, V, 1.0))
        mp.setattr(oracle, "attention", opa.attention)
        assert _fails(lambda: test_worked_example_matches_page(2, True))
    # 3. wrong head mapping (h % KVH instead of h // G)
    with monkeypatch.context() as mp:
        mp.setattr(opa, "kv_head_of", lambda h, H, KVH: h % KVH)
        assert _fails(lambda: test_oracle_equals_dense_library_attention(8, 2, 16, 4, 8))
    # 4. off by one at the end of the sequence (drops the last token)
    orig_fast = opa.gather_sequence_fast
    orig_slow = opa.gather_sequence
    with monkeypatch.context() as mp:
        mp.setattr(opa, "gather_sequence_fast",
                   lambda kc, vc, row, L, h, B: orig_fast(kc, vc, row, max(0, L - 1), h, B))
        mp.setattr(opa, "gather_sequence",
                   lambda kc, vc, row, L, h, B: orig_slow(kc, vc, row, max(0, L - 1), h, B))
        assert _fails(lambda: test_oracle_equals_dense_library_attention(4, 4, 8, 4, 2))
    # 5. merge weights without l_p
    orig_merge = opa.lse_merge
    with monkeypatch.context() as mp:
        mp.setattr(opa, "lse_merge", lambda t, e, m, L, ps: orig_merge(t, np.ones_like(e), m, L, ps))
        mp.setattr(oracle, "lse_merge", opa.lse_merge)
        assert _fails(lambda: test_partition_merge_equals_unpartitioned(64))
