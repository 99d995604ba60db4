"""Pins of the prefill / chunked-prefill oracle (CPU).

* A full prefill (every token has a query) equals torch's scaled dot-product
  attention in float64 with is_causal=True over the contiguous K/V (the
  library routine; grouped-query heads via enable_gqa), for ragged lengths.
* One query per sequence is exactly the decode oracle.
* Causality brute force: query j of a chunk equals a decode over the
  sequence truncated to its position p + 1.
* A causal mask shifted by one (keys 0..p-1 or 0..p+1) fails the first pin.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def case(lens, n_q, H=8, KVH=2, D=32, seed=0):
    w = wl.small_workload("prefill", num_seqs=len(lens), num_heads=H, num_kv_heads=KVH,
                          head_size=D, seq_len_lo=1, seq_len_hi=max(lens))
    inp = wl.make_inputs(w, seed)
    # keep the generated placement, use the lengths asked for (tables are long enough)
    lens = np.array(lens, np.int32)
    assert (-(-lens // 16) <= inp.block_tables.shape[1]).all()
    nb = -(-lens // 16)
    bt = inp.block_tables.copy()
    for s in range(len(lens)):          # the placement gives every row max-length blocks? fill missing
        have = (bt[s] >= 0).sum()
        if have < nb[s]:
            free = np.setdiff1d(np.arange(inp.num_blocks), bt[bt >= 0])
            bt[s, have:nb[s]] = free[:nb[s] - have]
    qsl = np.concatenate([[0], np.cumsum(n_q)]).astype(np.int32)
    rng = np.random.default_rng(seed + 1)
    q = rng.standard_normal((int(qsl[-1]), H, D)).astype(np.float16)
    return inp, bt, lens, qsl, q


def sdpa_causal(q, K, V, scale, G):
    # q [n, H, D] for the last n positions of K/V [L, KVH, D]
    qt = torch.from_numpy(q.astype(np.float64)).transpose(0, 1)        # [H, n, D]
    kt = torch.from_numpy(K.astype(np.float64)).transpose(0, 1)        # [KVH, L, D]
    vt = torch.from_numpy(V.astype(np.float64)).transpose(0, 1)
    n, L = q.shape[0], K.shape[0]
    mask = torch.ones(n, L, dtype=torch.bool).tril(diagonal=L - n)
    kt = kt.repeat_interleave(G, dim=0)
    vt = vt.repeat_interleave(G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.transpose(0, 1).numpy()


def dense(inp, bt, s, L):
    KVH = inp.k_cache.shape[1]
    Ks, Vs = [], []
    for h in range(KVH):
        K, V = oracle.gather_sequence(inp.k_cache, inp.v_cache, bt[s], L, h, 16)
        Ks.append(K)
        Vs.append(V)
    return np.stack(Ks, 1), np.stack(Vs, 1)


@pytest.mark.parametrize("lens", [[1, 17, 40], [33, 16, 5]])
def test_full_prefill_equals_sdpa_causal(lens):
    inp, bt, lens, qsl, q = case(lens, lens)
    out = oracle.paged_prefill(q, inp.k_cache, inp.v_cache, bt, lens, qsl, 0.3, 16)
    for s in range(len(lens)):
        K, V = dense(inp, bt, s, int(lens[s]))
        ref = sdpa_causal(q[qsl[s]:qsl[s + 1]], K, V, 0.3, 4)
        np.testing.assert_allclose(out[qsl[s]:qsl[s + 1]], ref, rtol=1e-12, atol=1e-12)


def test_one_query_is_the_decode_oracle():
    inp, bt, lens, qsl, q = case([20, 45, 3], [1, 1, 1])
    out = oracle.paged_prefill(q, inp.k_cache, inp.v_cache, bt, lens, qsl, 0.2, 16)
    ref = oracle.paged_decode(q, inp.k_cache, inp.v_cache, bt, lens, 0.2, 16)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)


def test_chunk_rows_equal_truncated_decodes():
    inp, bt, lens, qsl, q = case([50, 29], [7, 12])
    out = oracle.paged_prefill(q, inp.k_cache, inp.v_cache, bt, lens, qsl, 0.25, 16)
    for s in range(2):
        n = qsl[s + 1] - qsl[s]
        for j in range(n):
            p = int(lens[s]) - n + j
            one = oracle.paged_decode(q[qsl[s] + j][None], inp.k_cache, inp.v_cache, bt[s:s + 1],
                                      np.array([p + 1]), 0.25, 16)
            np.testing.assert_allclose(out[qsl[s] + j], one[0], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("shift", [-1, 1])
def test_shifted_mask_is_caught(shift, monkeypatch):
    inp, bt, lens, qsl, q = case([40, 23], [40, 23])
    monkeypatch.setattr(oracle.paged_attention, "visible_keys", lambda p: max(1, p + 1 + shift))
    bad = oracle.paged_prefill(q, inp.k_cache, inp.v_cache, bt, lens, qsl, 0.3, 16)
    monkeypatch.undo()
    K, V = dense(inp, bt, 0, 40)
    ref = sdpa_causal(q[:40], K, V, 0.3, 4)
    assert not np.allclose(bad[:40], ref, rtol=1e-9, atol=1e-9)
