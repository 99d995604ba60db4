"""The seeded input generators: determinism, shapes, placement structure and
the byte counts the measurements are quoted in.  CPU only."""
import math

import numpy as np
import pytest

import workloads as wl


def test_same_seed_same_inputs():
    w = wl.WORKLOADS["tiny"]
    a = wl.make_inputs(w, 1)
    b = wl.make_inputs(w, 1)
    for f in ("seq_lens", "block_tables", "q", "k_cache", "v_cache"):
        assert getattr(a, f).tobytes() == getattr(b, f).tobytes()
    c = wl.make_inputs(w, 2)
    assert c.q.tobytes() != a.q.tobytes()


def test_fill_is_thread_count_independent(monkeypatch):
    out1 = np.empty(3 << 20, dtype=np.float16)
    out2 = np.empty(3 << 20, dtype=np.float16)
    wl.fill_normal_fp16(out1, np.random.SeedSequence(5), 0.5, chunk=1 << 18)
    monkeypatch.setattr(wl, "_threads", lambda: 1)
    wl.fill_normal_fp16(out2, np.random.SeedSequence(5), 0.5, chunk=1 << 18)
    assert out1.tobytes() == out2.tobytes()
    assert abs(float(out1.astype(np.float32).std()) - 0.5) < 0.01


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_structure(name):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, 1, fill_values=(name != "long_gqa"))
    S, B = w.num_seqs, w.block_size
    assert inp.q.shape == (S, w.num_heads, w.head_size) and inp.q.dtype == np.float16
    assert inp.k_cache.shape == (inp.num_blocks, w.num_kv_heads, w.head_size // 8, B, 8)
    assert inp.v_cache.shape == (inp.num_blocks, w.num_kv_heads, w.head_size, B)
    L = inp.seq_lens
    if w.group_size:
        assert (L >= w.prefix_len + w.seq_len_lo + 1).all() and (L <= w.max_seq_len).all()
    else:
        assert (L >= w.seq_len_lo).all() and (L <= w.seq_len_hi).all()
    nb = -(-L // B)
    ids = []
    for s in range(S):
        row = inp.block_tables[s]
        assert (row[:nb[s]] >= 0).all() and (row[:nb[s]] < inp.num_blocks).all()
        assert (row[nb[s]:] == -1).all()
        ids.append(row[:nb[s]])
    allids = np.concatenate(ids)
    if w.group_size:
        pre = w.prefix_len // B
        for g in range(S // w.group_size):
            rows = inp.block_tables[g * w.group_size:(g + 1) * w.group_size, :pre]
            assert (rows == rows[0]).all()          # shared prefix ids
        uniq = np.unique(allids)
        assert len(uniq) == (S // w.group_size) * pre + int((nb - pre).sum())
    else:
        assert len(np.unique(allids)) == len(allids)  # no block used twice


def test_mha_layer_bytes_match_llama7b_sizing():
    """One decode call over the LLaMA-7B layer shape reads
    16 seqs * 2048 tokens * 2 (K,V) * 32 heads * 128 * 2 B = 536,870,912 B,
    i.e. the 17.2 GB KV size of page "KV Cache与PagedAttention内存管理"
    (内存占用模型: 2*32*4096*2048*16*2 B) divided by its 32 layers."""
    inp = wl.make_inputs(wl.WORKLOADS["mha7b"], 3, fill_values=False)
    assert inp.kv_bytes == 536_870_912
    assert inp.kv_bytes * 32 == 2 * 32 * 4096 * 2048 * 16 * 2


def test_shared_prefix_new_token_slots():
    inp = wl.make_inputs(wl.WORKLOADS["shared_prefix"], 5, fill_values=False)
    slots = wl.new_token_slots(inp)
    assert slots.dtype == np.int64 and len(np.unique(slots)) == len(slots)
    B = 16
    for s in range(0, 256, 37):
        pos = int(inp.seq_lens[s]) - 1
        assert slots[s] // B == inp.block_tables[s, pos // B] and slots[s] % B == pos % B
        assert pos // B >= 64                       # never inside the shared prefix
    assert inp.unique_kv_bytes < inp.kv_bytes / 3
