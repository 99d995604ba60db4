"""GPU tests of copy-on-write: copy_blocks bit-exact against the oracle, and
parallel sampling end to end -- the native block manager hands out the
slots, tables and copies, copy_blocks and reshape_and_cache update the
pools, and pa_decode_v1 / pa_decode_v2 (and _shared) + pa_reduce must give, for every
sample, the dense attention over that sample's own token history (its
prompt plus its own generated tokens), which the oracle computes on
contiguous arrays.  Sharing and copy-on-write change where K/V live, never
what attention computes (blog page §4.2; kernel page §4)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_302_amd as pa
from tests._util import assert_parity, device, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("KVH,D", [(4, 128), (8, 64), (1, 128)])
def test_copy_blocks_bit_exact(KVH, D):
    rng = np.random.default_rng(KVH * D)
    NB = 96
    kc = rng.standard_normal((NB, KVH, D // 8, 16, 8)).astype(np.float16)
    vc = rng.standard_normal((NB, KVH, D, 16)).astype(np.float16)
    src = rng.permutation(NB)[:20]
    dst = rng.permutation(np.setdiff1d(np.arange(NB), src))[:20]
    pairs = np.stack([src, dst], axis=1).astype(np.int32)
    pairs = np.concatenate([pairs, [[NB + 3, 0], [1, -1]]]).astype(np.int32)   # skipped on the device
    dk, dv = to_dev(kc), to_dev(vc)
    pa.copy_blocks(dk, dv, to_dev(pairs))
    oracle.copy_blocks(kc, vc, [tuple(p) for p in pairs])
    assert dk.cpu().numpy().tobytes() == kc.tobytes()
    assert dv.cpu().numpy().tobytes() == vc.tobytes()


def test_copy_blocks_no_pairs_is_a_no_op():
    kc = torch.zeros((4, 1, 16, 16, 8), dtype=torch.float16, device=device())
    vc = torch.zeros((4, 1, 128, 16), dtype=torch.float16, device=device())
    pa.copy_blocks(kc, vc, torch.zeros((0, 2), dtype=torch.int32, device=device()))
    torch.cuda.synchronize()


@pytest.mark.parametrize("prompts,samples,steps", [
    ((37, 64, 100, 1), 4, 21),      # block-aligned and ragged prompts
    ((1000,), 8, 3),                # a non-block-aligned shared prefix, 8-way
])
def test_parallel_sampling_decode_matches_dense_histories(prompts, samples, steps):
    H, KVH, D, B = 8, 2, 128, 16
    NB = 1024
    scale = 1.0 / np.sqrt(D)
    rng = np.random.default_rng(sum(prompts) + samples)
    dev = device()
    bm = pa.BlockManager(NB, B)
    kc = torch.full((NB, KVH, D // 8, B, 8), float("nan"), dtype=torch.float16, device=dev)
    vc = torch.full((NB, KVH, D, B), float("nan"), dtype=torch.float16, device=dev)
    hist_k, hist_v = {}, {}
    seqs = []
    # prefill: each prompt's K/V written through its slots, then forked
    for g, n in enumerate(prompts):
        root = g * samples
        slots = bm.add_sequence(root, n)
        k = rng.standard_normal((n, KVH, D)).astype(np.float16)
        v = rng.standard_normal((n, KVH, D)).astype(np.float16)
        if n:
            pa.reshape_and_cache(to_dev(k), to_dev(v), kc, vc, to_dev(slots))
        for c in range(samples):
            if c:
                bm.fork(root, root + c)
            hist_k[root + c], hist_v[root + c] = list(k), list(v)
            seqs.append(root + c)
    n_copies = 0
    for step in range(steps):
        slots, copies = bm.append_slots(seqs)
        n_copies += len(copies)
        if len(copies):
            pa.copy_blocks(kc, vc, to_dev(copies))
        k = rng.standard_normal((len(seqs), KVH, D)).astype(np.float16)
        v = rng.standard_normal((len(seqs), KVH, D)).astype(np.float16)
        pa.reshape_and_cache(to_dev(k), to_dev(v), kc, vc, to_dev(slots))
        for i, s in enumerate(seqs):
            hist_k[s].append(k[i])
            hist_v[s].append(v[i])
    assert n_copies == sum(samples - 1 for n in prompts if n % B)   # one split per shared partial block
    # attend with every sample's current state
    width = max(-(-(max(prompts) + steps) // B), 1)
    tables, lens = bm.block_tables(seqs, width)
    q = rng.standard_normal((len(seqs), H, D)).astype(np.float16)
    G = H // KVH
    want = np.empty((len(seqs), H, D))
    for i, s in enumerate(seqs):
        K = np.stack(hist_k[s])          # [L, KVH, D]
        V = np.stack(hist_v[s])
        for h in range(H):
            want[i, h] = oracle.attention(q[i, h][None], K[:, h // G], V[:, h // G], scale)[0]
    dq, dt, dl = to_dev(q), to_dev(tables), to_dev(lens)
    out1 = pa.paged_attention_v1(dq, kc, vc, dt, dl, scale).cpu().numpy()
    assert_parity(out1, want, "v1 after fork / copy-on-write")
    out2 = pa.paged_attention_v2(dq, kc, vc, dt, dl, scale, 64, int(lens.max())).cpu().numpy()
    assert_parity(out2, want, "v2 after fork / copy-on-write")
    out3 = pa.paged_attention_v2(dq, kc, vc, dt, dl, scale, 64, int(lens.max()),
                                 shared_blocks=True).cpu().numpy()
    assert_parity(out3, want, "v2 shared after fork / copy-on-write")
