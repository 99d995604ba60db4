"""GPU tests of the fp8 (E4M3) KV cache against the oracle: the cache write's
codes bit for bit (rounding, ties, saturation, NaN, -0), the gather and the
block copy of codes bit for bit, and decode attention (v1, v2 partials and
merge) over fp8 pools against the oracle's attention over the decoded,
scaled values, with NaN codes poisoning every slot the kernels must not
read."""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
import paged_kv_cache_302_amd as pa
import workloads as wl
from tests._util import assert_parity, device, to_dev

pytestmark = pytest.mark.gpu


def k16_to_logical(kc):
    NB, KVH, Dx, B, x = kc.shape
    return kc.transpose(0, 1, 2, 4, 3).reshape(NB, KVH, Dx * x, B)        # [NB, KVH, D, B]


def logical_to_k8(kl):
    NB, KVH, D, B = kl.shape
    return np.ascontiguousarray(kl.reshape(NB, KVH, D // 16, 16, B).transpose(0, 1, 2, 4, 3))


def fp8_case(label, S, H, KVH, D, lo, hi, seed, ks=0.05, vs=0.03):
    w = wl.small_workload(label, num_seqs=S, num_heads=H, num_kv_heads=KVH, head_size=D,
                          seq_len_lo=lo, seq_len_hi=hi)
    inp = wl.make_inputs(w, seed)
    oracle.poison_unused(inp.k_cache, inp.v_cache, inp.block_tables, inp.seq_lens, 16)
    k8 = logical_to_k8(fp8.quantize(k16_to_logical(inp.k_cache), ks))
    v8 = fp8.quantize(inp.v_cache, vs)
    return inp, k8, v8, ks, vs


CASES = [
    ("mfma_d128_g4", 3, 16, 4, 128, 1, 700),
    ("mfma_d128_g7", 3, 14, 2, 128, 100, 600),
    ("mfma_d64_g8", 3, 16, 2, 64, 1, 400),
    ("mfma_d128_g24", 2, 24, 1, 128, 1, 300),
    ("valu_d128", 4, 6, 6, 128, 1, 300),
    ("valu_d64", 4, 4, 4, 64, 1, 130),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_decode_matches_oracle(case):
    inp, k8, v8, ks, vs = fp8_case(*case, seed=31)
    assert (k8 == 0x7F).any()            # poisoned slots really hold NaN codes
    dk, dv = fp8.dequantize_pools(k8, v8, ks, vs)
    ref = oracle.paged_decode(inp.q, dk, dv, inp.block_tables, inp.seq_lens, inp.scale, 16)
    q, bt, sl = to_dev(inp.q), to_dev(inp.block_tables), to_dev(inp.seq_lens)
    kc, vc = to_dev(k8), to_dev(v8)
    out1 = pa.paged_attention_v1(q, kc, vc, bt, sl, inp.scale, ks, vs).cpu().numpy()
    assert_parity(out1, ref, case[0] + " fp8 v1")
    out2 = pa.paged_attention_v2(q, kc, vc, bt, sl, inp.scale, 64, inp.workload.max_seq_len,
                                 ks, vs).cpu().numpy()
    assert_parity(out2, ref, case[0] + " fp8 v2")


def test_fp8_v2_partials_match_oracle():
    inp, k8, v8, ks, vs = fp8_case("parts", 3, 16, 4, 128, 50, 900, seed=32)
    dk, dv = fp8.dequantize_pools(k8, v8, ks, vs)
    S, H, D = inp.q.shape
    PS = 128
    P = pa.pa_v2_max_partitions(inp.workload.max_seq_len, PS)
    t_ref, e_ref, m_ref = oracle.partition_partials(inp.q, dk, dv, inp.block_tables, inp.seq_lens,
                                                    inp.scale, 16, PS, P)
    tmp, es, ml = pa.v2_scratch(S, H, D, P, device())
    pa.pa_decode_v2(tmp, es, ml, to_dev(inp.q), to_dev(k8), to_dev(v8), to_dev(inp.block_tables),
                    to_dev(inp.seq_lens), inp.scale, PS, ks, vs)
    tmp = tmp.cpu().numpy().transpose(0, 2, 1, 3)
    es = es.cpu().numpy().transpose(0, 2, 1)
    ml = ml.cpu().numpy().transpose(0, 2, 1)
    valid = ~np.isnan(e_ref)
    assert_parity(tmp[valid], t_ref[valid], "fp8 o_p")
    np.testing.assert_allclose(ml[valid], m_ref[valid], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(es[valid], e_ref[valid], rtol=2e-5)


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_cache_write_codes_bit_exact(D):
    rng = np.random.default_rng(D)
    T, KVH, NB, B = 40, 3, 12, 16
    ks, vs = 0.02, 0.37
    key = (rng.standard_normal((T, KVH, D)) * 3).astype(np.float16)
    val = (rng.standard_normal((T, KVH, D)) * 50).astype(np.float16)   # some beyond 448 * vs
    # exact midpoints between codes (ties), zeros of both signs, NaN, huge values
    mids = (fp8.decode_e4m3(np.arange(0x30, 0x40)) + fp8.decode_e4m3(np.arange(0x31, 0x41))) / 2
    key[0, 0, :16] = (mids * ks).astype(np.float16)
    key[1, 0, :4] = np.array([0.0, -0.0, np.nan, 6e4], np.float16)
    val[1, 1, :3] = np.array([-6e4, -0.0, np.nan], np.float16)
    slots = rng.permutation(NB * B)[:T].astype(np.int64)
    slots[5] = -1
    k8 = np.zeros((NB, KVH, D // 16, B, 16), np.uint8)
    v8 = np.zeros((NB, KVH, D, B), np.uint8)
    kc, vc = to_dev(k8), to_dev(v8)
    pa.reshape_and_cache(to_dev(key), to_dev(val), kc, vc, to_dev(slots), ks, vs)
    fp8.reshape_and_cache_fp8(key, val, k8, v8, slots, B, ks, vs)
    assert kc.cpu().numpy().tobytes() == k8.tobytes()
    assert vc.cpu().numpy().tobytes() == v8.tobytes()


def test_fp8_gather_and_copy_blocks_bit_exact():
    inp, k8, v8, ks, vs = fp8_case("gather", 3, 8, 2, 128, 1, 200, seed=33)
    S = inp.q.shape[0]
    cu = np.concatenate([[0], np.cumsum(inp.seq_lens)[:-1]]).astype(np.int64)
    total = int(inp.seq_lens.sum())
    ko = torch.empty((total, 2, 128), dtype=torch.uint8, device=device())
    vo = torch.empty_like(ko)
    kc, vc = to_dev(k8), to_dev(v8)
    pa.pa_gather_kv(ko, vo, kc, vc, to_dev(inp.block_tables), to_dev(inp.seq_lens), to_dev(cu))
    ko, vo = ko.cpu().numpy(), vo.cpu().numpy()
    for s in range(S):
        L = int(inp.seq_lens[s])
        for h in range(2):
            K, V = oracle.gather_sequence(k8, v8, inp.block_tables[s], L, h, 16)
            assert np.array_equal(ko[cu[s]:cu[s] + L, h], K)
            assert np.array_equal(vo[cu[s]:cu[s] + L, h], V)
    NB = k8.shape[0]
    pairs = np.array([[0, NB - 1], [1, NB - 2], [NB + 5, 0]], np.int32)
    pa.copy_blocks(kc, vc, to_dev(pairs))
    oracle.copy_blocks(k8, v8, [tuple(p) for p in pairs])
    assert kc.cpu().numpy().tobytes() == k8.tobytes()
    assert vc.cpu().numpy().tobytes() == v8.tobytes()


def test_fp8_write_then_decode_pipeline():
    """fp16 keys/values written into fp8 pools by the GPU cache write, then
    decoded: equals the oracle's quantize-then-attend."""
    rng = np.random.default_rng(34)
    S, H, KVH, D, B = 4, 8, 2, 128, 16
    lens = np.array([1, 17, 250, 96], np.int32)
    NB = int(sum(-(-l // B) for l in lens)) + 3
    perm = rng.permutation(NB)
    bt = np.full((S, 16), -1, np.int32)
    slots, keys, vals = [], [], []
    nxt = 0
    for s in range(S):
        nb = -(-lens[s] // B)
        bt[s, :nb] = perm[nxt:nxt + nb]
        nxt += nb
        for t in range(lens[s]):
            slots.append(bt[s, t // B] * B + t % B)
    T = len(slots)
    key = rng.standard_normal((T, KVH, D)).astype(np.float16)
    val = rng.standard_normal((T, KVH, D)).astype(np.float16)
    slots = np.array(slots, np.int64)
    ks, vs = 0.01, 0.008
    k8 = np.full((NB, KVH, D // 16, B, 16), 0x7F, np.uint8)      # unwritten slots: NaN codes
    v8 = np.full((NB, KVH, D, B), 0x7F, np.uint8)
    kc, vc = to_dev(k8), to_dev(v8)
    pa.reshape_and_cache(to_dev(key), to_dev(val), kc, vc, to_dev(slots), ks, vs)
    fp8.reshape_and_cache_fp8(key, val, k8, v8, slots, B, ks, vs)
    q = rng.standard_normal((S, H, D)).astype(np.float16)
    dk, dv = fp8.dequantize_pools(k8, v8, ks, vs)
    ref = oracle.paged_decode(q, dk, dv, bt, lens, 1 / np.sqrt(D), B)
    out = pa.paged_attention_v1(to_dev(q), kc, vc, to_dev(bt), to_dev(lens), 1 / np.sqrt(D),
                                ks, vs).cpu().numpy()
    assert_parity(out, ref, "fp8 write + decode")


@pytest.mark.parametrize("S,entry", [(8, False), (8, True), (72, True)],
                         ids=["units", "set_kernel_8", "set_kernel_72"])
def test_fp8_partitions_shared_by_sequences_match_private_copies(S, entry):
    """fp8 pools: v2 units of sequences that read the same blocks over a
    partition (one tile for the aligned set of four, G = 4) equal, bit for bit,
    the same sequences reading private copies of the codes, and the oracle over
    the decoded values; through pa_decode_v2_shared the set kernel runs."""
    KVH, G, D, PS = 2, 4, 128, 128
    inp, k8, v8, ks, vs = fp8_case("share8", S, G * KVH, KVH, D, 400, 400, seed=33)
    nb = -(-400 // 16)
    bt = inp.block_tables.copy()
    for d in (1, 2, 3):
        bt[d, :nb] = bt[0, :nb]                      # seqs 0-3 read one copy
    for d in (5, 6, 7):
        bt[d, :16] = bt[4, :16]                      # seqs 4-7 share their first two partitions
    L = inp.seq_lens.copy()
    used = [(s, i) for s in range(S) for i in range(nb)]
    k8p = np.full((len(used),) + k8.shape[1:], 0x7F, np.uint8)
    v8p = np.full((len(used),) + v8.shape[1:], 0x7F, np.uint8)
    bt2 = np.full_like(bt, -1)
    for n, (s, i) in enumerate(used):
        k8p[n], v8p[n], bt2[s, i] = k8[bt[s, i]], v8[bt[s, i]], n

    def run(kc8, vc8, table):
        P = pa.pa_v2_max_partitions(400, PS)
        tmp, es, ml = pa.v2_scratch(S, G * KVH, D, P, device())
        pa.pa_decode_v2(tmp, es, ml, to_dev(inp.q), to_dev(kc8), to_dev(vc8), to_dev(table),
                        to_dev(L), inp.scale, PS, ks, vs, shared_blocks=entry)
        out = torch.empty((S, G * KVH, D), dtype=torch.float32, device=device())
        pa.pa_reduce(out, tmp, es, ml, to_dev(L), PS)
        return tmp.cpu().numpy(), es.cpu().numpy(), ml.cpu().numpy(), out.cpu().numpy()

    shared, private = run(k8, v8, bt), run(k8p, v8p, bt2)
    for a, b in zip(shared, private):
        assert np.array_equal(a, b)
    dk, dv = fp8.dequantize_pools(k8, v8, ks, vs)
    ref = oracle.paged_decode(inp.q, dk, dv, bt, L, inp.scale, 16)
    assert_parity(shared[3], ref, "fp8 shared")


def fp8_decode_both(inp, k8, v8, ks, vs, ps, shared=False):
    q, bt, sl = to_dev(inp.q), to_dev(inp.block_tables), to_dev(inp.seq_lens)
    kc, vc = to_dev(k8), to_dev(v8)
    out1 = pa.paged_attention_v1(q, kc, vc, bt, sl, inp.scale, ks, vs).cpu().numpy()
    out2 = pa.paged_attention_v2(q, kc, vc, bt, sl, inp.scale, ps, inp.workload.max_seq_len,
                                 ks, vs, shared_blocks=shared).cpu().numpy()
    return out1, out2


# One sequence and one KV head: the launch uses 8 waves per unit, so these
# lengths put 64, 65, 128 and 156 blocks on a wave (v1, and v2 with 16K-token
# partitions), and the wave's table window of 64 entries is refilled during
# the walk on both fp8 paths.
FP8_WINDOW_LENS = [512 * 16, 512 * 16 + 1, 1024 * 16 + 7, 20000]


@pytest.mark.parametrize("H,D", [(4, 64), (1, 128)], ids=["mfma", "valu"])
@pytest.mark.parametrize("L", FP8_WINDOW_LENS)
def test_fp8_long_unit_crosses_table_windows(H, D, L):
    inp, k8, v8, ks, vs = fp8_case("windows8", 1, H, 1, D, L, L, seed=33)
    dk, dv = fp8.dequantize_pools(k8, v8, ks, vs)
    ref = oracle.paged_decode(inp.q, dk, dv, inp.block_tables, inp.seq_lens, inp.scale, 16)
    out1, out2 = fp8_decode_both(inp, k8, v8, ks, vs, 16384)
    assert_parity(out1, ref, f"fp8 v1 L={L}")
    assert_parity(out2, ref, f"fp8 v2 L={L}")


# v2 unit orders on fp8 pools: 64 sequences x 8 KV heads x up to 16
# partitions is more than the device holds at once and shares no blocks (the
# XCD-major order); 1,200 sequences exceed it with the plain order; 200
# sequences fit (largest-first order over four lookup chunks).  The set_
# cases go through pa_decode_v2_shared, which takes the set kernel for G = 4
# and 8.
FP8_ORDER_CASES = [
    ("xcd_major", 64, 32, 8, 128, 1, 1024, 64),
    ("big_grid", 1200, 14, 2, 64, 1, 1000, 128),
    ("resident_200", 200, 14, 2, 64, 1, 700, 128),
    ("set_g4_big_grid", 1200, 8, 2, 64, 1, 1000, 128),
    ("set_g8_d128", 130, 16, 2, 128, 1, 900, 256),
    ("long_four_waves", 8, 32, 8, 128, 1, 20000, 256),
]


@pytest.mark.parametrize("case", FP8_ORDER_CASES, ids=[c[0] for c in FP8_ORDER_CASES])
def test_fp8_v2_unit_orders(case):
    label, S, H, KVH, D, lo, hi, ps = case
    inp, k8, v8, ks, vs = fp8_case(label, S, H, KVH, D, lo, hi, seed=34)
    dk, dv = fp8.dequantize_pools(k8, v8, ks, vs)
    ref = oracle.paged_decode(inp.q, dk, dv, inp.block_tables, inp.seq_lens, inp.scale, 16)
    out1, out2 = fp8_decode_both(inp, k8, v8, ks, vs, ps, label.startswith("set_"))
    assert_parity(out2, ref, label + " fp8 v2")
    assert_parity(out1, ref, label + " fp8 v1")
