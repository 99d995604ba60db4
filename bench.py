"""Benchmark: paged decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_gqa]
                    [--kernel v2|v1] [--seed S] [--no-cpu-baseline]

One step is one decode step of the whole hot path over one synthetic batch:
the cache write of the step's new token per sequence (reshape_and_cache at
logical position L_s - 1), then the decode attention over L_s tokens
(pa_decode_v2 + pa_reduce, or pa_decode_v1; batches that share blocks, the
shared_prefix and fork workloads, call pa_decode_v2_shared).  Inputs are
generated once and are resident in HBM before timing starts.

The metric is effective KV bandwidth: sum_s L_s * 2 * num_kv_heads * head_size
* 2 bytes per step divided by the step time, also given as a fraction of the
MI355X HBM peak (8 TB/s).  Rank 0 prints one JSON line.

`--workload fork` times the first decode step after a parallel-sampling fork:
the native block manager hands out the step's slots, tables and
copy-on-write pairs before timing, and the step is copy_blocks +
reshape_and_cache + pa_decode_v2_shared + pa_reduce.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode attention: effective KV GB/s (% of HBM peak) + µs/call"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_gqa")
    ap.add_argument("--kernel", default="v2", choices=["v1", "v2"])
    ap.add_argument("--kv-dtype", default="fp16", choices=["fp16", "fp8"],
                    help="element type of the K/V pools; fp8 = OCP E4M3 codes with per-pool "
                         "scales (k_scale = v_scale = 2**-6), written from the same fp16 values "
                         "by the library's own cache write before timing")
    ap.add_argument("--seed", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time budget of the oracle baseline sample")
    ap.add_argument("--scrub", action="store_true",
                    help="read 1 GiB before every step so no K/V is left in the 256 MB "
                         "Infinity Cache or L2 (a read, not a write: written lines stay dirty "
                         "in the caches and their write-back would be billed to the step); "
                         "the step time is then taken from HIP events (first to last kernel "
                         "of the step), not the wall clock")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the steps, run three plain device copies of exactly 1 GiB "
                         "(the known-size reference for rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    return ap.parse_args()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


class Parity:
    """GPU output against the oracle on the sampled rows: max-abs, relative L2,
    and whether the max-abs error is within 2e-3 and the relative L2 within
    1e-2."""

    def __init__(self):
        self.max_abs, self.err2, self.ref2, self.within = 0.0, 0.0, 0.0, True

    def add(self, ref, gpu):
        diff = ref - gpu
        self.max_abs = max(self.max_abs, float(np.abs(diff).max()))
        self.err2 += float((diff ** 2).sum())
        self.ref2 += float((ref ** 2).sum())
        self.within = self.within and bool(np.isfinite(gpu).all() and np.abs(diff).max() <= 2e-3)

    def result(self):
        rel = (self.err2 / self.ref2) ** 0.5 if self.ref2 > 0 else 0.0
        return {"max_abs": self.max_abs, "rel_l2": rel, "pass": self.within and rel <= 1e-2}


def cpu_baseline(k_cache, v_cache, block_tables, seq_lens, q, scale, num_kv_heads, block_size,
                 gpu_out, budget_s: float, fp8_scales=None):
    """The oracle (fp64 NumPy) on a bounded sample of the same workload:
    whole (sequence, KV head) units in order until the time budget is spent.
    The pools must already hold the step's cache writes.  Returns its
    throughput in the metric's unit, and its agreement with the GPU output
    on the sampled rows."""
    import oracle
    S, H, D = q.shape
    G = H // num_kv_heads
    done_bytes = 0
    spent = 0.0
    units = 0
    par = Parity()
    esz = 1 if fp8_scales is not None else 2     # bytes per element, as in the metric
    for s in range(S):
        L = int(seq_lens[s])
        for kvh in range(num_kv_heads):
            t0 = time.perf_counter()
            K, V = oracle.gather_sequence_fast(k_cache, v_cache, block_tables[s], L, kvh, block_size)
            if fp8_scales is not None:      # the oracle's own quantization of the fp16 values
                K = oracle.fp8.dequantize(oracle.fp8.quantize(K, fp8_scales[0]), fp8_scales[0])
                V = oracle.fp8.dequantize(oracle.fp8.quantize(V, fp8_scales[1]), fp8_scales[1])
            ref = oracle.attention(q[s, kvh * G:(kvh + 1) * G], K, V, scale)
            spent += time.perf_counter() - t0
            done_bytes += L * 2 * D * esz
            units += 1
            par.add(ref, gpu_out[s, kvh * G:(kvh + 1) * G])
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    return {
        "value": round(done_bytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"{units} whole (sequence, KV head) units of the same inputs "
                  f"({done_bytes / 1e9:.3f} GB of K/V), fp64 NumPy gather + two-pass softmax",
        "seconds": round(spent, 3),
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
        "max_abs_diff_vs_gpu": par.max_abs,
        "parity": par.result(),
    }


DECODE_SOURCES = ("pa_decode.hip", "pa_paths.h", "pa_device.h")
PREFILL_SOURCES = ("pa_prefill.hip", "pa_paths.h", "pa_device.h")


def kernel_source_hash(names=DECODE_SOURCES) -> str:
    """First 16 hex digits of the SHA-256 of the kernel sources `names`."""
    import hashlib
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "paged_kv_cache_302_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kname: str, workload: str, sources=DECODE_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/traffic_<kernel>_<workload>.txt), or None when there is none or
    the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kname}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def to_fp8_pools(pa, inp, kc16, vc16, bt, sl, k_scale, v_scale, dev):
    """fp8 pools holding the E4M3 codes of the fp16 pools' live tokens, made by
    the library itself: gather every sequence's K/V in logical order, then
    write them through reshape_and_cache into fp8 pools at the same slots."""
    import torch
    w = inp.workload
    B, KVH, D = w.block_size, w.num_kv_heads, w.head_size
    lens = inp.seq_lens.astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)[:-1]])
    total = int(lens.sum())
    slots = np.empty(total, np.int64)
    for s in range(w.num_seqs):
        t = np.arange(lens[s])
        slots[cu[s]:cu[s] + lens[s]] = inp.block_tables[s, t // B].astype(np.int64) * B + t % B
    ko = torch.empty((total, KVH, D), dtype=torch.float16, device=dev)
    vo = torch.empty_like(ko)
    pa.pa_gather_kv(ko, vo, kc16, vc16, bt, sl, torch.from_numpy(cu).to(dev))
    NB = inp.num_blocks
    kc8 = torch.zeros((NB, KVH, D // 16, B, 16), dtype=torch.uint8, device=dev)
    vc8 = torch.zeros((NB, KVH, D, B), dtype=torch.uint8, device=dev)
    pa.reshape_and_cache(ko, vo, kc8, vc8, torch.from_numpy(slots).to(dev), k_scale, v_scale)
    torch.cuda.synchronize()
    del ko, vo
    return kc8, vc8


def pct(ms):
    """p10 and p90 of per-step kernel times (ms) in microseconds."""
    return [round(float(np.percentile(ms, 10)) * 1e3, 2), round(float(np.percentile(ms, 90)) * 1e3, 2)]


def copy_calibration(dev):
    """Three device copies of exactly 1 GiB, so that a rocprofv3 --pmc run of
    the same process can scale FETCH_SIZE / WRITE_SIZE by what the counters
    read for a copy of known size."""
    import torch
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def device_copy_gbs(dev, nbytes=1 << 30, reps=5):
    """Device-to-device copy bandwidth, (read + write bytes) / time, median of
    `reps` copies of `nbytes`."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ms.append(a.elapsed_time(b))
    del src, dst
    return 2 * nbytes / (float(np.median(ms)) / 1e3) / 1e9


PREWARM_S = 0.25          # untimed back-to-back steps before the warm-up steps
PREWARM_MAX_STEPS = 5000
TIMING_WALL = ("wall clock over the timed steps, which record no events; per-kernel warm times "
               "from a second pass of as many steps with HIP events around each launch")


def timed_steps(args, step, n_events):
    """Warm-up, then exactly args.steps steps between two synchronisations;
    returns (ms_per_step, per-step event lists, wall ms per step).

    Without --scrub the timed steps record no events: an event record on the
    stream costs the step a few microseconds of its own, so the per-kernel
    warm times come from a second pass of args.steps back-to-back steps that
    does record them.  With --scrub each timed step sits behind a 1 GiB read
    and the step time is taken between its own first and last events."""
    import torch
    dev = torch.device("cuda:0")
    # Untimed pre-warm: the step back to back for PREWARM_S seconds before the
    # W warm-up steps.  The first tens of milliseconds of back-to-back steps
    # run slower than the rest (the 8 x 2K prefill step: 430 us over its first
    # 50 steps, 384 us after), so a few warm-up steps alone would leave that
    # ramp inside the timed region.
    t_end = time.perf_counter() + PREWARM_S
    for _ in range(PREWARM_MAX_STEPS // 10):
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            break
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    scrub_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev) if args.scrub else None
    scrub_sum = torch.empty((), dtype=torch.float32, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_events)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        if scrub_buf is not None:
            torch.sum(scrub_buf, dim=0, out=scrub_sum)
            step(evs[k])
        else:
            step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t_start) * 1e3 / args.steps
    if scrub_buf is not None:
        ms = float(np.mean([e[0].elapsed_time(e[-1]) for e in evs]))
    else:
        ms = wall
        for k in range(args.steps):   # the instrumented warm pass
            step(evs[k])
        torch.cuda.synchronize()
    return ms, evs, wall


def scrubbed_pass(step, n_events, steps):
    """`steps` more steps after the timed region, each behind a 1 GiB read
    that leaves no K/V in the Infinity Cache or L2 (a read, so no dirty
    lines are left for the step to write back): the cold-cache kernel times
    the roofline is taken from.  Returns the per-step event lists."""
    import torch
    dev = torch.device("cuda:0")
    scrub_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    scrub_sum = torch.empty((), dtype=torch.float32, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_events)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        torch.sum(scrub_buf, dim=0, out=scrub_sum)
        step(evs[k])
    torch.cuda.synchronize()
    del scrub_buf
    return evs


def cold_and_warm(args, step, n_events, evs, i):
    """Mean duration (s) of kernel i (events i, i + 1) over the scrubbed pass
    (the timed steps themselves under --scrub) and over the warm timed
    steps, and the scrubbed pass's events."""
    cold = evs if args.scrub else scrubbed_pass(step, n_events, args.steps)
    mean = lambda ev: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in ev])) / 1e3
    return mean(cold), mean(evs), cold


def roofline_entry(kname, nbytes, secs, traffic=None, cache="cold"):
    achieved = nbytes / secs / 1e9
    r = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
         "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": round(secs * 1e6, 2)}
    r["cache"] = ("cold: mean over launches each behind a 1 GiB read scrub, HIP events"
                  if cache == "cold" else "warm: mean over the back-to-back timed steps, HIP events")
    return r


def main_fork(args):
    """First decode step after a parallel-sampling fork (see the module
    docstring)."""
    import torch

    import paged_kv_cache_302_amd as pa
    import workloads as wl

    dev = torch.device("cuda:0")
    w = wl.FORK
    t0 = time.time()
    fi = wl.make_fork_inputs(w, args.seed)
    gen_s = time.time() - t0
    S, H, D, KVH, B = w.num_seqs, w.num_heads, w.head_size, w.num_kv_heads, w.block_size
    NB = w.pool_blocks

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    kc = torch.zeros((NB, KVH, D // 8, B, 8), dtype=torch.float16, device=dev)
    vc = torch.zeros((NB, KVH, D, B), dtype=torch.float16, device=dev)
    bm = pa.BlockManager(NB, B)
    seqs, prompt_slots = [], []
    for g in range(w.groups):
        root = g * w.samples
        sl_g = bm.add_sequence(root, w.prompt_len)
        prompt_slots.append(sl_g)
        pa.reshape_and_cache(t(fi.prompt_k[g]), t(fi.prompt_v[g]), kc, vc, t(sl_g))
        for c in range(1, w.samples):
            bm.fork(root, root + c)
        seqs += list(range(root, root + w.samples))
    slots, copies = bm.append_slots(seqs)
    width = -(-(w.prompt_len + 1) // B)
    tables, lens = bm.block_tables(seqs, width)
    q, key, val = t(fi.q), t(fi.key), t(fi.value)
    pairs_d, slot_d, bt, sl = t(copies), t(slots), t(tables), t(lens)
    PS = w.partition_size
    P = pa.pa_v2_max_partitions(int(lens.max()), PS)
    tmp, es, ml = pa.v2_scratch(S, H, D, P, dev)
    out = torch.empty((S, H, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        # the step is idempotent: the copies read blocks no write of the step
        # touches before them, and every write lands on the same slot again
        if ev is not None:
            ev[0].record(stream)
        pa.copy_blocks(kc, vc, pairs_d)
        if ev is not None:
            ev[1].record(stream)
        pa.reshape_and_cache(key, val, kc, vc, slot_d)
        if ev is not None:
            ev[2].record(stream)
        pa.pa_decode_v2_shared(tmp, es, ml, q, kc, vc, bt, sl, w.scale, PS)
        if ev is not None:
            ev[3].record(stream)
        pa.pa_reduce(out, tmp, es, ml, sl, PS)
        if ev is not None:
            ev[4].record(stream)

    ms_per_step, evs, wall = timed_steps(args, step, 5)
    dec_s, dec_warm_s, cold = cold_and_warm(args, step, 5, evs, 2)
    if args.copy_calibration:
        copy_calibration(dev)
    med = lambda i: float(np.median([e[i].elapsed_time(e[i + 1]) for e in evs]))
    copy_s = med(0) / 1e3
    block_bytes = KVH * D * B * 2                       # one block of one pool
    distinct = len(np.unique(tables[tables >= 0]))
    unique_bytes = distinct * 2 * block_bytes           # whole K and V tiles the decode reads
    kv_bytes = int(lens.astype(np.int64).sum()) * KVH * D * 4
    copy_bytes = len(copies) * 2 * block_bytes * 2      # read + write, both pools
    value = kv_bytes / (ms_per_step / 1e3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "fork",
            "kernel": "copy_blocks + reshape_and_cache + pa_decode_v2_shared + pa_reduce",
            "groups": w.groups, "samples": w.samples, "prompt_len": w.prompt_len,
            "num_seqs": S, "num_heads": H, "num_kv_heads": KVH, "head_size": D,
            "block_size": B, "partition_size": PS, "num_blocks": NB,
            "copy_pairs": int(len(copies)), "distinct_blocks": int(distinct),
            "kv_bytes_per_step": kv_bytes, "unique_kv_bytes_per_step": unique_bytes,
            "seed": args.seed,
        },
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kernels_us": {
            "copy_blocks": round(med(0) * 1e3, 2),
            "reshape_and_cache": round(med(1) * 1e3, 2),
            "pa_decode_v2_shared": round(med(2) * 1e3, 2),
            "pa_reduce": round(med(3) * 1e3, 2),
        },
        "kernels_us_cold": {"pa_decode_v2_shared": round(float(np.median(
            [e[2].elapsed_time(e[3]) for e in cold])) * 1e3, 2)},
        "roofline": roofline_entry("pa_decode_v2_shared", unique_bytes, dec_s,
                                   read_traffic("pa_decode_v2_shared", "fork")),
        "roofline_warm": roofline_entry("pa_decode_v2_shared", unique_bytes, dec_warm_s,
                                        cache="warm"),
        "copy_blocks": {
            "bytes_per_launch": copy_bytes,
            "achieved_gbs": round(copy_bytes / copy_s / 1e9, 2),
            "frac_of_peak": round(copy_bytes / copy_s / 1e9 / HBM_PEAK_GBS, 4),
        },
        "timing": ("HIP events per step, 1 GiB read scrub between steps (wall %.4f ms/step incl. scrub)"
                   % wall) if args.scrub else TIMING_WALL,
        "input_gen_s": round(gen_s, 2),
    }
    if not args.no_cpu_baseline:
        import oracle
        gpu_out = out.cpu().numpy()
        # the oracle replays the same writes and copies on host pools
        hk = np.zeros((NB, KVH, D // 8, B, 8), np.float16)
        hv = np.zeros((NB, KVH, D, B), np.float16)
        for g in range(w.groups):
            oracle.reshape_and_cache(fi.prompt_k[g], fi.prompt_v[g], hk, hv, prompt_slots[g], B,
                                     inplace=True)
        oracle.copy_blocks(hk, hv, [tuple(p) for p in copies])
        oracle.reshape_and_cache(fi.key, fi.value, hk, hv, slots, B, inplace=True)
        res["cpu_baseline"] = cpu_baseline(hk, hv, tables, lens, fi.q, w.scale, KVH, B, gpu_out,
                                           args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def main_prefill(args, w):
    """Multi-token queries: the step writes the last query_len tokens' K/V of
    every sequence (reshape_and_cache) and runs their causal attention
    (pa_prefill).  Metric: attention TFLOP/s (4 H D flops per query-key pair
    inside the causal mask); MFMA-bound."""
    import torch

    import paged_kv_cache_302_amd as pa
    import workloads as wl

    dev = torch.device("cuda:0")
    t0 = time.time()
    inp = wl.make_inputs(w, args.seed)
    qh, keyh, valh, slots, qsl = wl.make_chunk(w, inp, args.seed)
    gen_s = time.time() - t0
    S, H, D, KVH, B, n = w.num_seqs, w.num_heads, w.head_size, w.num_kv_heads, w.block_size, w.query_len

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    kc, vc = t(inp.k_cache), t(inp.v_cache)
    bt, sl = t(inp.block_tables), t(inp.seq_lens)
    fp8 = args.kv_dtype == "fp8"
    ks = vs = 2.0 ** -6
    if fp8:
        kc, vc = to_fp8_pools(pa, inp, kc, vc, bt, sl, ks, vs, dev)
    q, key, val, slot_d, qsl_d = t(qh), t(keyh), t(valh), t(slots), t(qsl)
    out = torch.empty((S * n, H, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        pa.reshape_and_cache(key, val, kc, vc, slot_d, ks, vs)
        if ev is not None:
            ev[1].record(stream)
        pa.pa_prefill(out, q, kc, vc, bt, sl, qsl_d, n, inp.scale, ks, vs)
        if ev is not None:
            ev[2].record(stream)

    ms_per_step, evs, wall = timed_steps(args, step, 3)
    if args.copy_calibration:
        copy_calibration(dev)
    pf_s = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) / 1e3
    # query-key pairs inside the causal mask: sum over queries of (position + 1)
    pairs = sum(int(n * (int(L) - n) + n * (n + 1) // 2) for L in inp.seq_lens)
    flops = 4.0 * H * D * pairs
    kv_bytes = int(inp.seq_lens.astype(np.int64).sum()) * KVH * D * 2 * (1 if fp8 else 2)
    value = flops / (ms_per_step / 1e3) / 1e12
    achieved = flops / pf_s / 1e12
    peak = 2500.0
    res = {
        "metric": "paged prefill attention: causal TFLOP/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA, f32 accumulate" + (" (f8e4m3 K/V)" if fp8 else ""),
        "data": "synthetic",
        "config": {
            "workload": args.workload + ("_fp8" if fp8 else ""),
            "kernel": "reshape_and_cache (query_len tokens) + pa_prefill",
            "num_seqs": S, "num_heads": H, "num_kv_heads": KVH, "head_size": D,
            "query_len": n, "seq_lens": [int(inp.seq_lens.min()), int(inp.seq_lens.max())],
            "causal_pairs": pairs, "flops_per_step": flops, "kv_bytes": kv_bytes,
            "kv_cache_dtype": args.kv_dtype, "seed": args.seed,
        },
        "us_per_step": round(ms_per_step * 1e3, 2),
        "kernels_us": {
            "reshape_and_cache": round(float(np.median([e[0].elapsed_time(e[1]) for e in evs])) * 1e3, 2),
            "pa_prefill": round(float(np.median([e[1].elapsed_time(e[2]) for e in evs])) * 1e3, 2),
        },
        "roofline": {
            "kernel": "pa_prefill",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": read_traffic("pa_prefill", args.workload + ("_fp8" if fp8 else ""),
                                    PREFILL_SOURCES),
            "algorithmic_flops_per_launch": flops,
            "kv_bytes_per_launch": kv_bytes,
            # q and the contexts' K/V, each read once; out (fp32) is written once
            "read_bytes_per_launch": kv_bytes + S * n * H * D * 2,
            "write_bytes_per_launch": S * n * H * D * 4,
            "avg_launch_us": round(pf_s * 1e6, 2),
            "hbm_floor_us": round(kv_bytes / 8e12 * 1e6, 2),
        },
        "timing": ("HIP events per step, 1 GiB read scrub between steps (wall %.4f ms/step incl. scrub)"
                   % wall) if args.scrub else TIMING_WALL,
        "input_gen_s": round(gen_s, 2),
    }
    if not args.no_cpu_baseline:
        import oracle
        gpu_out = out.cpu().numpy()
        oracle.reshape_and_cache(keyh, valh, inp.k_cache, inp.v_cache, slots, B, inplace=True)
        G = H // KVH
        done, spent, rows = 0.0, 0.0, 0
        par = Parity()
        # query rows spread over each chunk, sequence by sequence, until the budget is spent
        for s in range(S):
            L = int(inp.seq_lens[s])
            for kvh in range(KVH):
                K, V = oracle.gather_sequence_fast(inp.k_cache, inp.v_cache, inp.block_tables[s], L, kvh, B)
                if fp8:
                    K = oracle.fp8.dequantize(oracle.fp8.quantize(K, ks), ks)
                    V = oracle.fp8.dequantize(oracle.fp8.quantize(V, vs), vs)
                for j in range(n - 1 - (s + kvh) % 13, -1, -13):
                    p = L - n + j
                    row = int(qsl[s]) + j
                    t1 = time.perf_counter()
                    ref = oracle.attention(qh[row, kvh * G:(kvh + 1) * G], K[:p + 1], V[:p + 1], inp.scale)
                    spent += time.perf_counter() - t1
                    done += 4.0 * G * D * (p + 1)
                    rows += 1
                    par.add(ref, gpu_out[row, kvh * G:(kvh + 1) * G])
                    if spent >= args.cpu_seconds:
                        break
                if spent >= args.cpu_seconds:
                    break
            if spent >= args.cpu_seconds:
                break
        res["cpu_baseline"] = {
            "value": round(done / spent / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{rows} (query row, KV head) attentions, every 13th query row of each chunk "
                      f"from sequence 0 on, fp64 NumPy two-pass softmax",
            "seconds": round(spent, 3), "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "max_abs_diff_vs_gpu": par.max_abs,
            "parity": par.result(),
        }
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode "
              "kernels run on one GPU; sharding over GPUs is not implemented.", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_302_amd as pa
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    if args.workload == "fork":
        return main_fork(args)
    w = wl.WORKLOADS[args.workload]
    if w.query_len:
        return main_prefill(args, w)
    t0 = time.time()
    inp = wl.make_inputs(w, args.seed)
    gen_s = time.time() - t0
    S, H, D, KVH = w.num_seqs, w.num_heads, w.head_size, w.num_kv_heads
    G = H // KVH

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q, kc, vc = t(inp.q), t(inp.k_cache), t(inp.v_cache)
    bt, sl = t(inp.block_tables), t(inp.seq_lens)
    fp8 = args.kv_dtype == "fp8"
    ks = vs = 2.0 ** -6
    if fp8:
        kc, vc = to_fp8_pools(pa, inp, kc, vc, bt, sl, ks, vs, dev)
    # the step's new token per sequence, written at logical position L_s - 1
    slots = wl.new_token_slots(inp)
    key, val, slot_d = t(inp.key), t(inp.value), t(slots)

    PS = w.partition_size
    P = pa.pa_v2_max_partitions(w.max_seq_len, PS)
    tmp, es, ml = pa.v2_scratch(S, H, D, P, dev)
    out = torch.empty((S, H, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # batches built to share blocks take the entry point made for them
    shared = bool(w.group_size)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        pa.reshape_and_cache(key, val, kc, vc, slot_d, ks, vs)
        if ev is not None:
            ev[1].record(stream)
        if args.kernel == "v2":
            pa.pa_decode_v2(tmp, es, ml, q, kc, vc, bt, sl, inp.scale, PS, ks, vs,
                            shared_blocks=shared)
            if ev is not None:
                ev[2].record(stream)
            pa.pa_reduce(out, tmp, es, ml, sl, PS)
        else:
            pa.pa_decode_v1(out, q, kc, vc, bt, sl, inp.scale, ks, vs)
            if ev is not None:
                ev[2].record(stream)
        if ev is not None:
            ev[3].record(stream)

    # timed region: exactly `steps` steps, synchronised on both sides
    ms_per_step, evs, wall_ms_per_step = timed_steps(args, step, 4)
    dec_avg_s, dec_warm_s, cold = cold_and_warm(args, step, 4, evs, 1)

    if args.copy_calibration:
        copy_calibration(dev)

    cache_ms = [e[0].elapsed_time(e[1]) for e in evs]
    decode_ms = [e[1].elapsed_time(e[2]) for e in evs]
    reduce_ms = [e[2].elapsed_time(e[3]) for e in evs]
    cold_ms = [[e[i].elapsed_time(e[i + 1]) for e in cold] for i in range(3)]
    copy_gbs = device_copy_gbs(dev)

    esz = 1 if fp8 else 2
    kv_bytes = inp.kv_bytes * esz // 2
    unique_bytes = (inp.unique_kv_bytes if w.group_size else inp.kv_bytes) * esz // 2
    value = kv_bytes / (ms_per_step / 1e3) / 1e9
    achieved = unique_bytes / dec_avg_s / 1e9
    kname = ("pa_decode_v2_shared" if shared else "pa_decode_v2") if args.kernel == "v2" \
        else "pa_decode_v1"
    names = ["reshape_and_cache", kname] + (["pa_reduce"] if args.kernel == "v2" else [])
    traffic = read_traffic(kname, args.workload + ("_fp8" if fp8 else ""))

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f8e4m3 K/V, f16 q, f32 accumulate" if fp8 else "f16",
        "data": "synthetic",
        "config": {
            "workload": args.workload + ("_fp8" if fp8 else ""),
            "kv_cache_dtype": args.kv_dtype,
            **({"k_scale": ks, "v_scale": vs} if fp8 else {}),
            "kernel": f"reshape_and_cache + {kname}" + (" + pa_reduce" if args.kernel == "v2" else ""),
            "num_seqs": S, "num_heads": H, "num_kv_heads": KVH, "head_size": D,
            "block_size": w.block_size, "partition_size": PS if args.kernel == "v2" else None,
            "seq_lens": [int(x) for x in inp.seq_lens] if S <= 16 else
                        [int(inp.seq_lens.min()), int(inp.seq_lens.max())],
            "sum_seq_len": int(inp.seq_lens.sum()),
            "kv_bytes_per_step": kv_bytes,
            "unique_kv_bytes_per_step": unique_bytes,
            "num_blocks": inp.num_blocks, "seed": args.seed,
        },
        "kv_tokens_per_s": round(float(inp.seq_lens.astype(np.int64).sum()) * KVH / (ms_per_step / 1e3), 1),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kernels_us": {
            "reshape_and_cache": round(float(np.median(cache_ms)) * 1e3, 2),
            kname: round(float(np.median(decode_ms)) * 1e3, 2),
            **({"pa_reduce": round(float(np.median(reduce_ms)) * 1e3, 2)} if args.kernel == "v2" else {}),
        },
        "kernels_us_p10_p90": {
            "reshape_and_cache": pct(cache_ms),
            kname: pct(decode_ms),
            **({"pa_reduce": pct(reduce_ms)} if args.kernel == "v2" else {}),
        },
        "kernels_us_cold": {n: round(float(np.median(cold_ms[i])) * 1e3, 2) for i, n in enumerate(names)},
        # second denominator: a measured device-to-device copy (read + write bytes)
        "device_copy_gbs": round(copy_gbs, 1),
        "pct_of_device_copy": round(100 * achieved / copy_gbs, 2),
        "roofline": roofline_entry(kname, unique_bytes, dec_avg_s, traffic),
        "roofline_warm": roofline_entry(kname, unique_bytes, dec_warm_s, cache="warm"),
        "timing": ("HIP events per step, 1 GiB read scrub between steps (wall %.4f ms/step incl. scrub)"
                   % wall_ms_per_step) if args.scrub else TIMING_WALL,
        "input_gen_s": round(gen_s, 2),
    }
    if not args.no_cpu_baseline:
        import oracle
        gpu_out = out.cpu().numpy()
        # the same cache write the GPU step made, so both see the same K/V
        oracle.reshape_and_cache(inp.key, inp.value, inp.k_cache, inp.v_cache, slots,
                                 w.block_size, inplace=True)
        res["cpu_baseline"] = cpu_baseline(inp.k_cache, inp.v_cache, inp.block_tables,
                                           inp.seq_lens, inp.q, inp.scale, KVH, w.block_size,
                                           gpu_out, args.cpu_seconds,
                                           fp8_scales=(ks, vs) if fp8 else None)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
