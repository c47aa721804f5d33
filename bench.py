"""Benchmark of the attention hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic inputs:

  1. causal prefill, B=4, S=2048, H=32, d=128 (attn_prefill);
  2. bulk KV append of that prefill's K/V into a [4, 32, 4096, 128] cache
     from position 0 (kv_cache_scatter);
  3. long-context GQA decode step, M=16, H=64, Hkv=8, d=128,
     max_len=32768, L_m ~ U{16384..32768}: append each sequence's new K/V row
     at L_m - 1 (kv_cache_scatter), then attend over L_m keys
     (attn_decode_gqa_batched: split pass + merge pass).

Inputs are resident in HBM before the timed region.  Every call is bracketed
by HIP events on the stream it is launched on (torch's current stream, which
the binding passes to the library), so each kernel's duration is measured
live over the timed steps; every rate is computed from the median of those
durations (mean, min and p90 are printed next to it).  ``value`` is the
decode's algorithmic HBM throughput (K/V rows 0..L_m-1 of every KV head read
once, q read, out written) over the decode's median time; the prefill's
algorithmic TFLOP/s (visible query/key pairs only) is reported next to it
and, being the longest kernel of the step, in the ``roofline`` object.
Between two decodes of the step, the prefill and the bulk append move more
than 1 GB, four times the 256 MB MALL.

Outside the step, each timed on its own (median of 10 calls after 5 warm-up
calls, a 1 GiB write between calls so that no call finds the previous one's
data in the MALL): ``next_rows`` (chunked prefill behind a cache, rotary
append and decode, reduced-precision prefill, slot copy) and
``other_workloads`` (the 64-token and the 1500-token non-causal prefills and
the short-context decode, M=32, H=32, Hkv=8, max_len=4096, L_m ~ U{1..4096});
the last two also as roofline objects of their own
(``roofline_prefill_encoder``, ``roofline_decode_short``).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
LOWP_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix peak
FP32_MFMA_PEAK_TFLOPS = 157.3

METRIC = "decode attn HBM GB/s (% peak) + prefill TFLOP/s (% fp32 MFMA peak), 1 GPU"

# HBM bytes per dispatch measured with rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE on
# this workload, scaled by what the same counters read for a plain 1 GiB copy
# (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0).  A figure is reported only while the
# kernel source (for the decode, its kernels and its host-side work
# decomposition, hashed together) still has the hash it was measured on.
MEASURED_TRAFFIC = {
    "prefill": {"source": "prefill.hip", "sha256_16": "2e250bd89cb5273c", "bytes": 1_151_588_064},
    "decode": {"source": "decode.hip+decode_plan.h", "sha256_16": "364bc48a3b689f09", "bytes": 3_347_954_224},
    "decode_short": {"source": "decode.hip+decode_plan.h", "sha256_16": "364bc48a3b689f09", "bytes": 489_910_976},
    "prefill_encoder": {"source": "prefill_small.hip", "sha256_16": "e6ad1eee23282454", "bytes": 12_489_865},
}

def measured_traffic(kernel):
    import hashlib

    rec = MEASURED_TRAFFIC[kernel]
    h = hashlib.sha256()
    for name in rec["source"].split("+"):
        h.update(open(os.path.join(ROOT, "transformer_attention_flash_amd", "csrc", name), "rb").read())
    digest = h.hexdigest()[:16]
    return rec["bytes"] if digest == rec["sha256_16"] else None


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=10, help="untimed steps (also let the clocks settle)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    p.add_argument("--no-next-rows", action="store_true",
                   help="skip the separately timed chunked-prefill-behind-cache measurement")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy 3 times (counter calibration) and exit")
    p.add_argument("--decode-shape", metavar="M,H,HKV,D,MAX_LEN,L",
                   help="only time the decode of one shape (every sequence L keys; seeded normal caches and "
                        "queries made on the GPU; a 1 GiB fill before each call) over --steps calls, print "
                        "one JSON line and exit")
    return p.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(inp, cfg, target_s):
    """The oracle's decode on whole sequences of the same workload, on the host cores.

    The sample grows (more sequences, then repeats of all of them) until it has
    taken about ``target_s`` seconds; throughput counts the same algorithmic
    bytes as the GPU figure.
    """
    import oracle

    orc = oracle.default()

    def run(n):
        t0 = time.perf_counter()
        orc.decode(inp["q"][:n], inp["k_cache"][:n], inp["v_cache"][:n], inp["lens"][:n], n, cfg.H,
                   cfg.Hkv, cfg.d, cfg.max_len, cfg.scale)
        return time.perf_counter() - t0

    t_one = run(1)
    n = int(min(cfg.M, max(1, np.ceil(target_s / max(t_one, 1e-3)))))
    reps, total = 0, 0.0
    while total < target_s and reps < 100:
        total += run(n)
        reps += 1
    lens = inp["lens"][:n]
    nbytes = (2 * cfg.Hkv * cfg.d * 4 * int(lens.sum()) + 2 * n * cfg.H * cfg.d * 4) * reps
    return {
        "value": round(nbytes / total / 1e9, 4),
        "unit": "GB/s",
        "cores": orc.num_threads(),
        "kind": "oracle",
        "sample": f"fp64 oracle decode of the first {n} of {cfg.M} sequences (all {cfg.H} heads, "
                  f"sum L = {int(lens.sum())} keys) of the same workload, run {reps} times, {total:.1f} s wall",
    }


def oracle_timings(wl, gpu_us, prefill3_inputs):
    """The oracle on each workload of the calls (one wall-clock run each; the
    64- and 1500-token prefills also on one thread), with its speedup of the GPU
    figure measured in the same run.  Large workloads run a sample: the causal
    prefill a set of query rows, the long-context decode (the ``cpu_baseline``
    object) a bounded number of sequences.
    """
    import oracle

    orc = oracle.default()
    threads = orc.num_threads()
    out = {"threads": threads}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    for cid in (1, 2):
        c = wl.PREFILL[cid]
        q, k, v = wl.prefill_inputs(c)
        run = lambda: orc.prefill(q, k, v, c.B, c.S, c.H, c.d, c.scale, c.causal)
        t_all = timed(run)
        orc.set_num_threads(1)
        t_one = timed(run)
        orc.set_num_threads(threads)
        out[c.name] = {"gflops": round(c.flops / t_all / 1e9, 3), "s": round(t_all, 3),
                       "gflops_1thread": round(c.flops / t_one / 1e9, 3), "s_1thread": round(t_one, 3),
                       "gpu_speedup": round(t_all / (gpu_us[c.name] * 1e-6), 1)}
    c3 = wl.PREFILL[3]
    q, k, v = prefill3_inputs
    rows = np.arange(0, c3.S, 64)  # every 64th query, every batch element and head
    sel = np.array([(b, i, h) for b in range(c3.B) for i in rows for h in range(c3.H)], np.int64)
    t3 = timed(lambda: orc.prefill_rows(q, k, v, sel, c3.B, c3.S, c3.H, c3.d, c3.scale, True))
    f3 = int(sum(4 * c3.d * (int(i) + 1) for _, i, _ in sel))
    out[c3.name] = {"gflops": round(f3 / t3 / 1e9, 3), "s": round(t3, 3),
                    "sample": f"query rows 0, 64, ..., {int(rows[-1])} of every (b, h): {len(sel)} rows",
                    "gpu_speedup": round((c3.flops / (gpu_us[c3.name] * 1e-6)) / (f3 / t3), 1)}
    sc = wl.BULK_SCATTER
    kc = wl.sentinel_cache((sc.M, sc.Hkv, sc.max_len, sc.d))
    vc = kc.copy()
    ts = timed(lambda: orc.scatter(k, v, kc, vc, np.zeros(sc.M, np.int32), sc.M, sc.n_new, sc.Hkv, sc.d,
                                   sc.max_len))
    out[sc.name] = {"gbs": round(sc.bytes / ts / 1e9, 3), "s": round(ts, 3),
                    "gpu_speedup": round(ts / (gpu_us[sc.name] * 1e-6), 1)}
    del kc, vc
    c4 = wl.DECODE[4]
    d4 = wl.decode_inputs(c4)
    t4 = timed(lambda: orc.decode(d4["q"], d4["k_cache"], d4["v_cache"], d4["lens"], c4.M, c4.H, c4.Hkv, c4.d,
                                  c4.max_len, c4.scale))
    b4 = c4.decode_bytes(d4["lens"])
    out[c4.name] = {"gbs": round(b4 / t4 / 1e9, 3), "s": round(t4, 3),
                    "gpu_speedup": round(t4 / (gpu_us[c4.name] * 1e-6), 1)}
    return out


class Evictor:
    """A 1 GiB buffer whose fill (a plain write kernel, outside the timed events) leaves
    nothing of the previous call's data in the 256 MB MALL."""

    def __init__(self, torch, dev):
        self.buf = torch.empty(1 << 28, device=dev)

    def __call__(self):
        self.buf.fill_(1.0)


def time_call(torch, run, filler=None, warm=5, reps=10, evict=None):
    """Median milliseconds of `run` over `reps` calls, each bracketed by events on the current stream.

    `filler` (a long call) is enqueued first, so that the GPU is still busy with it
    while the host enqueues the timed calls: the events then see GPU time only,
    not the host's launch latency between two short calls.  `evict`, if given,
    runs before every timed call, outside its events.
    """
    for _ in range(warm):
        run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    if filler is not None:
        filler()
    for e0, e1 in ev:
        if evict is not None:
            evict()
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))


def decode_shape(torch, taf, wl, dev, args):
    """One decode shape on its own: batch M, H query heads over Hkv KV heads of
    head_dim D, caches of MAX_LEN rows of which every sequence attends L."""
    M, H, Hkv, d, max_len, L = (int(x) for x in args.decode_shape.split(","))
    g = torch.Generator(device=dev)
    g.manual_seed(20240611)
    kc = torch.randn(M, Hkv, max_len, d, device=dev, generator=g)
    vc = torch.randn(M, Hkv, max_len, d, device=dev, generator=g)
    q = torch.randn(M, H * d, device=dev, generator=g)
    out = torch.empty_like(q)
    lens = [L] * M
    ws = torch.empty(taf.attn_decode_workspace_bytes(M, H, d, max_len) // 4, device=dev)
    scale = wl.scale_for(d)
    run = lambda: taf.attn_decode_gqa_batched(q, kc, vc, lens, out, M, H, Hkv, d, max_len, scale, ws)
    ms = time_call(torch, run, reps=max(1, args.steps), evict=Evictor(torch, dev))
    nbytes = 2 * Hkv * d * 4 * M * L + 2 * M * H * d * 4
    print(json.dumps({"decode_shape": {"M": M, "H": H, "Hkv": Hkv, "d": d, "max_len": max_len, "L": L},
                      "median_us": round(ms * 1e3, 2), "algorithmic_bytes": nbytes,
                      "gbs": round(nbytes / ms / 1e6, 1), "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
                      "note": "median of the timed calls, a 1 GiB fill before each, outside its events"}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library and this benchmark have no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch

    import transformer_attention_flash_amd as taf
    from transformer_attention_flash_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        # A plain copy of known size: 1 GiB read and 1 GiB written per dispatch.
        src = torch.ones(1 << 28, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_dispatch": {"read": 1 << 30, "write": 1 << 30}}))
        return
    taf.library()  # fail loudly before any setup if the HIP library is missing
    if args.decode_shape:
        decode_shape(torch, taf, wl, dev, args)
        return

    pcfg, scfg, dcfg = wl.PREFILL[3], wl.BULK_SCATTER, wl.DECODE[5]

    log("generating inputs ...")
    q, k, v = wl.prefill_inputs(pcfg)
    dinp = wl.decode_inputs(dcfg)
    lens = dinp["lens"]

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    pq, pk, pv = up(q), up(k), up(v)
    pout = torch.empty_like(pq)
    cache_shape = (scfg.M, scfg.Hkv, scfg.max_len, scfg.d)
    bk = torch.from_numpy(wl.sentinel_cache(cache_shape)).to(dev)
    bv = torch.from_numpy(wl.sentinel_cache(cache_shape)).to(dev)
    dq, dkn, dvn = up(dinp["q"]), up(dinp["k_new"]), up(dinp["v_new"])
    dkc, dvc = up(dinp["k_cache"]), up(dinp["v_cache"])
    dout = torch.empty((dcfg.M, dcfg.H * dcfg.d), device=dev)
    ws = torch.empty(taf.attn_decode_workspace_bytes(dcfg.M, dcfg.H, dcfg.d, dcfg.max_len) // 4, device=dev)
    evict = Evictor(torch, dev)
    torch.cuda.synchronize()
    log("inputs resident on the GPU")

    append_pos = (lens - 1).tolist()
    lens_list = lens.tolist()
    names = ("prefill", "bulk_scatter", "append", "decode")
    calls = {
        "prefill": lambda: taf.attn_prefill(pq, pk, pv, pout, pcfg.B, pcfg.S, pcfg.H, pcfg.d, pcfg.scale, True),
        "bulk_scatter": lambda: taf.kv_cache_scatter(pk, pv, bk, bv, [0] * scfg.M, scfg.M, scfg.n_new,
                                                     scfg.Hkv, scfg.d, scfg.max_len),
        "append": lambda: taf.kv_cache_scatter(dkn, dvn, dkc, dvc, append_pos, dcfg.M, 1, dcfg.Hkv, dcfg.d,
                                               dcfg.max_len),
        "decode": lambda: taf.attn_decode_gqa_batched(dq, dkc, dvc, lens_list, dout, dcfg.M, dcfg.H, dcfg.Hkv,
                                                      dcfg.d, dcfg.max_len, dcfg.scale, ws),
    }

    def step(events=None):
        for i, n in enumerate(names):
            if events is not None:
                events[n][0].record()
            calls[n]()
            if events is not None:
                events[n][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    samples = {n: np.array([e[n][0].elapsed_time(e[n][1]) for e in evs]) for n in names}
    per = {n: float(np.median(samples[n])) for n in names}  # ms; every rate below uses the median

    def spread(n):
        """mean / min / p90 of one call's event times over the timed steps (us)."""
        x = samples[n] * 1e3
        return {"mean_us": round(float(np.mean(x)), 2), "min_us": round(float(np.min(x)), 2),
                "p90_us": round(float(np.percentile(x, 90)), 2)}
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step; medians: " +
        ", ".join(f"{n} {per[n] * 1e3:.1f} us" for n in names))

    if not (torch.isfinite(pout).all() and torch.isfinite(dout).all()):
        raise RuntimeError("non-finite outputs")

    pre_flops = pcfg.flops
    pre_tflops = pre_flops / (per["prefill"] * 1e-3) / 1e12
    dec_bytes = dcfg.decode_bytes(lens)
    dec_gbs = dec_bytes / (per["decode"] * 1e-3) / 1e9
    blk_gbs = scfg.bytes / (per["bulk_scatter"] * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(dec_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "causal prefill B4 S2048 H32 d128 + bulk KV append into [4,32,4096,128] from 0, "
                        "then GQA decode step M16 H64 Hkv8 d128 max_len 32768 L~U{16384..32768} "
                        "(append at L-1, attend over L)",
            "prefill": {"B": pcfg.B, "S": pcfg.S, "H": pcfg.H, "d": pcfg.d, "causal": True},
            "decode": {"M": dcfg.M, "H": dcfg.H, "Hkv": dcfg.Hkv, "d": dcfg.d, "max_len": dcfg.max_len,
                       "sum_L": int(lens.sum())},
        },
        "decode": {"gbs": round(dec_gbs, 2), "frac_hbm": round(dec_gbs / HBM_PEAK_GBS, 4),
                   "median_us": round(per["decode"] * 1e3, 2), **spread("decode"), "algorithmic_bytes": dec_bytes},
        "prefill": {"tflops": round(pre_tflops, 3), "frac_mfma": round(pre_tflops / FP32_MFMA_PEAK_TFLOPS, 4),
                    "median_us": round(per["prefill"] * 1e3, 2), **spread("prefill"), "algorithmic_flops": pre_flops},
        "bulk_scatter": {"gbs": round(blk_gbs, 2), "frac_hbm": round(blk_gbs / HBM_PEAK_GBS, 4),
                         "median_us": round(per["bulk_scatter"] * 1e3, 2), **spread("bulk_scatter"),
                         "algorithmic_bytes": scfg.bytes},
        "append": {"median_us": round(per["append"] * 1e3, 2), **spread("append"), "algorithmic_bytes": dcfg.append_bytes},
        "roofline": {"kernel": "prefill_kernel<128, 8 waves, causal, 64-key tiles>", "bound": "mfma", "achieved": round(pre_tflops, 3),
                     "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(pre_tflops / FP32_MFMA_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("prefill")},
        "roofline_decode": {"kernels": "decode_split_kernel<128, 32-key chunks> + decode_combine_kernel<128>", "bound": "hbm",
                            "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                            "traffic": measured_traffic("decode")},
        "cpu_baseline": None,
        "oracle_timings": None,
        "next_rows": None,
        "other_workloads": None,
        "calibration": None,
    }

    if not args.no_next_rows:
        # Chunked prefill behind the cache the bulk append filled (rows 0..2047 of
        # each sequence): the next 2048 tokens, timed on their own, outside the step.
        ccfg = wl.CHUNK_BEHIND_CACHE
        rng = np.random.default_rng(4096)
        shape = (ccfg.M, ccfg.n_new, ccfg.H * ccfg.d)
        cq, ck, cv = (up(wl.normal(rng, shape, pcfg.std)) for _ in range(3))
        cout = torch.empty_like(cq)
        cached = [scfg.n_new] * ccfg.M
        run = lambda: taf.attn_prefill_cached(cq, ck, cv, bk, bv, cached, cout, ccfg.M, ccfg.n_new, ccfg.H,
                                              ccfg.Hkv, ccfg.d, ccfg.max_len, ccfg.scale)
        c_ms = time_call(torch, run, calls["prefill"], evict=evict)
        c_tflops = ccfg.flops(cached) / (c_ms * 1e-3) / 1e12
        result["next_rows"] = {"prefill_cached": {
            "workload": ccfg.name, "median_us": round(c_ms * 1e3, 2), "tflops": round(c_tflops, 3),
            "frac_mfma": round(c_tflops / FP32_MFMA_PEAK_TFLOPS, 4), "algorithmic_flops": ccfg.flops(cached),
            "note": "append of the chunk's K/V plus attention over 2048 cached + the chunk's own keys; "
                    "timed separately, not part of ms_per_step"}}
        log(f"prefill_cached: {c_ms * 1e3:.1f} us, {c_tflops:.1f} TFLOP/s")
        del cq, ck, cv, cout

        # Rotary embedding fused into the append and the decode: the bulk append
        # with every key rotated (base 10000), and the decode step with the new
        # key rotated into the cache and the query rotated (base 1e6, as Qwen).
        rot = pcfg.d
        fill = calls["prefill"]
        r_bulk = time_call(torch, lambda: taf.kv_cache_scatter_rope(pk, pv, bk, bv, [0] * scfg.M, scfg.M, scfg.n_new,
                                                                    scfg.Hkv, scfg.d, scfg.max_len, rot, 1e4), fill, evict=evict)
        r_app = time_call(torch, lambda: taf.kv_cache_scatter_rope(dkn, dvn, dkc, dvc, append_pos, dcfg.M, 1,
                                                                   dcfg.Hkv, dcfg.d, dcfg.max_len, rot, 1e6), fill, evict=evict)
        r_dec = time_call(torch, lambda: taf.attn_decode_gqa_batched_rope(dq, dkc, dvc, lens_list, dout, dcfg.M,
                                                                          dcfg.H, dcfg.Hkv, dcfg.d, dcfg.max_len,
                                                                          dcfg.scale, rot, 1e6, ws), fill, evict=evict)
        # The chunk behind the cache with its queries and keys rotated (base 10000).
        rng_r = np.random.default_rng(4098)
        rshape = (ccfg.M, ccfg.n_new, ccfg.H * ccfg.d)
        rq, rk, rv = (up(wl.normal(rng_r, rshape, pcfg.std)) for _ in range(3))
        rout = torch.empty_like(rq)
        r_chunk = time_call(torch, lambda: taf.attn_prefill_cached_rope(rq, rk, rv, bk, bv, cached, rout, ccfg.M,
                                                                        ccfg.n_new, ccfg.H, ccfg.Hkv, ccfg.d,
                                                                        ccfg.max_len, ccfg.scale, rot, 1e4),
                            fill, evict=evict)
        del rq, rk, rv, rout
        r_blk_gbs = scfg.bytes / (r_bulk * 1e-3) / 1e9
        r_dec_gbs = dec_bytes / (r_dec * 1e-3) / 1e9
        result["next_rows"]["rope"] = {
            "bulk_scatter_rope": {"median_us": round(r_bulk * 1e3, 2), "gbs": round(r_blk_gbs, 2),
                                  "frac_hbm": round(r_blk_gbs / HBM_PEAK_GBS, 4), "rotary_ndims": rot,
                                  "theta": 1e4, "plain_us": round(per["bulk_scatter"] * 1e3, 2)},
            "append_rope": {"median_us": round(r_app * 1e3, 2), "plain_us": round(per["append"] * 1e3, 2)},
            "prefill_cached_rope": {"workload": ccfg.name, "median_us": round(r_chunk * 1e3, 2),
                                    "tflops": round(ccfg.flops(cached) / (r_chunk * 1e-3) / 1e12, 3),
                                    "rotary_ndims": rot, "theta": 1e4,
                                    "plain_us": result["next_rows"]["prefill_cached"]["median_us"]},
            "decode_rope": {"median_us": round(r_dec * 1e3, 2), "gbs": round(r_dec_gbs, 2),
                            "frac_hbm": round(r_dec_gbs / HBM_PEAK_GBS, 4), "rotary_ndims": rot, "theta": 1e6,
                            "plain_us": round(per["decode"] * 1e3, 2)},
            "note": "timed separately (median of 10 calls after 5 warm-up calls, queued behind a prefill, "
                    "a 1 GiB write between calls), not part of ms_per_step"}
        log(f"rope: bulk append {r_bulk * 1e3:.1f} us ({r_blk_gbs:.0f} GB/s), append {r_app * 1e3:.1f} us, "
            f"decode {r_dec * 1e3:.1f} us ({r_dec_gbs:.0f} GB/s), chunk behind cache {r_chunk * 1e3:.1f} us")

        # Reduced-precision prefill: the step's causal prefill on 16-bit MFMA operands.
        lowp = {}
        for pname, prec in (("fp16", taf.ATTN_PREC_FP16), ("bf16", taf.ATTN_PREC_BF16)):
            lp_ms = time_call(torch, lambda: taf.attn_prefill_lowp(pq, pk, pv, pout, pcfg.B, pcfg.S, pcfg.H, pcfg.d,
                                                                   pcfg.scale, True, prec), fill, evict=evict)
            lp_tf = pre_flops / (lp_ms * 1e-3) / 1e12
            lowp[pname] = {"median_us": round(lp_ms * 1e3, 2), "tflops": round(lp_tf, 3),
                           "frac_mfma": round(lp_tf / LOWP_MFMA_PEAK_TFLOPS, 4)}
            log(f"prefill {pname}: {lp_ms * 1e3:.1f} us, {lp_tf:.1f} TFLOP/s")
        result["next_rows"]["prefill_lowp"] = {
            "workload": pcfg.name, "algorithmic_flops": pre_flops, "peak_tflops": LOWP_MFMA_PEAK_TFLOPS, **lowp,
            "note": "f32 in and out, q/k/v and probabilities rounded to the 16-bit type for the MFMA operands"}

        # Slot copy: a single-sequence cache holding a 2048-token prefill (the
        # bulk-append cache's slot 0) copied into slot 3 of the same batched shape.
        sk, sv = bk[0], bv[0]
        dk, dv = torch.empty_like(bk), torch.empty_like(bv)
        s_ms = time_call(torch, lambda: taf.kv_cache_copy_to_slot(sk, sv, scfg.max_len, scfg.n_new, dk, dv, 3,
                                                                  scfg.M, scfg.Hkv, scfg.d, scfg.max_len), fill, evict=evict)
        s_bytes = 2 * 2 * scfg.Hkv * scfg.n_new * scfg.d * 4
        s_gbs = s_bytes / (s_ms * 1e-3) / 1e9
        result["next_rows"]["slot_copy"] = {
            "workload": f"copy of {scfg.n_new} rows x {scfg.Hkv} KV heads x d {scfg.d} (K and V) into slot 3",
            "median_us": round(s_ms * 1e3, 2), "gbs": round(s_gbs, 2), "frac_hbm": round(s_gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": s_bytes}
        log(f"slot copy: {s_ms * 1e3:.1f} us ({s_gbs:.0f} GB/s)")
        del dk, dv

        # The other workloads of the same calls, each timed on its own: the two
        # small non-causal prefills and the short-context GQA decode step.
        others = {}
        for cid in (1, 2):
            c = wl.PREFILL[cid]
            oq, ok_, ov = (up(x) for x in wl.prefill_inputs(c))
            oo = torch.empty_like(oq)
            o_ms = time_call(torch, lambda: taf.attn_prefill(oq, ok_, ov, oo, c.B, c.S, c.H, c.d, c.scale, c.causal),
                             fill, evict=evict)
            o_tf = c.flops / (o_ms * 1e-3) / 1e12
            others[c.name] = {"median_us": round(o_ms * 1e3, 2), "tflops": round(o_tf, 3),
                              "frac_mfma": round(o_tf / FP32_MFMA_PEAK_TFLOPS, 4), "algorithmic_flops": c.flops}
            log(f"prefill {c.name}: {o_ms * 1e3:.1f} us, {o_tf:.1f} TFLOP/s")
            del oq, ok_, ov, oo
        c4 = wl.DECODE[4]
        d4 = wl.decode_inputs(c4)
        l4 = d4["lens"]
        q4, kn4, vn4, kc4, vc4 = (up(d4[n]) for n in ("q", "k_new", "v_new", "k_cache", "v_cache"))
        out4 = torch.empty((c4.M, c4.H * c4.d), device=dev)
        ws4 = torch.empty(taf.attn_decode_workspace_bytes(c4.M, c4.H, c4.d, c4.max_len) // 4, device=dev)
        a4_ms = time_call(torch, lambda: taf.kv_cache_scatter(kn4, vn4, kc4, vc4, (l4 - 1).tolist(), c4.M, 1, c4.Hkv,
                                                              c4.d, c4.max_len), fill, evict=evict)
        d4_ms = time_call(torch, lambda: taf.attn_decode_gqa_batched(q4, kc4, vc4, l4.tolist(), out4, c4.M, c4.H,
                                                                     c4.Hkv, c4.d, c4.max_len, c4.scale, ws4), fill, evict=evict)
        d4_bytes = c4.decode_bytes(l4)
        d4_gbs = d4_bytes / (d4_ms * 1e-3) / 1e9
        others[c4.name] = {"decode_median_us": round(d4_ms * 1e3, 2), "gbs": round(d4_gbs, 2),
                           "frac_hbm": round(d4_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": d4_bytes,
                           "append_median_us": round(a4_ms * 1e3, 2), "sum_L": int(l4.sum())}
        log(f"decode {c4.name}: {d4_ms * 1e3:.1f} us ({d4_gbs:.0f} GB/s), append {a4_ms * 1e3:.1f} us")
        c2 = wl.PREFILL[2]
        tf2 = others[c2.name]["tflops"]
        result["roofline_prefill_encoder"] = {
            "workload": c2.name, "kernel": "prefill_small_kernel<64, 3 query waves, non-causal>", "bound": "mfma",
            "achieved": tf2, "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf2 / FP32_MFMA_PEAK_TFLOPS, 4), "traffic": measured_traffic("prefill_encoder")}
        result["roofline_decode_short"] = {
            "workload": c4.name, "kernels": "decode_split_kernel<128, 16-key chunks> + decode_combine_kernel<128>", "bound": "hbm",
            "achieved": round(d4_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(d4_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("decode_short")}
        del q4, kn4, vn4, kc4, vc4, out4, ws4
        others["note"] = ("timed separately (median of 10 calls after 5 warm-up calls, queued behind a prefill, "
                          "a 1 GiB write between calls)")
        result["other_workloads"] = others

    if not args.no_next_rows:
        # Context for the roofline peaks, measured on this device with library
        # routines (not this package's kernels): an fp32 GEMM and a device copy.
        a32 = torch.randn(8192, 8192, device=dev)
        mm_ms = time_call(torch, lambda: torch.mm(a32, a32), None, warm=2, reps=5)
        cp_src = torch.empty(1 << 28, device=dev)
        cp_dst = torch.empty_like(cp_src)
        cp_ms = time_call(torch, lambda: cp_dst.copy_(cp_src), None, warm=2, reps=5)
        result["calibration"] = {
            "torch_mm_f32_8192_tflops": round(2 * 8192 ** 3 / (mm_ms * 1e-3) / 1e12, 2),
            "torch_copy_1GiB_gbs": round(2 * (1 << 30) / (cp_ms * 1e-3) / 1e9, 1),
            "note": "library routines on this device, for context next to the spec peaks"}
        log(f"calibration: fp32 GEMM {result['calibration']['torch_mm_f32_8192_tflops']} TFLOP/s, "
            f"copy {result['calibration']['torch_copy_1GiB_gbs']} GB/s")
        del a32, cp_src, cp_dst

    # Free the GPU copies before the host-side leg.
    del pq, pk, pv, pout, bk, bv, dq, dkn, dvn, dkc, dvc, dout, ws
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample of the decode workload ...")
        result["cpu_baseline"] = cpu_baseline(dinp, dcfg, args.cpu_seconds)
        if result["other_workloads"] is not None:
            ow = result["other_workloads"]
            gpu_us = {wl.PREFILL[1].name: ow[wl.PREFILL[1].name]["median_us"],
                      wl.PREFILL[2].name: ow[wl.PREFILL[2].name]["median_us"],
                      pcfg.name: result["prefill"]["median_us"], scfg.name: result["bulk_scatter"]["median_us"],
                      wl.DECODE[4].name: ow[wl.DECODE[4].name]["decode_median_us"]}
            log("timing the CPU oracle on the other workloads ...")
            result["oracle_timings"] = oracle_timings(wl, gpu_us, (q, k, v))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
