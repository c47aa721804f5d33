"""Calls from several host threads at once, each on its own stream.

The library keeps no per-call state; what it shares between calls are caches of
per-device and per-shape host decisions (compute-unit counts, decode occupancy,
the small prefill's queries per workgroup), filled on first use.  Four threads
start together on shapes this process has not run before, so they fill those
caches concurrently, and each repeats its calls on its own stream and buffers.
Afterwards the same work runs again on one thread; every output must agree bit for
bit (the results do not depend on the stream, and the host decisions must come
out the same).
"""
from __future__ import annotations

import threading

import numpy as np
import pytest

from gpu_common import bits, note, to_dev, to_host
import transformer_attention_flash_amd as taf
from transformer_attention_flash_amd import workloads as wl

pytestmark = pytest.mark.gpu

# (prefill B, S, H, d, causal), (decode M, H, Hkv, d, max_len) per thread: shapes that
# no other test file uses, small enough that the small prefill kernel runs.
SHAPES = [
    ((1, 333, 6, 64, 0), (3, 12, 4, 64, 700)),
    ((2, 190, 5, 32, 1), (7, 20, 5, 32, 300)),
    ((1, 410, 3, 128, 1), (2, 24, 6, 128, 900)),
    ((3, 150, 7, 64, 1), (5, 8, 8, 64, 520)),
]


def _work(idx, rng_seed):
    """Device inputs and output buffers of one thread's workload."""
    import torch

    (B, S, H, d, causal), (M, Hd, Hkv, dd, max_len) = SHAPES[idx]
    rng = np.random.default_rng(rng_seed)
    w = dict(
        pre=(B, S, H, d, causal),
        q=to_dev(rng.standard_normal((B, S, H * d), dtype=np.float32)),
        k=to_dev(rng.standard_normal((B, S, H * d), dtype=np.float32)),
        v=to_dev(rng.standard_normal((B, S, H * d), dtype=np.float32)),
        dec=(M, Hd, Hkv, dd, max_len),
        lens=[int(x) for x in rng.integers(1, max_len + 1, size=M)],
        dq=to_dev(rng.standard_normal((M, Hd * dd), dtype=np.float32)),
        k_new=to_dev(rng.standard_normal((M, 1, Hkv * dd), dtype=np.float32)),
        v_new=to_dev(rng.standard_normal((M, 1, Hkv * dd), dtype=np.float32)),
        kc0=to_dev(rng.standard_normal((M, Hkv, max_len, dd), dtype=np.float32)),
        vc0=to_dev(rng.standard_normal((M, Hkv, max_len, dd), dtype=np.float32)),
    )
    w["ws"] = torch.empty(taf.attn_decode_workspace_bytes(M, Hd, dd, max_len) // 4, dtype=torch.float32,
                          device="cuda:0")
    return w


def _run(w):
    """Prefill, then a decode step (append at L - 1, attend over L); returns the device outputs."""
    import torch

    B, S, H, d, causal = w["pre"]
    M, Hd, Hkv, dd, max_len = w["dec"]
    out = torch.full((B, S, H * d), float("nan"), device="cuda:0")
    taf.attn_prefill(w["q"], w["k"], w["v"], out, B, S, H, d, wl.scale_for(d), bool(causal))
    kc, vc = w["kc0"].clone(), w["vc0"].clone()
    taf.kv_cache_scatter(w["k_new"], w["v_new"], kc, vc, [L - 1 for L in w["lens"]], M, 1, Hkv, dd, max_len)
    dout = torch.full((M, Hd * dd), float("nan"), device="cuda:0")
    taf.attn_decode_gqa_batched(w["dq"], kc, vc, w["lens"], dout, M, Hd, Hkv, dd, max_len, wl.scale_for(dd),
                                w["ws"])
    return out, kc, vc, dout


def test_concurrent_host_threads_match_one_thread():
    import torch

    works = [_work(i, 1200 + i) for i in range(len(SHAPES))]
    torch.cuda.synchronize()
    results = [None] * len(works)
    errors = []
    start = threading.Barrier(len(works))

    def thread(i):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                start.wait()
                for _ in range(3):
                    results[i] = _run(works[i])
            stream.synchronize()
        except BaseException as exc:  # reported below, on the main thread
            errors.append((i, exc))

    note("four host threads, one stream each")
    threads = [threading.Thread(target=thread, args=(i,)) for i in range(len(works))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    note("the same work on one thread")
    for i, w in enumerate(works):
        again = _run(w)
        for name, a, b in zip(("prefill", "K cache", "V cache", "decode"), results[i], again):
            assert np.array_equal(bits(to_host(a)), bits(to_host(b))), f"thread {i}: {name} differs"
        assert np.all(np.isfinite(to_host(results[i][0]))) and np.all(np.isfinite(to_host(results[i][3])))
