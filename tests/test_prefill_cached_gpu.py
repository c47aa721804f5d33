"""Chunked prefill behind an existing KV cache on the GPU, against the fp64 oracle.

Small cases: ragged cached lengths (0 and up to max_len - n_new), chunks that
span several 128-query and 32-key tiles with ragged tails, GQA groups, every
head_dim, NaN in the cache rows not yet written (they must never be read).
Both outputs are checked: the attention (abs 1e-4, normwise rel 1e-3) and the
appended caches (bit-exact against the oracle's append).  GPU-side relations:
an empty cache with Hkv = H gives the causal prefill; two chunks give the same
outputs as one; a captured HIP graph replays to the eager result.  Mid-size
chunks that take each of the launcher's kernels, and at full size the second
half of the causal prefill workload behind its first half (M=4, H=32, d=128,
2048 cached + 2048 new of 4096) and a 256-token chunk behind long GQA
contexts (M=16, H=64, Hkv=8, 16K-32K cached), are compared output for output
against the numpy formulation of the oracle (oracle/brute.py, pinned to the
C oracle).
"""
import numpy as np
import pytest

import oracle
import transformer_attention_flash_amd as taf
from transformer_attention_flash_amd import workloads as wl
from gpu_common import assert_attn_close, bits, nan_like, note, to_dev, to_host
from oracle import brute

pytestmark = pytest.mark.gpu

SMALL = [
    # M, n_new, H, Hkv, d, max_len, lens (None = random)
    (1, 1, 1, 1, 32, 1, [0]),
    (2, 31, 4, 4, 64, 100, [0, 69]),
    (3, 129, 8, 2, 128, 300, [0, 17, 171]),
    (2, 200, 16, 2, 64, 700, None),
    (4, 64, 6, 3, 128, 512, None),
    (1, 300, 4, 1, 32, 301, [1]),
    (5, 40, 8, 8, 128, 200, [160, 0, 33, 128, 100]),
]


def make_case(seed, M, n, H, Hkv, d, max_len, lens):
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(0, max_len - n + 1, size=M)
    lens = np.asarray(lens, np.int32)
    q = rng.standard_normal((M, n, H * d), dtype=np.float32)
    kn = rng.standard_normal((M, n, Hkv * d), dtype=np.float32)
    vn = rng.standard_normal((M, n, Hkv * d), dtype=np.float32)
    kc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    vc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    for m in range(M):
        kc[m, :, lens[m]:] = np.nan
        vc[m, :, lens[m]:] = np.nan
    return lens, q, kn, vn, kc, vc


def run_gpu(lens, q, kn, vn, kc, vc, M, n, H, Hkv, d, max_len, scale):
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    out = nan_like((M, n, H * d))
    taf.attn_prefill_cached(to_dev(q), to_dev(kn), to_dev(vn), kc_d, vc_d, lens.tolist(), out, M, n, H, Hkv, d,
                            max_len, scale)
    return to_host(out), kc_d, vc_d


@pytest.mark.parametrize("case", SMALL, ids=[f"M{c[0]}_n{c[1]}_H{c[2]}_Hkv{c[3]}_d{c[4]}_max{c[5]}" for c in SMALL])
def test_prefill_cached_small(case):
    M, n, H, Hkv, d, max_len, lens = case
    lens, q, kn, vn, kc, vc = make_case(7 * M + n + H, M, n, H, Hkv, d, max_len, lens)
    scale = wl.scale_for(d)
    note(f"prefill_cached M={M} n={n} H={H} Hkv={Hkv} d={d} max_len={max_len} lens={lens.tolist()}")
    got, kc_d, vc_d = run_gpu(lens, q, kn, vn, kc, vc, M, n, H, Hkv, d, max_len, scale)
    orc = oracle.default()
    want = orc.prefill_cached(q, kn, vn, kc, vc, lens, M, n, H, Hkv, d, max_len, scale)
    assert_attn_close(got, want, f"prefill_cached {case}")
    kc2, vc2 = kc.copy(), vc.copy()
    orc.scatter(kn, vn, kc2, vc2, lens, M, n, Hkv, d, max_len)
    assert np.array_equal(bits(to_host(kc_d)), bits(kc2)), "K cache after the append"
    assert np.array_equal(bits(to_host(vc_d)), bits(vc2)), "V cache after the append"


def test_prefill_cached_empty_cache_is_causal_prefill():
    M, n, H, d, max_len = 2, 250, 4, 128, 256
    lens, q, kn, vn, kc, vc = make_case(3, M, n, H, H, d, max_len, [0, 0])
    scale = wl.scale_for(d)
    note("prefill_cached vs attn_prefill")
    got, _, _ = run_gpu(lens, q, kn, vn, kc, vc, M, n, H, H, d, max_len, scale)
    out = nan_like((M, n, H * d))
    taf.attn_prefill(to_dev(q), to_dev(kn), to_dev(vn), out, M, n, H, d, scale, True)
    assert np.max(np.abs(got - to_host(out))) <= 2e-5


def test_prefill_cached_two_chunks_equal_one():
    M, S, s1, H, Hkv, d, max_len = 3, 300, 130, 8, 2, 64, 320
    lens0 = np.zeros(M, np.int32)
    _, q, kn, vn, kc, vc = make_case(5, M, S, H, Hkv, d, max_len, lens0)
    scale = wl.scale_for(d)
    note("prefill_cached two chunks")
    whole, _, _ = run_gpu(lens0, q, kn, vn, kc, vc, M, S, H, Hkv, d, max_len, scale)
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    parts = []
    for lo, hi in ((0, s1), (s1, S)):
        out = nan_like((M, hi - lo, H * d))
        taf.attn_prefill_cached(to_dev(np.ascontiguousarray(q[:, lo:hi])), to_dev(np.ascontiguousarray(kn[:, lo:hi])),
                                to_dev(np.ascontiguousarray(vn[:, lo:hi])), kc_d, vc_d, [lo] * M, out, M, hi - lo, H,
                                Hkv, d, max_len, scale)
        parts.append(to_host(out))
    assert np.max(np.abs(np.concatenate(parts, axis=1) - whole)) <= 2e-5
    want = oracle.default().prefill_cached(q, kn, vn, kc, vc, lens0, M, S, H, Hkv, d, max_len, scale)
    assert_attn_close(whole, want, "whole chunk vs oracle")


CACHED_DECOMPOSITIONS = [
    # M, n, H, Hkv, d, max_len, lens: which kernel the launcher picks (M*H*ceil(n/128)
    # four-wave workgroups and the mean cached length P decide)
    (2, 1100, 16, 4, 64, 1600, [100, 480]),   # 288 workgroups, P < n: 16-query waves
    (1, 700, 32, 8, 128, 2000, [1200]),       # 192 workgroups: 16-query waves behind a long cache
    (2, 300, 64, 8, 128, 1300, [600, 950]),   # 384 workgroups, P > n: four waves
    (2, 200, 64, 8, 64, 900, [500, 700]),     # 256 workgroups, P > n: four waves at d = 64
    (1, 2100, 48, 16, 32, 2200, [64]),        # 816 workgroups at d = 32, P < n: 16-query waves
    (2, 1000, 64, 8, 128, 2100, [600, 1030]), # 512 eight-wave workgroups, 64-key tiles, ragged P + n
    (2, 1000, 64, 8, 128, 2100, [40, 1080]),  # the same; each diagonal starts 40 and 56 keys into a 64-key tile
    (2, 1000, 64, 8, 64, 2100, [600, 1030]),  # eight waves, 64-key tiles at d = 64
]


@pytest.mark.parametrize("case", CACHED_DECOMPOSITIONS,
                         ids=[f"M{c[0]}_n{c[1]}_H{c[2]}_Hkv{c[3]}_d{c[4]}" for c in CACHED_DECOMPOSITIONS])
def test_prefill_cached_decompositions(case):
    M, n, H, Hkv, d, max_len, lens = case
    lens, q, kn, vn, kc, vc = make_case(11 * M + n + d, M, n, H, Hkv, d, max_len, lens)
    scale = wl.scale_for(d)
    note(f"prefill_cached decomposition M={M} n={n} H={H} Hkv={Hkv} d={d} lens={lens.tolist()}")
    got, _, _ = run_gpu(lens, q, kn, vn, kc, vc, M, n, H, Hkv, d, max_len, scale)
    want = brute.prefill_cached(q, kn, vn, kc, vc, lens, M, n, H, Hkv, d, max_len, scale)
    assert_attn_close(got, want, f"prefill_cached {case}")


def test_prefill_cached_second_half_of_causal_prefill_full_size():
    """Chunk of 2048 tokens behind 2048 cached (the causal prefill workload's two halves)."""
    cfg = wl.PREFILL[3]
    M, H, d, max_len, P = cfg.B, cfg.H, cfg.d, 4096, 2048
    q, k, v = wl.prefill_inputs(cfg)      # the first half's K/V fill the cache
    rng = np.random.default_rng(2048)
    q2 = (rng.standard_normal(q.shape, dtype=np.float32) * np.float32(cfg.std))
    k2 = (rng.standard_normal(k.shape, dtype=np.float32) * np.float32(cfg.std))
    v2 = (rng.standard_normal(v.shape, dtype=np.float32) * np.float32(cfg.std))
    kc = wl.sentinel_cache((M, H, max_len, d))
    vc = kc.copy()
    orc = oracle.default()
    orc.scatter(k, v, kc, vc, np.zeros(M, np.int32), M, P, H, d, max_len)
    lens = np.full(M, P, np.int32)
    note("prefill_cached full size: 2048 behind 2048")
    got, kc_d, vc_d = run_gpu(lens, q2, k2, v2, kc, vc, M, 2048, H, H, d, max_len, cfg.scale)
    want = brute.prefill_cached(q2, k2, v2, kc, vc, lens, M, 2048, H, H, d, max_len, cfg.scale)
    assert_attn_close(got, want, "2048 behind 2048 (all outputs)")
    orc.scatter(k2, v2, kc, vc, lens, M, 2048, H, d, max_len)
    assert np.array_equal(bits(to_host(kc_d)), bits(kc)), "K cache after the append"
    assert np.array_equal(bits(to_host(vc_d)), bits(vc)), "V cache after the append"


def test_prefill_cached_long_gqa_context_full_size():
    """A 256-token chunk behind 16K-32K cached rows of the long-context GQA cache."""
    cfg = wl.DECODE[5]
    M, H, Hkv, d, max_len, n = cfg.M, cfg.H, cfg.Hkv, cfg.d, cfg.max_len, 256
    inp = wl.decode_inputs(cfg)
    lens = np.minimum(inp["lens"], max_len - n).astype(np.int32)
    rng = np.random.default_rng(512)
    q = rng.standard_normal((M, n, H * d), dtype=np.float32)
    kn = rng.standard_normal((M, n, Hkv * d), dtype=np.float32)
    vn = rng.standard_normal((M, n, Hkv * d), dtype=np.float32)
    note("prefill_cached full size: 256 behind long GQA contexts")
    got, _, _ = run_gpu(lens, q, kn, vn, inp["k_cache"], inp["v_cache"], M, n, H, Hkv, d, max_len, cfg.scale)
    want = brute.prefill_cached(q, kn, vn, inp["k_cache"], inp["v_cache"], lens, M, n, H, Hkv, d, max_len,
                                cfg.scale)
    assert_attn_close(got, want, "256 behind long contexts (all outputs)")


def test_prefill_cached_graph_replays_match_eager():
    """Append + attention of a chunk captured into a HIP graph: every replay (new chunk
    contents, same cached lengths) gives the eager outputs and caches, bit for bit."""
    import torch
    M, n, H, Hkv, d, max_len = 2, 300, 16, 4, 64, 1000
    lens = [250, 600]
    rng = np.random.default_rng(890)
    scale = wl.scale_for(d)
    kc0 = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    vc0 = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    qs = (M, n, H * d)
    ns = (M, n, Hkv * d)
    q_s, kn_s, vn_s = to_dev(np.zeros(qs, np.float32)), to_dev(np.zeros(ns, np.float32)), to_dev(np.zeros(ns, np.float32))
    kc_s, vc_s = to_dev(kc0), to_dev(vc0)
    out_s = torch.zeros(qs, device="cuda:0")
    note("prefill_cached graph capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        taf.attn_prefill_cached(q_s, kn_s, vn_s, kc_s, vc_s, lens, out_s, M, n, H, Hkv, d, max_len, scale)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        taf.attn_prefill_cached(q_s, kn_s, vn_s, kc_s, vc_s, lens, out_s, M, n, H, Hkv, d, max_len, scale)
    for rep in range(3):
        q = rng.standard_normal(qs, dtype=np.float32)
        kn = rng.standard_normal(ns, dtype=np.float32)
        vn = rng.standard_normal(ns, dtype=np.float32)
        for dst, src in ((q_s, q), (kn_s, kn), (vn_s, vn)):
            dst.copy_(to_dev(src))
        graph.replay()
        torch.cuda.synchronize()
        got, got_kc = to_host(out_s), to_host(kc_s)
        eager, eager_kc, _ = run_gpu(np.asarray(lens, np.int32), q, kn, vn, kc0, vc0, M, n, H, Hkv, d, max_len, scale)
        assert np.array_equal(bits(got), bits(eager)), f"replay {rep}: attention differs from the eager call"
        assert np.array_equal(bits(got_kc), bits(to_host(eager_kc))), f"replay {rep}: K cache differs"
