"""HIP-graph capture of the entry points whose replays the other GPU test files do not
cover: the append (plain and rotating), the slot copy, the rotating decode and the rotary
chunked prefill.

Each operation is captured once into a graph on static buffers and replayed three times,
with new inputs written between replays by eager torch work.  After every replay the same
call is made eagerly on a second set of buffers that started identical; outputs and
caches must agree bit for bit (the library enqueues kernels only, no memsets or copies,
so a replay does exactly what the eager call does).
"""
from __future__ import annotations

import numpy as np
import pytest

from gpu_common import bits, note, to_dev, to_host
import transformer_attention_flash_amd as taf
from transformer_attention_flash_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _capture(fn):
    """Warm fn up on a side stream (first-call host queries), then capture it."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def _refill(rng, *tensors):
    """New standard-normal contents for static input tensors (eager device work)."""
    for t in tensors:
        t.copy_(to_dev(rng.standard_normal(tuple(t.shape), dtype=np.float32)))


def _same(a, b, what):
    assert np.array_equal(bits(to_host(a)), bits(to_host(b))), what


@pytest.mark.parametrize("rope", [False, True], ids=["plain", "rope"])
def test_append_graph_replays_match_eager(rope):
    import torch

    M, n_new, Hkv, d, max_len = 3, 5, 4, 128, 64
    lens = [0, 17, 59]
    rng = np.random.default_rng(901 + int(rope))
    k_new = to_dev(rng.standard_normal((M, n_new, Hkv * d), dtype=np.float32))
    v_new = to_dev(rng.standard_normal((M, n_new, Hkv * d), dtype=np.float32))
    base = to_dev(rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32))
    caches = {side: (base.clone(), base.clone()) for side in ("graph", "eager")}

    def call(kc, vc):
        if rope:
            taf.kv_cache_scatter_rope(k_new, v_new, kc, vc, lens, M, n_new, Hkv, d, max_len, 64, 1e4)
        else:
            taf.kv_cache_scatter(k_new, v_new, kc, vc, lens, M, n_new, Hkv, d, max_len)

    note(f"append graph capture (rope={rope})")
    graph = _capture(lambda: call(*caches["graph"]))
    for rep in range(3):
        _refill(rng, k_new, v_new)
        graph.replay()
        torch.cuda.synchronize()
        call(*caches["eager"])
        _same(caches["graph"][0], caches["eager"][0], f"K cache after replay {rep}")
        _same(caches["graph"][1], caches["eager"][1], f"V cache after replay {rep}")


def test_slot_copy_graph_replays_match_eager():
    import torch

    M, Hkv, d, max_len, src_max_len, seq_len, slot = 4, 2, 64, 96, 80, 70, 2
    rng = np.random.default_rng(907)
    src_k = to_dev(rng.standard_normal((Hkv, src_max_len, d), dtype=np.float32))
    src_v = to_dev(rng.standard_normal((Hkv, src_max_len, d), dtype=np.float32))
    base = to_dev(rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32))
    caches = {side: (base.clone(), base.clone()) for side in ("graph", "eager")}

    def call(kc, vc):
        taf.kv_cache_copy_to_slot(src_k, src_v, src_max_len, seq_len, kc, vc, slot, M, Hkv, d, max_len)

    note("slot copy graph capture")
    graph = _capture(lambda: call(*caches["graph"]))
    for rep in range(3):
        _refill(rng, src_k, src_v)
        graph.replay()
        torch.cuda.synchronize()
        call(*caches["eager"])
        _same(caches["graph"][0], caches["eager"][0], f"K cache after replay {rep}")
        _same(caches["graph"][1], caches["eager"][1], f"V cache after replay {rep}")


def test_rope_decode_graph_replays_match_eager():
    import torch

    M, H, Hkv, d, max_len = 5, 16, 4, 128, 1024
    lens = [1, 1024, 0, 300, 77]
    rng = np.random.default_rng(911)
    kc = to_dev(rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32))
    vc = to_dev(rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32))
    q = to_dev(rng.standard_normal((M, H * d), dtype=np.float32))
    scale = wl.scale_for(d)
    ws = torch.empty(taf.attn_decode_workspace_bytes(M, H, d, max_len) // 4, dtype=torch.float32, device="cuda:0")
    outs = {side: torch.zeros((M, H * d), device="cuda:0") for side in ("graph", "eager")}

    def call(out):
        taf.attn_decode_gqa_batched_rope(q, kc, vc, lens, out, M, H, Hkv, d, max_len, scale, 96, 1e6, ws)

    note("rotating decode graph capture")
    graph = _capture(lambda: call(outs["graph"]))
    for rep in range(3):
        _refill(rng, q)
        graph.replay()
        torch.cuda.synchronize()
        call(outs["eager"])
        _same(outs["graph"], outs["eager"], f"output after replay {rep}")


def test_rope_chunked_prefill_graph_replays_match_eager():
    import torch

    M, n, H, Hkv, d, max_len = 2, 40, 8, 2, 64, 200
    lens = [0, 133]
    rng = np.random.default_rng(913)
    q = to_dev(rng.standard_normal((M, n, H * d), dtype=np.float32))
    k_new = to_dev(rng.standard_normal((M, n, Hkv * d), dtype=np.float32))
    v_new = to_dev(rng.standard_normal((M, n, Hkv * d), dtype=np.float32))
    base = to_dev(rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32))
    state = {side: (base.clone(), base.clone(), torch.zeros((M, n, H * d), device="cuda:0"))
             for side in ("graph", "eager")}
    scale = wl.scale_for(d)

    def call(kc, vc, out):
        taf.attn_prefill_cached_rope(q, k_new, v_new, kc, vc, lens, out, M, n, H, Hkv, d, max_len, scale, 32, 1e4)

    note("rotary chunked prefill graph capture")
    graph = _capture(lambda: call(*state["graph"]))
    for rep in range(3):
        _refill(rng, q, k_new, v_new)
        graph.replay()
        torch.cuda.synchronize()
        call(*state["eager"])
        for i, what in enumerate(("K cache", "V cache", "output")):
            _same(state["graph"][i], state["eager"][i], f"{what} after replay {rep}")
