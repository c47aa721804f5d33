"""Batched GQA decode on the GPU against the fp64 oracle.

Small cases cover every group size class (g = 1, 2, 3, 4, 8, 16, 32 -- the
last needs two 16-head blocks), every head_dim, empty sequences, lengths on
and around split/chunk boundaries, L = max_len, M = 32, and cache rows past
L_m filled with NaN (they must never be read).  Full-size cases run the two
decode workloads as one step: append the new row at L_m - 1, then attend
over L_m keys.  Results are bitwise the same on every stream and every
repeated call, and a decode captured into a HIP graph replays to the eager
result.
"""
import numpy as np
import pytest

import oracle
import transformer_attention_flash_amd as taf
from transformer_attention_flash_amd import workloads as wl
from gpu_common import assert_attn_close, bits, nan_like, note, to_dev, to_host

pytestmark = pytest.mark.gpu

SMALL = [
    # M, H, Hkv, d, max_len, lens (None = random in [0, max_len])
    (1, 1, 1, 32, 1, [1]),
    (2, 4, 4, 64, 70, [0, 70]),
    (4, 8, 2, 128, 300, [1, 31, 32, 33]),
    (3, 16, 2, 128, 1000, [64, 65, 1000]),
    (2, 32, 2, 64, 200, [199, 128]),
    (2, 64, 2, 128, 130, [130, 7]),
    (32, 8, 8, 32, 50, None),
    (5, 12, 4, 64, 2000, [0, 511, 512, 513, 1999]),
    (2, 6, 3, 128, 5000, [4097, 1024]),
    (3, 16, 8, 128, 9000, [8999, 256, 257]),
    # 32 sequences x 64 KV heads of at most 256 keys: the bulk key-block span
    # would pass max_len, so every key block is a tail block.
    (32, 64, 64, 64, 256, None),
]

# Long contexts with enough keys per workgroup slot that the decode streams
# 32-key chunks at d = 32 and d = 64 (d = 128 is the long-context full-size
# step below; short calls stream 16-key chunks): every output is compared.
LONG = [
    # M, H, Hkv, d, max_len, lowest length
    (16, 32, 16, 32, 32768, 24000),
    (8, 32, 16, 64, 32768, 28000),
    # Calls of fewer than 16 (sequence, KV head, head block) units: equal key
    # blocks, up to 512 splits per (m, h) and the 16-wave merge of the splits.
    (1, 8, 1, 128, 65536, 65536),   # 512 splits, the most a sequence can have
    (2, 8, 1, 128, 65536, 60000),
    (1, 32, 8, 128, 32768, 32768),
    (3, 20, 4, 64, 20000, 1),       # ragged: lengths from 1 up
    (1, 15, 15, 32, 9000, 9000),    # 15 units: the last count that takes equal blocks
    (1, 16, 16, 32, 9000, 9000),    # 16 units: the first-round decomposition again
    # 512 units (twice the CUs): the first round's largest block would exceed every
    # sequence and is clamped to the longest one left
    (16, 32, 32, 64, 2048, 1900),
]


def run_decode(q, kc, vc, lens, M, H, Hkv, d, max_len, scale):
    ws = __import__("torch").empty(taf.attn_decode_workspace_bytes(M, H, d, max_len) // 4,
                                   dtype=__import__("torch").float32, device=q.device)
    out = nan_like((M, H * d))
    taf.attn_decode_gqa_batched(q, kc, vc, lens, out, M, H, Hkv, d, max_len, scale, ws)
    return to_host(out)


@pytest.mark.parametrize("case", SMALL, ids=[f"M{c[0]}_H{c[1]}_Hkv{c[2]}_d{c[3]}_max{c[4]}" for c in SMALL])
def test_decode_small(case):
    M, H, Hkv, d, max_len, lens = case
    rng = np.random.default_rng(100 + M * 7 + H)
    if lens is None:
        lens = rng.integers(0, max_len + 1, size=M)
    lens = np.asarray(lens, np.int32)
    q = rng.standard_normal((M, H * d), dtype=np.float32)
    kc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    vc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    for m in range(M):  # rows past L_m are NaN: reading one would poison the output
        kc[m, :, lens[m]:] = np.nan
        vc[m, :, lens[m]:] = np.nan
    scale = wl.scale_for(d)
    note(f"decode M={M} H={H} Hkv={Hkv} d={d} max_len={max_len} lens={lens.tolist()}")
    got = run_decode(to_dev(q), to_dev(kc), to_dev(vc), lens.tolist(), M, H, Hkv, d, max_len, scale)
    want = oracle.default().decode(q, kc, vc, lens, M, H, Hkv, d, max_len, scale)
    assert_attn_close(got, want, f"decode {case}")
    for m in np.nonzero(lens == 0)[0]:
        assert np.all(got[m] == 0.0), "an empty sequence must give zeros"


@pytest.mark.parametrize("case", LONG, ids=[f"M{c[0]}_H{c[1]}_Hkv{c[2]}_d{c[3]}_max{c[4]}" for c in LONG])
def test_decode_long_contexts(case):
    M, H, Hkv, d, max_len, lo = case
    rng = np.random.default_rng(500 + d)
    lens = rng.integers(lo, max_len + 1, size=M).astype(np.int32)
    lens[0] = max_len
    q = rng.standard_normal((M, H * d), dtype=np.float32)
    kc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    vc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    scale = wl.scale_for(d)
    note(f"decode long M={M} H={H} Hkv={Hkv} d={d} max_len={max_len} sum(L)={int(lens.sum())}")
    got = run_decode(to_dev(q), to_dev(kc), to_dev(vc), lens.tolist(), M, H, Hkv, d, max_len, scale)
    want = oracle.default().decode(q, kc, vc, lens, M, H, Hkv, d, max_len, scale)
    assert_attn_close(got, want, f"decode long {case}")


def test_decode_large_scores():
    """Scores in the hundreds: the split-local maxima differ widely, the merge must rescale."""
    M, H, Hkv, d, max_len = 2, 8, 2, 128, 3000
    rng = np.random.default_rng(5)
    q = (rng.standard_normal((M, H * d), dtype=np.float32) * 8).astype(np.float32)
    kc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    vc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    kc[:, :, 2500] *= 4  # one dominant key late in the sequence
    lens = np.array([3000, 2600], np.int32)
    scale = wl.scale_for(d)
    note("decode large scores")
    got = run_decode(to_dev(q), to_dev(kc), to_dev(vc), lens.tolist(), M, H, Hkv, d, max_len, scale)
    want = oracle.default().decode(q, kc, vc, lens, M, H, Hkv, d, max_len, scale)
    assert_attn_close(got, want, "decode large scores")


def test_decode_equals_prefill_row_on_gpu():
    """GPU decode at step t over a GPU-appended cache equals row t of the GPU causal prefill."""
    import torch
    B, S, H, d, max_len = 1, 160, 4, 64, 192
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(3))
    scale = wl.scale_for(d)
    note("decode == prefill row")
    out = nan_like((B, S, H * d))
    taf.attn_prefill(to_dev(q), to_dev(k), to_dev(v), out, B, S, H, d, scale, True)
    pre = to_host(out)
    kc = torch.full((1, H, max_len, d), float("nan"), device=out.device)
    vc = torch.full((1, H, max_len, d), float("nan"), device=out.device)
    taf.kv_cache_scatter(to_dev(k), to_dev(v), kc, vc, [0], 1, S, H, d, max_len)
    want = oracle.default().prefill(q, k, v, B, S, H, d, scale, True)
    for t in (0, 1, 31, 32, 63, 64, 100, S - 1):
        got = run_decode(to_dev(np.ascontiguousarray(q[:, t])), kc, vc, [t + 1], 1, H, H, d, max_len, scale)
        assert np.max(np.abs(got[0] - pre[0, t])) <= 2e-5, f"decode vs prefill row {t}"
        assert_attn_close(got[0], want[0, t], f"decode step {t} vs oracle")


@pytest.mark.parametrize("cid", [4, 5])
def test_decode_step_full_size(cid):
    """Append at L_m - 1 then decode over L_m, on the full decode workloads."""
    import torch
    cfg = wl.DECODE[cid]
    inp = wl.decode_inputs(cfg)
    lens = inp["lens"]
    note(f"decode step full size {cfg.name} sum(L)={int(lens.sum())}")
    kc, vc = to_dev(inp["k_cache"]), to_dev(inp["v_cache"])
    taf.kv_cache_scatter(to_dev(inp["k_new"]), to_dev(inp["v_new"]), kc, vc, (lens - 1).tolist(),
                         cfg.M, 1, cfg.Hkv, cfg.d, cfg.max_len)
    got = run_decode(to_dev(inp["q"]), kc, vc, lens.tolist(), cfg.M, cfg.H, cfg.Hkv, cfg.d, cfg.max_len,
                     cfg.scale)
    del kc, vc
    torch.cuda.empty_cache()
    orc = oracle.default()
    k_host, v_host = inp["k_cache"], inp["v_cache"]
    orc.scatter(inp["k_new"], inp["v_new"], k_host, v_host, lens - 1, cfg.M, 1, cfg.Hkv, cfg.d, cfg.max_len)
    want = orc.decode(inp["q"], k_host, v_host, lens, cfg.M, cfg.H, cfg.Hkv, cfg.d, cfg.max_len, cfg.scale)
    assert_attn_close(got, want, f"{cfg.name} (all outputs)")


def _decode_on(stream, q, kc, vc, lens, M, H, Hkv, d, max_len, scale):
    import torch
    with torch.cuda.stream(stream):
        ws = torch.empty(taf.attn_decode_workspace_bytes(M, H, d, max_len) // 4, dtype=torch.float32,
                         device=q.device)
        out = torch.full((M, H * d), float("nan"), device=q.device)
        taf.attn_decode_gqa_batched(q, kc, vc, lens, out, M, H, Hkv, d, max_len, scale, ws, stream=stream)
    return out


def test_decode_deterministic_across_streams():
    """The same decode on 12 streams, twice each: identical bits every time (fixed merge order)."""
    import torch
    M, H, Hkv, d, max_len = 9, 16, 4, 128, 3000
    lens = [0, 1, 127, 128, 129, 700, 2999, 3000, 1500]
    rng = np.random.default_rng(808)
    q = to_dev(rng.standard_normal((M, H * d), dtype=np.float32))
    kc = to_dev(rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32))
    vc = to_dev(rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32))
    scale = wl.scale_for(d)
    note("decode determinism: 12 streams x 2 calls")
    streams = [torch.cuda.Stream() for _ in range(12)]
    outs = [_decode_on(s, q, kc, vc, lens, M, H, Hkv, d, max_len, scale) for s in streams for _ in range(2)]
    torch.cuda.synchronize()
    host = [bits(to_host(o)) for o in outs]
    for i, h in enumerate(host[1:], 1):
        assert np.array_equal(h, host[0]), f"call {i} (stream {i // 2}) differs from call 0"
    want = oracle.default().decode(to_host(q), to_host(kc), to_host(vc), np.asarray(lens, np.int32), M, H, Hkv,
                                   d, max_len, scale)
    assert_attn_close(to_host(outs[0]), want, "decode on side streams vs oracle")


def test_decode_many_kv_heads():
    """32 sequences x 1024 KV heads (32768 head groups, 4-row caches)."""
    M, H, Hkv, d, max_len = 32, 1024, 1024, 32, 4
    rng = np.random.default_rng(809)
    lens = rng.integers(0, max_len + 1, size=M).astype(np.int32)
    q = rng.standard_normal((M, H * d), dtype=np.float32)
    kc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    vc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    scale = wl.scale_for(d)
    note("decode with 32768 head groups")
    got = run_decode(to_dev(q), to_dev(kc), to_dev(vc), lens.tolist(), M, H, Hkv, d, max_len, scale)
    want = oracle.default().decode(q, kc, vc, lens, M, H, Hkv, d, max_len, scale)
    assert_attn_close(got, want, "decode 32768 groups")


def test_decode_graph_replays_match_eager():
    """A decode captured into a HIP graph replays to the eager result, bit for bit, over several
    replays with new queries and eager decodes in between."""
    import torch
    M, H, Hkv, d, max_len = 6, 32, 8, 128, 2048
    lens = [5, 2048, 0, 1000, 129, 64]
    rng = np.random.default_rng(810)
    kc = to_dev(rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32))
    vc = to_dev(rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32))
    scale = wl.scale_for(d)
    note("decode graph capture and replays")
    q_static = to_dev(rng.standard_normal((M, H * d), dtype=np.float32))
    ws = torch.empty(taf.attn_decode_workspace_bytes(M, H, d, max_len) // 4, dtype=torch.float32, device="cuda:0")
    out_static = torch.zeros((M, H * d), device="cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream (first-call host queries)
        taf.attn_decode_gqa_batched(q_static, kc, vc, lens, out_static, M, H, Hkv, d, max_len, scale, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        taf.attn_decode_gqa_batched(q_static, kc, vc, lens, out_static, M, H, Hkv, d, max_len, scale, ws)
    for rep in range(4):
        q_new = to_dev(rng.standard_normal((M, H * d), dtype=np.float32))
        q_static.copy_(q_new)
        graph.replay()
        torch.cuda.synchronize()
        got = to_host(out_static)
        eager = run_decode(q_new, kc, vc, lens, M, H, Hkv, d, max_len, scale)
        assert np.array_equal(bits(got), bits(eager)), f"replay {rep} differs from the eager decode"
