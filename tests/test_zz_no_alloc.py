"""The no-allocation decode (attn_decode_gqa_batched_noalloc) against the decode with a
caller workspace, through the C ABI.

Two calls in a row on one stream share the library's scratch array; the second is
smaller than the first, so stale partials of the first would show if the second read
any slot it did not write.  Each output must equal the workspace decode's bit for bit
(the same kernels on the same inputs) and meet the oracle tolerance.  A HIP graph that
captures the call (the reason it takes no workspace) must replay to the eager result.
"""
import numpy as np
import pytest

import oracle
import transformer_attention_flash_amd as taf
from transformer_attention_flash_amd import workloads as wl
from gpu_common import assert_attn_close, bits, nan_like, note, to_dev, to_host

pytestmark = pytest.mark.gpu

CASES = [
    # M, H, Hkv, d, max_len: the second call is smaller in every dimension
    (16, 32, 8, 128, 4096),
    (3, 8, 2, 64, 300),
]


def _inputs(seed, M, H, Hkv, d, max_len):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len + 1, size=M).astype(np.int32)
    lens[0] = max_len
    q = rng.standard_normal((M, H * d), dtype=np.float32)
    kc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    vc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    return lens, q, kc, vc


def test_noalloc_decode_matches_workspace_decode_twice():
    import torch
    dev_in, outs = [], []
    for i, (M, H, Hkv, d, max_len) in enumerate(CASES):
        lens, q, kc, vc = _inputs(4400 + i, M, H, Hkv, d, max_len)
        dev_in.append((lens, q, kc, vc, to_dev(q), to_dev(kc), to_dev(vc)))
    note("decode_noalloc: two calls in a row, the second smaller")
    for (M, H, Hkv, d, max_len), (lens, _, _, _, qd, kd, vd) in zip(CASES, dev_in):
        out = nan_like((M, H * d))
        taf.attn_decode_gqa_batched_noalloc(qd, kd, vd, lens.tolist(), out, M, H, Hkv, d, max_len, wl.scale_for(d))
        outs.append(out)
    torch.cuda.synchronize()
    orc = oracle.default()
    for (M, H, Hkv, d, max_len), (lens, q, kc, vc, qd, kd, vd), out in zip(CASES, dev_in, outs):
        ws = torch.empty(taf.attn_decode_workspace_bytes(M, H, d, max_len) // 4, device="cuda:0")
        ref = nan_like((M, H * d))
        taf.attn_decode_gqa_batched(qd, kd, vd, lens.tolist(), ref, M, H, Hkv, d, max_len, wl.scale_for(d), ws)
        got = to_host(out)
        assert np.array_equal(bits(got), bits(to_host(ref))), f"M={M} H={H}: differs from the workspace decode"
        want = orc.decode(q, kc, vc, lens, M, H, Hkv, d, max_len, wl.scale_for(d))
        assert_attn_close(got, want, f"decode_noalloc M={M} H={H} Hkv={Hkv} d={d}")


def test_noalloc_decode_graph_replays_match_eager():
    import torch
    M, H, Hkv, d, max_len = 6, 32, 8, 128, 2048
    lens = [5, 2048, 0, 1000, 129, 64]
    rng = np.random.default_rng(4410)
    kc = to_dev(rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32))
    vc = to_dev(rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32))
    scale = wl.scale_for(d)
    q_static = to_dev(rng.standard_normal((M, H * d), dtype=np.float32))
    out_static = torch.zeros((M, H * d), device="cuda:0")
    note("decode_noalloc: graph capture and replays")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # first call on the device: the scratch address lookup
        taf.attn_decode_gqa_batched_noalloc(q_static, kc, vc, lens, out_static, M, H, Hkv, d, max_len, scale)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        taf.attn_decode_gqa_batched_noalloc(q_static, kc, vc, lens, out_static, M, H, Hkv, d, max_len, scale)
    ws = torch.empty(taf.attn_decode_workspace_bytes(M, H, d, max_len) // 4, device="cuda:0")
    for rep in range(3):
        q_new = to_dev(rng.standard_normal((M, H * d), dtype=np.float32))
        q_static.copy_(q_new)
        graph.replay()
        torch.cuda.synchronize()
        got = to_host(out_static)
        eager = nan_like((M, H * d))
        taf.attn_decode_gqa_batched(q_new, kc, vc, lens, eager, M, H, Hkv, d, max_len, scale, ws)
        assert np.array_equal(bits(got), bits(to_host(eager))), f"replay {rep} differs from the eager decode"


def test_noalloc_decode_at_the_scratch_limit():
    """The largest decode the built-in scratch takes: 32 sequences x 63 heads (7 KV heads) at
    d 128 and max_len 8192 need 2016 x 64 split slots of 130 floats = 67 092 480 bytes of the
    67 108 864, every sequence at a different length up to the full cache.  Equal bit for bit
    to the workspace decode of the same inputs (whose parity with the oracle at full size is
    covered by the decode tests), on a call after a smaller one."""
    import torch
    M, H, Hkv, d, max_len = 32, 63, 7, 128, 8192
    assert taf.attn_decode_workspace_bytes(M, H, d, max_len) <= taf.ATTN_DECODE_SCRATCH_BYTES
    assert taf.attn_decode_workspace_bytes(M, H + 1, d, max_len) > taf.ATTN_DECODE_SCRATCH_BYTES
    g = torch.Generator(device="cuda:0")
    g.manual_seed(4420)
    kc = torch.randn((M, Hkv, max_len, d), generator=g, device="cuda:0")
    vc = torch.randn((M, Hkv, max_len, d), generator=g, device="cuda:0")
    q = torch.randn((M, H * d), generator=g, device="cuda:0")
    lens = np.random.default_rng(4421).integers(1, max_len + 1, size=M).astype(np.int32)
    lens[0], lens[1] = max_len, 1
    scale = wl.scale_for(d)
    note("decode_noalloc at the scratch limit: M=32 H=63 Hkv=7 d=128 max_len=8192")
    small = nan_like((2, 8 * 64))
    taf.attn_decode_gqa_batched_noalloc(q[:2, :8 * 64].contiguous(), kc[:2, :1, :64, :64].contiguous(),
                                        vc[:2, :1, :64, :64].contiguous(), [64, 3], small, 2, 8, 1, 64, 64, scale)
    out = nan_like((M, H * d))
    taf.attn_decode_gqa_batched_noalloc(q, kc, vc, lens.tolist(), out, M, H, Hkv, d, max_len, scale)
    ws = torch.empty(taf.attn_decode_workspace_bytes(M, H, d, max_len) // 4, device="cuda:0")
    ref = nan_like((M, H * d))
    taf.attn_decode_gqa_batched(q, kc, vc, lens.tolist(), ref, M, H, Hkv, d, max_len, scale, ws)
    got = to_host(out)
    assert np.all(np.isfinite(got))
    assert np.array_equal(bits(got), bits(to_host(ref))), "differs from the workspace decode"
