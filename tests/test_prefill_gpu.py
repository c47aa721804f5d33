"""Prefill (full-sequence attention) on the GPU against the fp64 oracle.

Small cases span one to many 128-query and 32-key tiles with ragged tails
(S = 1, 31, 33, 127, 129, 200, 500, 1500), every head_dim, batch > 1, head
counts on and off the XCD-grouping path (B*H a multiple of 8 or not), causal
and not, non-default scales and large scores.  Outputs start as NaN so an
unwritten element fails.  The full-size cases are the three prefill
workloads, every output element compared with the C oracle.  The larger
decomposition cases are compared whole against the numpy formulation of the
oracle (oracle/brute.py, pinned to the C oracle); only a single-head
S = 32640 case, whose score matrix alone would take 8.5 GB in fp64, is
checked on sampled rows.
Every work decomposition the launcher picks has cases of its own (the small
and mid-size ones on 16-query waves, causal and not, at every head_dim), and
each is also captured into a HIP graph whose replays must match eager calls
bit for bit.
"""
import numpy as np
import pytest

import oracle
import transformer_attention_flash_amd as taf
from transformer_attention_flash_amd import workloads as wl
from gpu_common import assert_attn_close, nan_like, note, to_dev, to_host
from oracle import brute

pytestmark = pytest.mark.gpu

SMALL = [
    # B, S, H, d
    (1, 1, 1, 32),
    (1, 31, 2, 32),
    (2, 33, 3, 64),
    (1, 127, 1, 128),
    (1, 128, 2, 128),
    (1, 129, 1, 128),
    (3, 200, 2, 64),
    (2, 300, 4, 128),
    (1, 500, 8, 128),
    (1, 257, 16, 32),
]


def run_prefill(q, k, v, B, S, H, d, scale, causal):
    out = nan_like((B, S, H * d))
    taf.attn_prefill(to_dev(q), to_dev(k), to_dev(v), out, B, S, H, d, scale, causal)
    return to_host(out)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}_S{c[1]}_H{c[2]}_d{c[3]}" for c in SMALL])
def test_prefill_small(case, causal):
    B, S, H, d = case
    rng = np.random.default_rng(1 + S * 13 + H + d)
    q, k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(3))
    scale = wl.scale_for(d)
    note(f"prefill B={B} S={S} H={H} d={d} causal={causal}")
    got = run_prefill(q, k, v, B, S, H, d, scale, causal)
    want = oracle.default().prefill(q, k, v, B, S, H, d, scale, causal)
    assert_attn_close(got, want, f"prefill {case} causal={causal}")


DECOMPOSITIONS = [
    # B, S, H, d -> which work decomposition the launcher picks (B*H*ceil(S/128) and
    # B*H*ceil(S/256) decide): small problems, and causal ones below 1024 four-wave
    # workgroups, run 16-query waves in 4 key groups; mid-size ones use 4 waves; large
    # ones 8 waves (d >= 64).
    (1, 1500, 8, 64),     # 16-query waves, 48 queries per workgroup (the Whisper-base shape)
    (1, 700, 4, 128),     # 16-query waves on 16-key tiles, ragged tail
    (3, 70, 5, 32),       # 16-query waves with fewer key tiles than groups
    (2, 1100, 16, 64),    # 288 workgroups: four waves, causal 16-query waves
    (2, 1000, 64, 128),   # eight waves, 64-key tiles; the last tile's second sub-tile partly past S
    (2, 1050, 64, 128),   # eight waves; the last tile's second 32-key sub-tile wholly past S
    (2, 1000, 64, 64),    # eight waves, 64-key tiles at d = 64; second sub-tile partly past S
    (2, 1050, 64, 64),    # the same with the last tile's second sub-tile wholly past S
]


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("case", DECOMPOSITIONS, ids=[f"B{c[0]}_S{c[1]}_H{c[2]}_d{c[3]}" for c in DECOMPOSITIONS])
def test_prefill_decompositions(case, causal):
    B, S, H, d = case
    rng = np.random.default_rng(5 + S + H + d)
    q, k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(3))
    scale = wl.scale_for(d)
    note(f"prefill decomposition B={B} S={S} H={H} d={d} causal={causal}")
    got = run_prefill(q, k, v, B, S, H, d, scale, causal)
    want = brute.prefill(q, k, v, B, S, H, d, scale, causal)
    assert_attn_close(got, want, f"prefill decomposition {case} causal={causal}")


SMALL_PROBLEMS = [
    # B, S, H, d: non-causal problems with B*H*ceil(S/128) < 256 run the 16-query-wave
    # kernel; the launcher picks 16, 32, 48 or 64 queries per workgroup (QW = 1..4)
    # so that the most loaded CU has the fewest queries (with 256 CUs: noted per case).
    # At d = 128 a key tile is one 16-key MFMA tile and QW 4 reads K chunk by chunk.
    (1, 1, 3, 32),       # QW 1; one key, three of the four key groups empty
    (1, 17, 2, 64),      # QW 1; one ragged key tile
    (2, 33, 3, 32),      # QW 1; two key tiles
    (1, 100, 5, 64),     # QW 1; four key tiles, ragged
    (1, 600, 8, 64),     # QW 2
    (2, 1000, 8, 64),    # QW 4
    (1, 1500, 8, 32),    # QW 3 (the encoder shape at d = 32)
    (3, 250, 2, 32),     # QW 1
    (1, 1, 3, 128),      # QW 1; one key
    (2, 100, 3, 128),    # QW 1; seven key tiles, ragged
    (1, 600, 8, 128),    # QW 2
    (1, 1500, 8, 128),   # QW 3
    (1, 1024, 16, 128),  # QW 4
]


@pytest.mark.parametrize("case", SMALL_PROBLEMS, ids=[f"B{c[0]}_S{c[1]}_H{c[2]}_d{c[3]}" for c in SMALL_PROBLEMS])
def test_prefill_small_problems(case):
    B, S, H, d = case
    rng = np.random.default_rng(900 + S + H + d)
    q, k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(3))
    scale = wl.scale_for(d)
    note(f"prefill small problem B={B} S={S} H={H} d={d}")
    got = run_prefill(q, k, v, B, S, H, d, scale, False)
    want = oracle.default().prefill(q, k, v, B, S, H, d, scale, False)
    assert_attn_close(got, want, f"prefill small problem {case}")


SMALL_CAUSAL = [
    # B, S, H, d, rows checked (None: all): causal small problems on the 16-query-wave
    # kernel; the launcher simulates the heavy-first dispatch to pick QW (with 256 CUs:
    # noted per case)
    (1, 17, 2, 64, None),      # QW 1, one ragged key tile
    (2, 33, 3, 32, None),      # QW 1
    (1, 1500, 8, 32, None),    # QW 1
    (1, 1500, 8, 64, None),    # QW 2
    (1, 3000, 6, 64, None),    # QW 3
    (1, 32640, 1, 64, "sampled"),  # QW 4 (255 query tiles of 128 on one head)
    (1, 17, 2, 128, None),     # QW 1
    (1, 512, 32, 128, None),   # QW 2
    (2, 700, 8, 128, None),    # QW 2
]


@pytest.mark.parametrize("case", SMALL_CAUSAL, ids=[f"B{c[0]}_S{c[1]}_H{c[2]}_d{c[3]}" for c in SMALL_CAUSAL])
def test_prefill_small_problems_causal(case):
    B, S, H, d, rows = case
    rng = np.random.default_rng(950 + S + H + d)
    q, k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(3))
    scale = wl.scale_for(d)
    note(f"prefill small causal problem B={B} S={S} H={H} d={d}")
    got = run_prefill(q, k, v, B, S, H, d, scale, True)
    assert np.all(np.isfinite(got)), "every output element is written"
    if rows is None:
        assert_attn_close(got, brute.prefill(q, k, v, B, S, H, d, scale, True), f"prefill small causal {case}")
        return
    # One head of 32640 queries: its fp64 score matrix would not fit a whole-output check.
    picks = sorted({0, 1, 15, 16, 17, 31, 32, 47, 48, 63, 64, S // 3, S // 2, S - 49, S - 48, S - 17, S - 16, S - 1}
                   | set(rng.integers(0, S, 16).tolist()))
    sel = np.array([(b, i, h) for b in range(B) for i in picks for h in range(H)], np.int64)
    want = oracle.default().prefill_rows(q, k, v, sel, B, S, H, d, scale, True)
    got_sel = np.stack([got[b, i, h * d:(h + 1) * d] for b, i, h in sel])
    assert_attn_close(got_sel, want, f"prefill small causal {case} (sampled rows)")


CAUSAL_MID = [
    # B, S, H, d: causal problems between the small and the eight-wave ones
    (1, 4096, 8, 128),    # 256 four-wave workgroups: 16-query waves
    (1, 2000, 12, 64),    # 192 / 96: 16-query waves (eight-wave needs 512)
    (1, 2048, 32, 32),    # 512: 16-query waves
    (2, 2048, 32, 32),    # 1024 at d = 32: four waves
]


@pytest.mark.parametrize("case", CAUSAL_MID, ids=[f"B{c[0]}_S{c[1]}_H{c[2]}_d{c[3]}" for c in CAUSAL_MID])
def test_prefill_causal_mid_size(case):
    B, S, H, d = case
    rng = np.random.default_rng(970 + S + H + d)
    q, k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(3))
    scale = wl.scale_for(d)
    note(f"prefill causal mid-size B={B} S={S} H={H} d={d}")
    got = run_prefill(q, k, v, B, S, H, d, scale, True)
    assert_attn_close(got, brute.prefill(q, k, v, B, S, H, d, scale, True), f"prefill causal mid-size {case}")


def test_prefill_small_problem_large_scores():
    """Scores spanning a wide range (q scaled by 8, a negative scale) on the 16-query-wave kernel."""
    B, S, H, d = 1, 777, 4, 64
    rng = np.random.default_rng(901)
    q = (rng.standard_normal((B, S, H * d), dtype=np.float32) * 8).astype(np.float32)
    k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(2))
    note("prefill small problem, large scores")
    for scale in (0.25, -0.2):
        got = run_prefill(q, k, v, B, S, H, d, scale, False)
        want = oracle.default().prefill(q, k, v, B, S, H, d, scale, False)
        assert_attn_close(got, want, f"prefill small problem large scores scale={scale}")


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_prefill_large_scores_and_custom_scale(causal):
    B, S, H, d = 1, 333, 2, 128
    rng = np.random.default_rng(3)
    q = (rng.standard_normal((B, S, H * d), dtype=np.float32) * 6).astype(np.float32)
    k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(2))
    scale = 0.3
    note(f"prefill large scores causal={causal}")
    got = run_prefill(q, k, v, B, S, H, d, scale, causal)
    want = oracle.default().prefill(q, k, v, B, S, H, d, scale, causal)
    assert_attn_close(got, want, "prefill large scores")


@pytest.mark.parametrize("cid", [1, 2])
def test_prefill_full_size_noncausal(cid):
    cfg = wl.PREFILL[cid]
    q, k, v = wl.prefill_inputs(cfg)
    note(f"prefill full size {cfg.name}")
    got = run_prefill(q, k, v, cfg.B, cfg.S, cfg.H, cfg.d, cfg.scale, cfg.causal)
    want = oracle.default().prefill(q, k, v, cfg.B, cfg.S, cfg.H, cfg.d, cfg.scale, cfg.causal)
    assert_attn_close(got, want, cfg.name)


def test_prefill_full_size_causal():
    """B=4, S=2048, H=32, d=128, causal: all 262,144 output rows against the C oracle."""
    cfg = wl.PREFILL[3]
    q, k, v = wl.prefill_inputs(cfg)
    note(f"prefill full size {cfg.name}")
    got = run_prefill(q, k, v, cfg.B, cfg.S, cfg.H, cfg.d, cfg.scale, cfg.causal)
    want = oracle.default().prefill(q, k, v, cfg.B, cfg.S, cfg.H, cfg.d, cfg.scale, True)
    assert_attn_close(got, want, f"{cfg.name} (all outputs)")


GRAPH_CASES = [
    # B, S, H, d, causal: one capture per work decomposition
    (1, 300, 4, 64, True),      # 16-query waves, causal
    (1, 700, 4, 128, False),    # 16-query waves on 16-key tiles
    (2, 1024, 32, 128, True),   # eight-wave workgroups (512 of them)
]


@pytest.mark.parametrize("case", GRAPH_CASES, ids=[f"B{c[0]}_S{c[1]}_H{c[2]}_d{c[3]}_c{int(c[4])}" for c in GRAPH_CASES])
def test_prefill_graph_replays_match_eager(case):
    """A prefill captured into a HIP graph replays to the eager result, bit for bit, over several
    replays with new inputs and eager prefills in between."""
    import torch
    from gpu_common import bits
    B, S, H, d, causal = case
    rng = np.random.default_rng(880 + S + H)
    scale = wl.scale_for(d)
    shape = (B, S, H * d)
    q_s, k_s, v_s = (to_dev(rng.standard_normal(shape, dtype=np.float32)) for _ in range(3))
    out_s = torch.zeros(shape, device="cuda:0")
    note(f"prefill graph capture B={B} S={S} H={H} d={d} causal={causal}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream (first-call host queries)
        taf.attn_prefill(q_s, k_s, v_s, out_s, B, S, H, d, scale, causal)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        taf.attn_prefill(q_s, k_s, v_s, out_s, B, S, H, d, scale, causal)
    for rep in range(3):
        q, k, v = (rng.standard_normal(shape, dtype=np.float32) for _ in range(3))
        for dst, src in ((q_s, q), (k_s, k), (v_s, v)):
            dst.copy_(to_dev(src))
        graph.replay()
        torch.cuda.synchronize()
        got = to_host(out_s)
        eager = run_prefill(q, k, v, B, S, H, d, scale, causal)
        assert np.array_equal(bits(got), bits(eager)), f"replay {rep} differs from the eager prefill"
