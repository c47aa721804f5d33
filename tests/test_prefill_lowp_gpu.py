"""Reduced-precision prefill (16-bit MFMA operands) on the GPU against the oracle.

The oracle computes the exact (fp64) attention of q, k and v rounded to the
16-bit format.  The kernel additionally rounds the probabilities to that
format for the P.V product while normalising with the f32 sum, so an output
element may move by up to u * max|v| (u = 2^-11 for binary16, 2^-8 for
bfloat16) on top of f32 rounding; the contract asserted here is

    max |gpu - oracle_lowp| <= 2 u max|v_rounded| + 1e-5.

Cases: ragged S across 32/64-key and 128/256-query tiles, every head_dim,
batch > 1, causal and not, the three work decompositions (4 and 8 waves per
workgroup, and for small problems at d <= 64 key tiles split over 4 groups of
2 query waves, at d = 128 over 2 groups of 4, causal too), the two causal
eight-wave schedules (pairs of query tiles, one of them walking its keys
downwards, and single tiles heaviest first), a non-default and a
negative scale with
large scores, both formats, and the three prefill workloads at full size,
every output compared.  Large cases are compared whole against the numpy
formulation of the oracle (oracle/brute.py, pinned to the C oracle) on the
inputs rounded by the oracle; only the single S = 32768 case is sampled.  The
error against the exact f32-input attention is printed for reference (it is
dominated by the rounding of q and k, not part of the contract).
"""
import numpy as np
import pytest

import oracle
import transformer_attention_flash_amd as taf
from transformer_attention_flash_amd import workloads as wl
from gpu_common import nan_like, note, to_dev, to_host
from oracle import brute

pytestmark = pytest.mark.gpu

FORMATS = {"fp16": (taf.ATTN_PREC_FP16, 2.0 ** -11), "bf16": (taf.ATTN_PREC_BF16, 2.0 ** -8)}

SMALL = [
    # B, S, H, d
    (1, 1, 1, 32),
    (1, 31, 2, 32),
    (2, 33, 3, 64),
    (1, 127, 1, 128),
    (1, 129, 2, 128),
    (3, 200, 2, 64),
    (2, 300, 4, 128),
    (1, 500, 8, 128),
    (1, 257, 16, 32),
]


def run_lowp(q, k, v, B, S, H, d, scale, causal, prec):
    out = nan_like((B, S, H * d))
    taf.attn_prefill_lowp(to_dev(q), to_dev(k), to_dev(v), out, B, S, H, d, scale, causal, prec)
    return to_host(out)


def check(got, want, v_rounded, u, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    tol = 2.0 * u * float(np.max(np.abs(v_rounded))) + 1e-5
    err = float(np.max(np.abs(got - want)))
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.3e}"
    return err


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}_S{c[1]}_H{c[2]}_d{c[3]}" for c in SMALL])
def test_prefill_lowp_small(case, causal, fmt):
    B, S, H, d = case
    prec, u = FORMATS[fmt]
    rng = np.random.default_rng(11 + S * 13 + H + d)
    q, k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(3))
    scale = wl.scale_for(d)
    note(f"prefill_lowp {fmt} B={B} S={S} H={H} d={d} causal={causal}")
    got = run_lowp(q, k, v, B, S, H, d, scale, causal, prec)
    orc = oracle.default()
    want = orc.prefill_lowp(q, k, v, B, S, H, d, scale, causal, prec)
    check(got, want, orc.round16(v, prec), u, f"{fmt} {case} causal={causal}")


SMALL_CAUSAL = [
    # B, S, H, d: causal problems with B*H*ceil(S/128) < 256 split each workgroup's
    # visible key tiles over groups of query waves (d <= 64: 4 groups of 2 waves,
    # 64 queries per workgroup; d = 128: 2 groups of 4 waves, 128 queries)
    (1, 1500, 8, 64),
    (2, 1000, 8, 32),
    (1, 2048, 8, 128),
]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("case", SMALL_CAUSAL, ids=[f"B{c[0]}_S{c[1]}_H{c[2]}_d{c[3]}" for c in SMALL_CAUSAL])
def test_prefill_lowp_small_causal_key_groups(case, fmt):
    B, S, H, d = case
    prec, u = FORMATS[fmt]
    rng = np.random.default_rng(23 + S + H + d)
    q, k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(3))
    scale = wl.scale_for(d)
    note(f"prefill_lowp {fmt} causal key groups B={B} S={S} H={H} d={d}")
    got = run_lowp(q, k, v, B, S, H, d, scale, True, prec)
    orc = oracle.default()
    want = orc.prefill_lowp(q, k, v, B, S, H, d, scale, True, prec)
    check(got, want, orc.round16(v, prec), u, f"{fmt} {case} causal key groups")


EIGHT_WAVE = [
    # B, S, H, d: B*H*ceil(S/256) >= 512 runs the 256-query, 64-key-tile path; ragged S.
    # Causal, the first three run as pairs of query tiles (T-1-j upwards, then j
    # downwards from its diagonal); the last, with 3 query tiles per (b, h), as
    # single tiles heaviest first.
    (2, 1000, 64, 128),
    (4, 777, 32, 64),
    (16, 300, 32, 32),
    (4, 600, 64, 32),
    # B*H not a multiple of 8 (no XCD grouping); causal, 64 pairs of 128 query tiles per head
    (1, 32768, 4, 32),
]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
@pytest.mark.parametrize("case", EIGHT_WAVE, ids=[f"B{c[0]}_S{c[1]}_H{c[2]}_d{c[3]}" for c in EIGHT_WAVE])
def test_prefill_lowp_eight_wave_path(case, causal, fmt):
    B, S, H, d = case
    prec, u = FORMATS[fmt]
    rng = np.random.default_rng(17 + S + H + d)
    q, k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(3))
    scale = wl.scale_for(d)
    note(f"prefill_lowp {fmt} eight-wave B={B} S={S} H={H} d={d} causal={causal}")
    got = run_lowp(q, k, v, B, S, H, d, scale, causal, prec)
    assert np.all(np.isfinite(got)), "every output element is written"
    orc = oracle.default()
    rq, rk, rv = (orc.round16(x, prec) for x in (q, k, v))
    if S * S <= 2 ** 24:
        # The attention of the rounded inputs (pinned on the CPU), every output.
        check(got, brute.prefill(rq, rk, rv, B, S, H, d, scale, causal), rv, u,
              f"{fmt} eight-wave {case} causal={causal}")
        return
    # S = 32768: a head's fp64 score matrix would not fit a whole-output check.
    rows = sorted({0, 1, 31, 32, 63, 64, 127, 128, 255, 256, S // 2, S - 65, S - 64, S - 1})
    sel = np.array([(b, i, h) for b in range(B) for i in rows for h in range(0, H, max(1, H // 8))], np.int64)
    want = orc.prefill_rows(rq, rk, rv, sel, B, S, H, d, scale, causal)
    got_sel = np.stack([got[b, i, h * d:(h + 1) * d] for b, i, h in sel])
    check(got_sel, want, rv, u, f"{fmt} eight-wave {case} causal={causal} (sampled rows)")


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_prefill_lowp_large_scores_and_custom_scale(fmt):
    B, S, H, d = 1, 333, 2, 128
    prec, u = FORMATS[fmt]
    rng = np.random.default_rng(4)
    q = (rng.standard_normal((B, S, H * d), dtype=np.float32) * 6).astype(np.float32)
    k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(2))
    note(f"prefill_lowp {fmt} large scores")
    orc = oracle.default()
    for causal in (False, True):
        for scale in (0.3, -0.2):
            got = run_lowp(q, k, v, B, S, H, d, scale, causal, prec)
            want = orc.prefill_lowp(q, k, v, B, S, H, d, scale, causal, prec)
            check(got, want, orc.round16(v, prec), u, f"{fmt} large scores scale={scale} causal={causal}")


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("cid", [1, 2])
def test_prefill_lowp_full_size_noncausal(cid, fmt):
    cfg = wl.PREFILL[cid]
    prec, u = FORMATS[fmt]
    q, k, v = wl.prefill_inputs(cfg)
    note(f"prefill_lowp {fmt} full size {cfg.name}")
    got = run_lowp(q, k, v, cfg.B, cfg.S, cfg.H, cfg.d, cfg.scale, cfg.causal, prec)
    orc = oracle.default()
    want = orc.prefill_lowp(q, k, v, cfg.B, cfg.S, cfg.H, cfg.d, cfg.scale, cfg.causal, prec)
    err = check(got, want, orc.round16(v, prec), u, f"{fmt} {cfg.name}")
    exact = orc.prefill(q, k, v, cfg.B, cfg.S, cfg.H, cfg.d, cfg.scale, cfg.causal)
    note(f"  {fmt} {cfg.name}: err vs rounded-input oracle {err:.2e}, "
         f"vs f32-input attention {float(np.max(np.abs(got - exact))):.2e}")


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_prefill_lowp_full_size_causal(fmt):
    """B=4, S=2048, H=32, d=128, causal: every output against the attention of the rounded inputs."""
    cfg = wl.PREFILL[3]
    prec, u = FORMATS[fmt]
    q, k, v = wl.prefill_inputs(cfg)
    note(f"prefill_lowp {fmt} full size {cfg.name}")
    got = run_lowp(q, k, v, cfg.B, cfg.S, cfg.H, cfg.d, cfg.scale, cfg.causal, prec)
    orc = oracle.default()
    rq, rk, rv = (orc.round16(x, prec) for x in (q, k, v))
    want = brute.prefill(rq, rk, rv, cfg.B, cfg.S, cfg.H, cfg.d, cfg.scale, True)
    check(got, want, rv, u, f"{fmt} {cfg.name} (all outputs)")


LOWP_GRAPH_CASES = [
    # B, S, H, d: causal eight-wave schedules (pairs of query tiles; single tiles)
    (16, 300, 32, 32),
    (4, 600, 64, 32),
]


@pytest.mark.parametrize("case", LOWP_GRAPH_CASES, ids=[f"B{c[0]}_S{c[1]}_H{c[2]}_d{c[3]}" for c in LOWP_GRAPH_CASES])
def test_prefill_lowp_graph_replays_match_eager(case):
    """A causal reduced-precision prefill captured into a HIP graph replays to the eager result,
    bit for bit, over several replays with new inputs and eager prefills in between."""
    import torch
    from gpu_common import bits
    B, S, H, d = case
    prec, _ = FORMATS["bf16"]
    rng = np.random.default_rng(990 + S + H)
    scale = wl.scale_for(d)
    shape = (B, S, H * d)
    q_s, k_s, v_s = (to_dev(rng.standard_normal(shape, dtype=np.float32)) for _ in range(3))
    out_s = torch.zeros(shape, device="cuda:0")
    note(f"prefill_lowp graph capture B={B} S={S} H={H} d={d}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on the capture stream (first-call host queries)
        taf.attn_prefill_lowp(q_s, k_s, v_s, out_s, B, S, H, d, scale, True, prec)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        taf.attn_prefill_lowp(q_s, k_s, v_s, out_s, B, S, H, d, scale, True, prec)
    for rep in range(3):
        q, k, v = (rng.standard_normal(shape, dtype=np.float32) for _ in range(3))
        for dst, src in ((q_s, q), (k_s, k), (v_s, v)):
            dst.copy_(to_dev(src))
        graph.replay()
        torch.cuda.synchronize()
        got = to_host(out_s)
        eager = run_lowp(q, k, v, B, S, H, d, scale, True, prec)
        assert np.array_equal(bits(got), bits(eager)), f"replay {rep} differs from the eager prefill"
