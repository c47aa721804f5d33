"""Chunked prefill behind a KV cache with the rotary embedding fused in
(attn_prefill_cached_rope), on the GPU, against the oracle.

The oracle (``prefill_cached_rope``) turns query and new key row r of
sequence m to position cache_lens[m] + r with its own fp64 rotation, hands
them over as f32 and runs its chunked prefill; cache rows below the chunk are
rotated keys the oracle appended itself.  Both outputs are checked: the
attention (abs 1e-4, normwise rel 1e-3) and the appended caches (rotated key
dims within ROPE_ABS_TOL of the oracle's rotation, values and untouched rows
bit for bit).  Cases take each of the launcher's kernels (16-query waves,
four and eight waves), partial and full rotary widths, bases 10^4 and 10^6,
ragged cached lengths and GQA groups; a width of 0 equals the plain entry
point bit for bit; and at full size the second half of the causal prefill
workload follows its first half (M=4, H=32, d=128, 2048 cached + 2048 new),
every output compared against the numpy formulation of the oracle
(oracle/brute.py, pinned to the C oracle).
"""
import numpy as np
import pytest

import oracle
import transformer_attention_flash_amd as taf
from transformer_attention_flash_amd import workloads as wl
from gpu_common import assert_attn_close, bits, nan_like, note, to_dev, to_host
from oracle import brute

pytestmark = pytest.mark.gpu

ROPE_ABS_TOL = 1e-5  # a rotated f32 element against the exact rotation (see test_rope_gpu.py)

CASES = [
    # M, n_new, H, Hkv, d, max_len, lens (None = random), rotary_ndims, theta
    (1, 1, 1, 1, 32, 1, [0], 32, 1e4),
    (2, 31, 4, 4, 64, 100, [0, 69], 64, 1e4),
    (3, 129, 8, 2, 128, 300, [0, 17, 171], 128, 1e6),
    (2, 200, 16, 2, 64, 700, None, 16, 1e4),
    (4, 64, 6, 3, 128, 512, None, 32, 1e6),
    (5, 40, 8, 8, 128, 200, [160, 0, 33, 128, 100], 64, 500.0),
    # the launcher's kernels: 16-query waves (small and mid-size), four waves (P > n)
    (2, 1100, 16, 4, 64, 1600, [100, 480], 64, 1e4),
    (2, 300, 64, 8, 128, 1300, [600, 950], 128, 1e6),
    (1, 2100, 48, 16, 32, 2200, [64], 24, 1e4),
    # eight waves (512 workgroups, 64-key tiles), ragged cached lengths, half rotary width
    (2, 1000, 64, 8, 128, 2100, [600, 1030], 64, 1e4),
    (2, 1000, 64, 8, 64, 2100, [40, 1080], 32, 1e4),   # the same at d = 64 (64-key tiles)
]


def make_case(seed, M, n, H, Hkv, d, max_len, lens, rot, theta):
    rng = np.random.default_rng(seed)
    if lens is None:
        lens = rng.integers(0, max_len - n + 1, size=M)
    lens = np.asarray(lens, np.int32)
    q = rng.standard_normal((M, n, H * d), dtype=np.float32)
    kn = rng.standard_normal((M, n, Hkv * d), dtype=np.float32)
    vn = rng.standard_normal((M, n, Hkv * d), dtype=np.float32)
    # The cached rows hold keys rotated to their positions (as an earlier rotary append
    # would have left them): rotated here by the oracle; rows past the length are NaN.
    kc = np.full((M, Hkv, max_len, d), np.nan, np.float32)
    vc = np.full((M, Hkv, max_len, d), np.nan, np.float32)
    orc = oracle.default()
    for m in range(M):
        P = int(lens[m])
        if P == 0:
            continue
        raw = rng.standard_normal((P, Hkv * d), dtype=np.float32)
        rot_k = orc.rope(raw, np.arange(P, dtype=np.int32), Hkv, d, rot, theta).astype(np.float32)
        kc[m, :, :P] = rot_k.reshape(P, Hkv, d).transpose(1, 0, 2)
        vc[m, :, :P] = rng.standard_normal((Hkv, P, d), dtype=np.float32)
    return lens, q, kn, vn, kc, vc


def run_gpu(lens, q, kn, vn, kc, vc, M, n, H, Hkv, d, max_len, scale, rot, theta):
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    out = nan_like((M, n, H * d))
    taf.attn_prefill_cached_rope(to_dev(q), to_dev(kn), to_dev(vn), kc_d, vc_d, lens.tolist(), out, M, n, H, Hkv,
                                 d, max_len, scale, rot, theta)
    return to_host(out), to_host(kc_d), to_host(vc_d)


def check_caches(orc, got_k, got_v, kc, vc, kn, vn, lens, M, n, Hkv, d, rot, theta):
    """Rows P..P+n-1: keys rotated to their rows (tolerance), values copied; every other row untouched."""
    pos = (lens[:, None].astype(np.int64) + np.arange(n)[None, :]).reshape(-1)
    want_k = orc.rope(kn.reshape(M * n, Hkv * d), pos.astype(np.int32), Hkv, d, rot, theta).reshape(M, n, Hkv, d)
    for m in range(M):
        P = int(lens[m])
        rows_k = got_k[m, :, P:P + n].transpose(1, 0, 2).astype(np.float64)
        err = float(np.max(np.abs(rows_k - want_k[m])))
        assert err <= ROPE_ABS_TOL, f"sequence {m}: appended keys off by {err:.3e}"
        assert np.array_equal(bits(got_v[m, :, P:P + n]), bits(vn[m].reshape(n, Hkv, d).transpose(1, 0, 2))), \
            f"sequence {m}: appended values"
        for rows in (slice(0, P), slice(P + n, None)):
            assert np.array_equal(bits(got_k[m, :, rows]), bits(kc[m, :, rows])), f"sequence {m}: K rows touched"
            assert np.array_equal(bits(got_v[m, :, rows]), bits(vc[m, :, rows])), f"sequence {m}: V rows touched"


@pytest.mark.parametrize("case", CASES, ids=[f"M{c[0]}_n{c[1]}_H{c[2]}_Hkv{c[3]}_d{c[4]}_rot{c[7]}" for c in CASES])
def test_prefill_cached_rope(case):
    M, n, H, Hkv, d, max_len, lens, rot, theta = case
    lens, q, kn, vn, kc, vc = make_case(31 * M + n + rot, M, n, H, Hkv, d, max_len, lens, rot, theta)
    scale = wl.scale_for(d)
    note(f"prefill_cached_rope M={M} n={n} H={H} Hkv={Hkv} d={d} lens={lens.tolist()} rot={rot} theta={theta}")
    got, got_k, got_v = run_gpu(lens, q, kn, vn, kc, vc, M, n, H, Hkv, d, max_len, scale, rot, theta)
    orc = oracle.default()
    if M * n * H * max(int(lens.max()) + n, 1) <= 2_000_000:
        want = orc.prefill_cached_rope(q, kn, vn, kc, vc, lens, M, n, H, Hkv, d, max_len, scale, rot, theta)
    else:  # larger chunks: the numpy formulation on the oracle's own rotation
        pos = (lens[:, None].astype(np.int64) + np.arange(n)[None, :]).reshape(-1).astype(np.int32)
        qr = orc.rope(q.reshape(M * n, H * d), pos, H, d, rot, theta).astype(np.float32).reshape(q.shape)
        kr = orc.rope(kn.reshape(M * n, Hkv * d), pos, Hkv, d, rot, theta).astype(np.float32).reshape(kn.shape)
        want = brute.prefill_cached(qr, kr, vn, kc, vc, lens, M, n, H, Hkv, d, max_len, scale)
    assert_attn_close(got, want, f"prefill_cached_rope {case}")
    check_caches(orc, got_k, got_v, kc, vc, kn, vn, lens, M, n, Hkv, d, rot, theta)


def test_prefill_cached_rope_zero_width_is_plain():
    """rotary_ndims = 0: outputs and caches bit for bit those of attn_prefill_cached."""
    M, n, H, Hkv, d, max_len = 3, 150, 8, 2, 64, 400
    lens, q, kn, vn, kc, vc = make_case(77, M, n, H, Hkv, d, max_len, [0, 120, 250], 64, 1e4)
    scale = wl.scale_for(d)
    note("prefill_cached_rope width 0 vs plain")
    got, got_k, got_v = run_gpu(lens, q, kn, vn, kc, vc, M, n, H, Hkv, d, max_len, scale, 0, 1e4)
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    out = nan_like((M, n, H * d))
    taf.attn_prefill_cached(to_dev(q), to_dev(kn), to_dev(vn), kc_d, vc_d, lens.tolist(), out, M, n, H, Hkv, d,
                            max_len, scale)
    assert np.array_equal(bits(got), bits(to_host(out)))
    assert np.array_equal(bits(got_k), bits(to_host(kc_d))) and np.array_equal(bits(got_v), bits(to_host(vc_d)))


def test_prefill_cached_rope_second_half_full_size():
    """The causal prefill workload's second half (2048 tokens) behind its first half, rotary 128, base 1e4:
    the GPU builds its cache with a first rotary chunk, the oracle with its own rotation and append."""
    cfg = wl.PREFILL[3]
    M, H, d, max_len, P, rot, theta = cfg.B, cfg.H, cfg.d, 4096, 2048, 128, 1e4
    q, k, v = wl.prefill_inputs(cfg)
    rng = np.random.default_rng(4097)
    q2, k2, v2 = (rng.standard_normal(q.shape, dtype=np.float32) * np.float32(cfg.std) for _ in range(3))
    scale = cfg.scale
    note("prefill_cached_rope full size: 2048 behind 2048")
    kc_d = to_dev(wl.sentinel_cache((M, H, max_len, d)))
    vc_d = to_dev(wl.sentinel_cache((M, H, max_len, d)))
    first = nan_like((M, P, H * d))
    taf.attn_prefill_cached_rope(to_dev(q), to_dev(k), to_dev(v), kc_d, vc_d, [0] * M, first, M, P, H, H, d,
                                 max_len, scale, rot, theta)
    out = nan_like((M, P, H * d))
    taf.attn_prefill_cached_rope(to_dev(q2), to_dev(k2), to_dev(v2), kc_d, vc_d, [P] * M, out, M, P, H, H, d,
                                 max_len, scale, rot, theta)
    got, got_first = to_host(out), to_host(first)
    del kc_d, vc_d
    orc = oracle.default()
    pos0 = np.tile(np.arange(P, dtype=np.int32), M)
    pos1 = pos0 + P
    rot_rows = lambda x, pos: orc.rope(x.reshape(M * P, H * d), pos, H, d, rot, theta).astype(np.float32).reshape(x.shape)
    q_r, k_r, q2_r, k2_r = rot_rows(q, pos0), rot_rows(k, pos0), rot_rows(q2, pos1), rot_rows(k2, pos1)
    empty = wl.sentinel_cache((M, H, max_len, d))
    want_first = brute.prefill_cached(q_r, k_r, v, empty, empty, np.zeros(M, np.int32), M, P, H, H, d, max_len,
                                      scale)
    assert_attn_close(got_first, want_first, "first 2048 (all outputs)")
    kc, vc = empty.copy(), empty.copy()
    orc.scatter(k_r, v, kc, vc, np.zeros(M, np.int32), M, P, H, d, max_len)
    want = brute.prefill_cached(q2_r, k2_r, v2, kc, vc, np.full(M, P, np.int32), M, P, H, H, d, max_len, scale)
    assert_attn_close(got, want, "2048 behind 2048 (all outputs)")
