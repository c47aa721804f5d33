"""Rotary position embedding fused into the KV append and the decode, on the GPU,
against the fp64 oracle.

kv_cache_scatter_rope: values and every byte the append does not rotate are
compared bit for bit (untouched cache rows keep their sentinel, key dims past
rotary_ndims are copied verbatim); the rotated key dims against the oracle's
fp64 rotation within ROPE_ABS_TOL.

attn_decode_gqa_batched_rope: the oracle rotates the query to position
L_m - 1 in fp64, hands it over in f32, and runs its decode; the GPU output
must meet the attention tolerance.  Cases cover full and partial rotary widths
(8 .. head_dim), bases 500 / 10000 / 1000000, positions up to ~10^6 (where a
single-precision angle would be off by ~0.03 rad), rotary_ndims = 0 (equal to
the plain entry points, bit for bit), and the full decode workloads as one
step: rotate-and-append the new key at L_m - 1, then rotate the query and
attend over L_m keys.
"""
import numpy as np
import pytest

import oracle
import transformer_attention_flash_amd as taf
from transformer_attention_flash_amd import workloads as wl
from gpu_common import assert_attn_close, bits, nan_like, note, to_dev, to_host

pytestmark = pytest.mark.gpu

# A rotated f32 element against the exact rotation: the angle reaches the
# single-precision sin/cos as a fraction of a turn reduced in double (error
# ~2e-7 rad after the f32 hand-over), sin/cos and the two products add a few
# ulps, so |error| <~ |x| * 5e-7; inputs are N(0, 1), |x| < 7.
ROPE_ABS_TOL = 1e-5


def rope_rows(orc, x, pos, heads, d, rot, theta):
    """Oracle rotation of rows x [n, heads * d] at positions pos [n] (fp64)."""
    return orc.rope(x.reshape(len(pos), heads * d), np.asarray(pos, np.int32), heads, d, rot, theta)


SCATTER = [
    # M, n_new, Hkv, d, max_len, lens (None = random valid), rotary_ndims, theta
    (1, 1, 1, 32, 1, [0], 32, 10000.0),
    (3, 5, 2, 64, 40000, [0, 32000, 39990], 64, 10000.0),
    (2, 37, 3, 128, 100, [63, 0], 32, 10000.0),
    (4, 300, 5, 32, 600, None, 16, 1e6),
    (2, 129, 8, 128, 1000, [0, 871], 128, 1e6),
    (3, 2, 2, 64, 300, [5, 9, 290], 8, 500.0),
    (1, 2, 1, 32, 1 << 20, [(1 << 20) - 2], 32, 10000.0),
]


def _scatter_check(orc, M, n_new, Hkv, d, max_len, lens, rot, theta, kn, vn):
    sent = wl.sentinel_cache((M, Hkv, max_len, d))
    kc, vc = to_dev(sent), to_dev(sent)
    taf.kv_cache_scatter_rope(to_dev(kn), to_dev(vn), kc, vc, list(lens), M, n_new, Hkv, d, max_len, rot, theta)
    got_k, got_v = to_host(kc), to_host(vc)
    del kc, vc
    pos = (np.asarray(lens, np.int64)[:, None] + np.arange(n_new)[None, :]).reshape(-1)
    want_rows = rope_rows(orc, kn, pos, Hkv, d, rot, theta).reshape(M, n_new, Hkv, d)
    # Values: a plain append.
    want_v = sent.copy()
    orc.scatter(kn, vn, sent.copy(), want_v, np.asarray(lens, np.int32), M, n_new, Hkv, d, max_len)
    assert np.array_equal(bits(got_v), bits(want_v)), "V cache differs from the oracle append"
    # Keys: outside the rotated dims of the written rows, the oracle append of
    # the f32-rounded rotation (identical bits: those dims are copies);
    # inside, the fp64 rotation within ROPE_ABS_TOL.
    want_k = sent.copy()
    orc.scatter(want_rows.astype(np.float32).reshape(M, n_new, Hkv * d), vn, want_k, sent.copy(),
                np.asarray(lens, np.int32), M, n_new, Hkv, d, max_len)
    mask = np.zeros(got_k.shape, bool)
    for m in range(M):
        mask[m, :, lens[m]:lens[m] + n_new, :rot] = True
    assert np.array_equal(bits(got_k)[~mask], bits(want_k)[~mask]), "K bytes outside the rotated dims differ"
    got_rows = np.stack([got_k[m, :, lens[m]:lens[m] + n_new, :].transpose(1, 0, 2) for m in range(M)])
    err = float(np.max(np.abs(got_rows.astype(np.float64) - want_rows))) if got_rows.size else 0.0
    assert err <= ROPE_ABS_TOL, f"rotated keys: max abs err {err:.3e}"
    return err


@pytest.mark.parametrize("case", SCATTER, ids=[f"M{c[0]}_n{c[1]}_hkv{c[2]}_d{c[3]}_max{c[4]}_rot{c[6]}"
                                               for c in SCATTER])
def test_scatter_rope_small(case):
    M, n_new, Hkv, d, max_len, lens, rot, theta = case
    rng = np.random.default_rng(31 + M * 1000 + n_new)
    if lens is None:
        lens = rng.integers(0, max_len - n_new + 1, size=M).tolist()
    kn = rng.standard_normal((M, n_new, Hkv * d), dtype=np.float32)
    vn = rng.standard_normal((M, n_new, Hkv * d), dtype=np.float32)
    vn.view(np.uint32).reshape(-1)[::97] = 0x7FA00001   # values are bytes: NaN payloads survive
    note(f"scatter_rope M={M} n_new={n_new} Hkv={Hkv} d={d} max_len={max_len} rot={rot} theta={theta}")
    _scatter_check(oracle.default(), M, n_new, Hkv, d, max_len, lens, rot, theta, kn, vn)


def test_scatter_rope_zero_width_is_plain_append():
    M, n_new, Hkv, d, max_len = 2, 9, 4, 128, 64
    rng = np.random.default_rng(77)
    kn = rng.standard_normal((M, n_new, Hkv * d), dtype=np.float32)
    vn = rng.standard_normal((M, n_new, Hkv * d), dtype=np.float32)
    sent = wl.sentinel_cache((M, Hkv, max_len, d))
    note("scatter_rope rot=0")
    a_k, a_v, b_k, b_v = (to_dev(sent) for _ in range(4))
    taf.kv_cache_scatter_rope(to_dev(kn), to_dev(vn), a_k, a_v, [3, 50], M, n_new, Hkv, d, max_len, 0, 10000.0)
    taf.kv_cache_scatter(to_dev(kn), to_dev(vn), b_k, b_v, [3, 50], M, n_new, Hkv, d, max_len)
    assert np.array_equal(bits(to_host(a_k)), bits(to_host(b_k)))
    assert np.array_equal(bits(to_host(a_v)), bits(to_host(b_v)))


def test_scatter_rope_bulk_full_size():
    """The bulk append (4 x 2048 rows into [4, 32, 4096, 128]) with a full-width rotation, base 10000."""
    import torch
    cfg = wl.BULK_SCATTER
    rng = np.random.default_rng(4242)
    lens = [0, 1024, 2048, 2047]
    kn = wl.normal(rng, (cfg.M, cfg.n_new, cfg.Hkv * cfg.d))
    vn = wl.normal(rng, (cfg.M, cfg.n_new, cfg.Hkv * cfg.d))
    note("scatter_rope bulk full size")
    _scatter_check(oracle.default(), cfg.M, cfg.n_new, cfg.Hkv, cfg.d, cfg.max_len, lens, cfg.d, 10000.0, kn, vn)
    torch.cuda.empty_cache()


def run_decode_rope(q, kc, vc, lens, M, H, Hkv, d, max_len, scale, rot, theta):
    import torch
    ws = torch.empty(taf.attn_decode_workspace_bytes(M, H, d, max_len) // 4, dtype=torch.float32, device=q.device)
    out = nan_like((M, H * d))
    taf.attn_decode_gqa_batched_rope(q, kc, vc, lens, out, M, H, Hkv, d, max_len, scale, rot, theta, ws)
    return to_host(out)


def rotated_queries(orc, q, lens, H, d, rot, theta):
    """The oracle's queries turned to position L_m - 1, handed over in f32."""
    pos = np.maximum(np.asarray(lens, np.int64) - 1, 0)
    return rope_rows(orc, q, pos, H, d, rot, theta).astype(np.float32)


DECODE = [
    # M, H, Hkv, d, max_len, lens (None = random), rotary_ndims, theta
    (1, 1, 1, 32, 1, [1], 32, 10000.0),
    (2, 4, 4, 64, 70, [0, 70], 64, 10000.0),
    (4, 8, 2, 128, 300, [1, 31, 32, 33], 32, 10000.0),
    (3, 16, 2, 128, 40000, [64, 32768, 40000], 128, 1e6),
    (5, 12, 4, 64, 2000, [0, 511, 512, 513, 1999], 16, 500.0),
    (32, 8, 8, 32, 50, None, 8, 10000.0),
    (2, 64, 2, 128, 130, [130, 7], 64, 1e6),
    # long enough per workgroup slot for 32-key chunks at d = 64
    (8, 32, 16, 64, 32768, [32768, 31000, 30500, 29000, 32000, 28000, 30000, 31500], 64, 1e4),
]


@pytest.mark.parametrize("case", DECODE, ids=[f"M{c[0]}_H{c[1]}_Hkv{c[2]}_d{c[3]}_max{c[4]}_rot{c[6]}"
                                              for c in DECODE])
def test_decode_rope_small(case):
    M, H, Hkv, d, max_len, lens, rot, theta = case
    rng = np.random.default_rng(300 + M * 7 + H)
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
    note(f"decode_rope M={M} H={H} Hkv={Hkv} d={d} max_len={max_len} rot={rot} theta={theta} lens={lens.tolist()}")
    got = run_decode_rope(to_dev(q), to_dev(kc), to_dev(vc), lens.tolist(), M, H, Hkv, d, max_len, scale, rot, theta)
    orc = oracle.default()
    want = orc.decode(rotated_queries(orc, q, lens, H, d, rot, theta), kc, vc, lens, M, H, Hkv, d, max_len, scale)
    assert_attn_close(got, want, f"decode_rope {case}")
    for m in np.nonzero(lens == 0)[0]:
        assert np.all(got[m] == 0.0), "an empty sequence must give zeros"


def test_decode_rope_zero_width_is_plain_decode():
    M, H, Hkv, d, max_len = 3, 16, 4, 128, 700
    rng = np.random.default_rng(78)
    q = rng.standard_normal((M, H * d), dtype=np.float32)
    kc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    vc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    lens = [700, 1, 333]
    scale = wl.scale_for(d)
    note("decode_rope rot=0")
    import torch
    qd, kd, vd = to_dev(q), to_dev(kc), to_dev(vc)
    got = run_decode_rope(qd, kd, vd, lens, M, H, Hkv, d, max_len, scale, 0, 10000.0)
    ws = torch.empty(taf.attn_decode_workspace_bytes(M, H, d, max_len) // 4, dtype=torch.float32, device=qd.device)
    out = nan_like((M, H * d))
    taf.attn_decode_gqa_batched(qd, kd, vd, lens, out, M, H, Hkv, d, max_len, scale, ws)
    assert np.array_equal(bits(got), bits(to_host(out)))


@pytest.mark.parametrize("cid,rot,theta", [(4, 64, 10000.0), (5, 128, 1e6)])
def test_decode_rope_step_full_size(cid, rot, theta):
    """Rotate-and-append the new key at L_m - 1, then rotate the query and attend over L_m keys."""
    import torch
    cfg = wl.DECODE[cid]
    inp = wl.decode_inputs(cfg)
    lens = inp["lens"]
    note(f"decode_rope step full size {cfg.name} rot={rot} theta={theta} sum(L)={int(lens.sum())}")
    kc, vc = to_dev(inp["k_cache"]), to_dev(inp["v_cache"])
    taf.kv_cache_scatter_rope(to_dev(inp["k_new"]), to_dev(inp["v_new"]), kc, vc, (lens - 1).tolist(),
                              cfg.M, 1, cfg.Hkv, cfg.d, cfg.max_len, rot, theta)
    got = run_decode_rope(to_dev(inp["q"]), kc, vc, lens.tolist(), cfg.M, cfg.H, cfg.Hkv, cfg.d, cfg.max_len,
                          cfg.scale, rot, theta)
    new_rows = to_host(kc[torch.arange(cfg.M, device=kc.device), :, torch.as_tensor((lens - 1).astype(np.int64), device=kc.device)])
    del kc, vc
    torch.cuda.empty_cache()
    orc = oracle.default()
    k_rot = rope_rows(orc, inp["k_new"], lens - 1, cfg.Hkv, cfg.d, rot, theta)
    err = float(np.max(np.abs(new_rows.reshape(cfg.M, -1).astype(np.float64) - k_rot)))
    assert err <= ROPE_ABS_TOL, f"appended rotated keys: max abs err {err:.3e}"
    k_host, v_host = inp["k_cache"], inp["v_cache"]
    orc.scatter(k_rot.astype(np.float32).reshape(cfg.M, 1, -1), inp["v_new"], k_host, v_host, lens - 1, cfg.M, 1,
                cfg.Hkv, cfg.d, cfg.max_len)
    q_rot = rotated_queries(orc, inp["q"], lens, cfg.H, cfg.d, rot, theta)
    want = orc.decode(q_rot, k_host, v_host, lens, cfg.M, cfg.H, cfg.Hkv, cfg.d, cfg.max_len, cfg.scale)
    assert_attn_close(got, want, f"{cfg.name} rotated (all outputs)")
