"""Seeded random shapes through the C ABI against the oracle.

Hand-picked cases sit on tile and block boundaries; these draw shapes from a
fixed seed instead, so that work decompositions nobody picked by hand are
compared too.  Decode draws batches up to 32 sequences, group sizes 1 to 20,
every head_dim and cache lengths up to 4000, with an empty, a one-key and a
full sequence in every batch of three or more: the launcher's split into bulk
and tail key blocks then sees sequence mixes of every kind; a second set draws
caches of up to 70000 rows and mostly one to four sequences.  Prefill draws
batch, length, heads, head_dim and causality (every small-problem and 4-wave
decomposition), the chunked prefill draws cached lengths behind a GQA cache,
and the append draws positions and row counts.  Attention outputs are compared
element by element at the f32 tolerance, appended caches bit for bit.
"""
import numpy as np
import pytest

import oracle
import transformer_attention_flash_amd as taf
from transformer_attention_flash_amd import workloads as wl
from gpu_common import assert_attn_close, bits, nan_like, note, to_dev, to_host

pytestmark = pytest.mark.gpu

CACHE_CAP = 24 << 20  # bytes per cache tensor, so that the oracle stays fast


def _decode_cases(n=48, seed=7777):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        d = int(rng.choice([32, 64, 128]))
        Hkv = int(rng.choice([1, 2, 3, 4, 8]))
        g = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 20]))
        M = int(rng.integers(1, 33))
        max_len = int(rng.integers(1, 4001))
        max_len = max(1, min(max_len, CACHE_CAP // (M * Hkv * d * 4)))
        lens = rng.integers(0, max_len + 1, size=M)
        if M >= 3:
            lens[:3] = [0, 1, max_len]
            rng.shuffle(lens)
        cases.append((M, Hkv * g, Hkv, d, max_len, [int(x) for x in lens]))
    return cases


def _decode_cases_wide(n=48, seed=4242):
    """Caches of 1 to 70000 rows (log-uniform), batches weighted to one or a few
    sequences, group sizes up to 32: calls of few units (equal key blocks, up to
    512 splits per head and the 16-wave merge) as often as calls of many, full,
    ragged and top-half lengths."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        d = int(rng.choice([32, 64, 128]))
        Hkv = int(rng.choice([1, 2, 4, 8, 16, 32]))
        g = int(rng.choice([1, 2, 4, 5, 8, 16, 17, 32]))
        M = int(rng.choice([1, 1, 2, 3, 4, 8, 16, 32]))
        max_len = int(np.exp(rng.uniform(0, np.log(70000))))
        max_len = max(1, min(max_len, 2 * CACHE_CAP // (M * Hkv * d * 4)))
        mode = rng.integers(3)
        lens = (rng.integers(0, max_len + 1, size=M) if mode == 0 else np.full(M, max_len) if mode == 1
                else rng.integers(max_len // 2, max_len + 1, size=M))
        cases.append((M, Hkv * g, Hkv, d, max_len, [int(x) for x in lens]))
    return cases


def _prefill_cases(n=24, seed=8888):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        d = int(rng.choice([32, 64, 128]))
        B = int(rng.integers(1, 4))
        S = int(rng.integers(1, 700))
        H = int(rng.integers(1, 11))
        cases.append((B, S, H, d, bool(rng.integers(2))))
    return cases


def _chunk_cases(n=12, seed=9999):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        d = int(rng.choice([32, 64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        H = Hkv * int(rng.choice([1, 2, 4, 8]))
        M = int(rng.integers(1, 5))
        n_new = int(rng.integers(1, 300))
        max_len = n_new + int(rng.integers(0, 1200))
        cached = rng.integers(0, max_len - n_new + 1, size=M)
        cases.append((M, n_new, H, Hkv, d, max_len, [int(x) for x in cached]))
    return cases


def _scatter_cases(n=16, seed=6666):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        d = int(rng.choice([32, 64, 128]))
        Hkv = int(rng.integers(1, 9))
        M = int(rng.integers(1, 33))
        n_new = int(rng.integers(1, 200))
        max_len = n_new + int(rng.integers(0, 300))
        pos = rng.integers(0, max_len - n_new + 1, size=M)
        cases.append((M, n_new, Hkv, d, max_len, [int(x) for x in pos]))
    return cases


DECODE = _decode_cases() + _decode_cases_wide()
PREFILL = _prefill_cases()
CHUNK = _chunk_cases()
SCATTER = _scatter_cases()


@pytest.mark.parametrize("case", DECODE, ids=[f"M{c[0]}_H{c[1]}_Hkv{c[2]}_d{c[3]}_max{c[4]}" for c in DECODE])
def test_random_decode(case):
    M, H, Hkv, d, max_len, lens = case
    rng = np.random.default_rng(M * 131 + H * 7 + d + max_len)
    lens = np.asarray(lens, np.int32)
    q = rng.standard_normal((M, H * d), dtype=np.float32)
    kc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    vc = rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32)
    for m in range(M):  # rows past L_m are NaN: reading one would poison the output
        kc[m, :, lens[m]:] = np.nan
        vc[m, :, lens[m]:] = np.nan
    scale = wl.scale_for(d)
    note(f"random decode M={M} H={H} Hkv={Hkv} d={d} max_len={max_len} lens={lens.tolist()}")
    import torch
    qd = to_dev(q)
    ws = torch.empty(taf.attn_decode_workspace_bytes(M, H, d, max_len) // 4, dtype=torch.float32, device=qd.device)
    out = nan_like((M, H * d))
    taf.attn_decode_gqa_batched(qd, to_dev(kc), to_dev(vc), lens.tolist(), out, M, H, Hkv, d, max_len, scale, ws)
    got = to_host(out)
    want = oracle.default().decode(q, kc, vc, lens, M, H, Hkv, d, max_len, scale)
    assert_attn_close(got, want, f"random decode {case}")
    for m in np.nonzero(lens == 0)[0]:
        assert np.all(got[m] == 0.0), "an empty sequence must give zeros"


@pytest.mark.parametrize("case", PREFILL, ids=[f"B{c[0]}_S{c[1]}_H{c[2]}_d{c[3]}_{'c' if c[4] else 'nc'}"
                                               for c in PREFILL])
def test_random_prefill(case):
    B, S, H, d, causal = case
    rng = np.random.default_rng(B * 1009 + S * 13 + H * 7 + d)
    q, k, v = (rng.standard_normal((B, S, H * d), dtype=np.float32) for _ in range(3))
    scale = wl.scale_for(d)
    note(f"random prefill B={B} S={S} H={H} d={d} causal={causal}")
    out = nan_like((B, S, H * d))
    taf.attn_prefill(to_dev(q), to_dev(k), to_dev(v), out, B, S, H, d, scale, causal)
    want = oracle.default().prefill(q, k, v, B, S, H, d, scale, causal)
    assert_attn_close(to_host(out), want, f"random prefill {case}")


@pytest.mark.parametrize("case", CHUNK, ids=[f"M{c[0]}_n{c[1]}_H{c[2]}_Hkv{c[3]}_d{c[4]}_max{c[5]}" for c in CHUNK])
def test_random_chunked_prefill(case):
    M, n, H, Hkv, d, max_len, cached = case
    rng = np.random.default_rng(M * 7 + n + H + max_len)
    cached = np.asarray(cached, np.int32)
    q = rng.standard_normal((M, n, H * d), dtype=np.float32)
    kn = rng.standard_normal((M, n, Hkv * d), dtype=np.float32)
    vn = rng.standard_normal((M, n, Hkv * d), dtype=np.float32)
    kc = wl.sentinel_cache((M, Hkv, max_len, d))
    vc = kc.copy()
    for m in range(M):  # rows before the chunk hold cached keys; rows past it stay NaN
        kc[m, :, :cached[m]] = rng.standard_normal((Hkv, cached[m], d), dtype=np.float32)
        vc[m, :, :cached[m]] = rng.standard_normal((Hkv, cached[m], d), dtype=np.float32)
    scale = wl.scale_for(d)
    note(f"random chunked prefill M={M} n={n} H={H} Hkv={Hkv} d={d} max_len={max_len} cached={cached.tolist()}")
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    out = nan_like((M, n, H * d))
    taf.attn_prefill_cached(to_dev(q), to_dev(kn), to_dev(vn), kc_d, vc_d, cached.tolist(), out, M, n, H, Hkv, d,
                            max_len, scale)
    orc = oracle.default()
    want = orc.prefill_cached(q, kn, vn, kc, vc, cached, M, n, H, Hkv, d, max_len, scale)
    assert_attn_close(to_host(out), want, f"random chunked prefill {case}")
    orc.scatter(kn, vn, kc, vc, cached, M, n, Hkv, d, max_len)
    assert np.array_equal(bits(to_host(kc_d)), bits(kc)), "K cache after the append"
    assert np.array_equal(bits(to_host(vc_d)), bits(vc)), "V cache after the append"


@pytest.mark.parametrize("case", SCATTER, ids=[f"M{c[0]}_n{c[1]}_hkv{c[2]}_d{c[3]}_max{c[4]}" for c in SCATTER])
def test_random_append(case):
    M, n_new, Hkv, d, max_len, pos = case
    rng = np.random.default_rng(M * 17 + n_new + Hkv + max_len)
    kn = rng.standard_normal((M, n_new, Hkv * d), dtype=np.float32)
    vn = rng.standard_normal((M, n_new, Hkv * d), dtype=np.float32)
    kc = wl.sentinel_cache((M, Hkv, max_len, d))
    vc = kc.copy()
    note(f"random append M={M} n_new={n_new} Hkv={Hkv} d={d} max_len={max_len} pos={pos}")
    kc_d, vc_d = to_dev(kc), to_dev(vc)
    taf.kv_cache_scatter(to_dev(kn), to_dev(vn), kc_d, vc_d, pos, M, n_new, Hkv, d, max_len)
    oracle.default().scatter(kn, vn, kc, vc, np.asarray(pos, np.int32), M, n_new, Hkv, d, max_len)
    assert np.array_equal(bits(to_host(kc_d)), bits(kc)), "K cache differs from the oracle"
    assert np.array_equal(bits(to_host(vc_d)), bits(vc)), "V cache differs from the oracle"
