"""KV-cache append on the GPU: bit-exact against the oracle, untouched bytes stay.

Cases span one and many blocks, ragged row counts, non-power-of-two KV head
counts (the kernel divides by Hkv), every supported head_dim, positions up to
max_len - n_new, NaN payloads in the source, and the full-size workloads: the
bulk append of the causal prefill's K/V into a [4, 32, 4096, 128] cache, and
the one-row-per-sequence append of both decode workloads.
"""
import numpy as np
import pytest

import oracle
import transformer_attention_flash_amd as taf
from transformer_attention_flash_amd import workloads as wl
from gpu_common import bits, note, to_dev, to_host

pytestmark = pytest.mark.gpu

SMALL = [
    # M, n_new, Hkv, d, max_len, lens (None = random valid)
    (1, 1, 1, 32, 1, [0]),
    (3, 5, 2, 64, 17, [0, 12, 7]),
    (32, 1, 8, 128, 64, None),
    (2, 37, 3, 128, 100, [63, 0]),
    (4, 300, 5, 32, 600, None),
    (7, 129, 6, 64, 130, [1, 0, 1, 0, 1, 0, 1]),
]


def run_case(orc, M, n_new, Hkv, d, max_len, lens, kc_host, vc_host, kn, vn):
    note(f"scatter M={M} n_new={n_new} Hkv={Hkv} d={d} max_len={max_len}")
    kc, vc = to_dev(kc_host), to_dev(vc_host)
    taf.kv_cache_scatter(to_dev(kn), to_dev(vn), kc, vc, lens, M, n_new, Hkv, d, max_len)
    got_k, got_v = to_host(kc), to_host(vc)
    want_k, want_v = kc_host.copy(), vc_host.copy()
    orc.scatter(kn, vn, want_k, want_v, lens, M, n_new, Hkv, d, max_len)
    assert np.array_equal(bits(got_k), bits(want_k)), "K cache differs from the oracle"
    assert np.array_equal(bits(got_v), bits(want_v)), "V cache differs from the oracle"


@pytest.mark.parametrize("case", SMALL, ids=[f"M{c[0]}_n{c[1]}_hkv{c[2]}_d{c[3]}_max{c[4]}" for c in SMALL])
def test_scatter_small(case):
    M, n_new, Hkv, d, max_len, lens = case
    rng = np.random.default_rng(7 + M * 1000 + n_new)
    if lens is None:
        lens = rng.integers(0, max_len - n_new + 1, size=M).tolist()
    kn = rng.standard_normal((M, n_new, Hkv * d), dtype=np.float32)
    vn = rng.standard_normal((M, n_new, Hkv * d), dtype=np.float32)
    kn.view(np.uint32).reshape(-1)[::97] = 0x7FA00001   # NaN payloads must survive
    sent = wl.sentinel_cache((M, Hkv, max_len, d))
    run_case(oracle.default(), M, n_new, Hkv, d, max_len, lens, sent.copy(), sent.copy(), kn, vn)


def test_scatter_fills_whole_cache_in_two_appends():
    M, Hkv, d, max_len = 2, 4, 128, 96
    rng = np.random.default_rng(11)
    orc = oracle.default()
    kc = wl.sentinel_cache((M, Hkv, max_len, d))
    vc = kc.copy()
    for n_new, lens in ((40, [0, 0]), (56, [40, 40])):
        kn = rng.standard_normal((M, n_new, Hkv * d), dtype=np.float32)
        vn = rng.standard_normal((M, n_new, Hkv * d), dtype=np.float32)
        run_case(orc, M, n_new, Hkv, d, max_len, lens, kc, vc, kn, vn)
        orc.scatter(kn, vn, kc, vc, lens, M, n_new, Hkv, d, max_len)
    assert not np.any(bits(kc) == wl.SENTINEL_BITS)


def test_scatter_bulk_prefill_rows_full_size():
    """Causal prefill's K/V (B=4, S=2048, H=32, d=128) into [4, 32, 4096, 128] from position 0."""
    cfg = wl.BULK_SCATTER
    _, k, v = wl.prefill_inputs(wl.PREFILL[3])
    sent = wl.sentinel_cache((cfg.M, cfg.Hkv, cfg.max_len, cfg.d))
    run_case(oracle.default(), cfg.M, cfg.n_new, cfg.Hkv, cfg.d, cfg.max_len, [0] * cfg.M, sent,
             sent.copy(), k, v)


@pytest.mark.parametrize("cid", [4, 5])
def test_scatter_decode_append_full_size(cid):
    """One new K/V row per sequence at position L_m - 1 of the N(0,1) decode caches."""
    cfg = wl.DECODE[cid]
    inp = wl.decode_inputs(cfg)
    run_case(oracle.default(), cfg.M, 1, cfg.Hkv, cfg.d, cfg.max_len, (inp["lens"] - 1).tolist(),
             inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"])
