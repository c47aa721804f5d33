"""Slot management on the GPU: copy of a prefilled single cache into a batch
slot (bit-exact against the oracle), and the length bookkeeping around it.

Cases: single and batched caches with different max_len, every head_dim, the
last slot of a 32-sequence batch, seq_len 0 (nothing launched), seq_len equal
to either cache's capacity, NaN payloads, and the full-size copy of a
2048-token prefill's K/V ([32, 2048, 128] per tensor) into slot 2 of the
[4, 32, 4096, 128] batched cache.  Two relations of the serving flow: a decode
of the slot equals a decode of the single cache, and a rollback after
speculative appends gives the decode from before them, bit for bit.
"""
import numpy as np
import pytest

import oracle
import transformer_attention_flash_amd as taf
from transformer_attention_flash_amd import workloads as wl
from gpu_common import assert_attn_close, bits, nan_like, note, to_dev, to_host

pytestmark = pytest.mark.gpu

SMALL = [
    # Hkv, d, src_max_len, seq_len, M, max_len, slot
    (1, 32, 1, 1, 1, 1, 0),
    (4, 64, 100, 37, 3, 64, 1),
    (8, 128, 4096, 1000, 2, 1000, 1),
    (2, 128, 50, 50, 32, 80, 31),
    (3, 32, 777, 0, 4, 777, 2),
    (5, 64, 300, 299, 5, 1024, 0),
]


def run_copy(orc, Hkv, d, src_max, seq_len, M, max_len, slot, sk, sv):
    sent = wl.sentinel_cache((M, Hkv, max_len, d))
    kc, vc = to_dev(sent), to_dev(sent)
    lens = [7] * M
    taf.kv_cache_copy_to_slot(to_dev(sk), to_dev(sv), src_max, seq_len, kc, vc, slot, M, Hkv, d, max_len, lens)
    assert lens[slot] == seq_len and all(lens[m] == 7 for m in range(M) if m != slot)
    got_k, got_v = to_host(kc), to_host(vc)
    want_k, want_v = sent.copy(), sent.copy()
    orc.copy_to_slot(sk, sv, src_max, seq_len, want_k, want_v, slot, M, Hkv, d, max_len)
    assert np.array_equal(bits(got_k), bits(want_k)), "K cache differs from the oracle copy"
    assert np.array_equal(bits(got_v), bits(want_v)), "V cache differs from the oracle copy"


@pytest.mark.parametrize("case", SMALL, ids=[f"hkv{c[0]}_d{c[1]}_src{c[2]}_n{c[3]}_M{c[4]}_max{c[5]}_slot{c[6]}"
                                             for c in SMALL])
def test_copy_to_slot_small(case):
    Hkv, d, src_max, seq_len, M, max_len, slot = case
    rng = np.random.default_rng(500 + Hkv * 100 + seq_len)
    sk = rng.standard_normal((Hkv, src_max, d), dtype=np.float32)
    sv = rng.standard_normal((Hkv, src_max, d), dtype=np.float32)
    sk.view(np.uint32).reshape(-1)[::101] = 0x7FA00001
    note(f"copy_to_slot Hkv={Hkv} d={d} src_max={src_max} seq_len={seq_len} M={M} max_len={max_len} slot={slot}")
    run_copy(oracle.default(), Hkv, d, src_max, seq_len, M, max_len, slot, sk, sv)


def test_copy_to_slot_full_size():
    """A 2048-token prefill's K/V as a single [32, 4096, 128] cache, copied into slot 2 of [4, 32, 4096, 128]."""
    import torch
    cfg = wl.BULK_SCATTER
    rng = np.random.default_rng(2048)
    src_max, seq_len = cfg.max_len, cfg.n_new
    sk = wl.sentinel_cache((cfg.Hkv, src_max, cfg.d))
    sv = sk.copy()
    sk[:, :seq_len] = wl.normal(rng, (cfg.Hkv, seq_len, cfg.d))
    sv[:, :seq_len] = wl.normal(rng, (cfg.Hkv, seq_len, cfg.d))
    note("copy_to_slot full size")
    run_copy(oracle.default(), cfg.Hkv, cfg.d, src_max, seq_len, cfg.M, cfg.max_len, 2, sk, sv)
    torch.cuda.empty_cache()


def _decode(q, kc, vc, lens, M, H, Hkv, d, max_len, scale):
    import torch
    ws = torch.empty(taf.attn_decode_workspace_bytes(M, H, d, max_len) // 4, dtype=torch.float32, device=q.device)
    out = nan_like((M, H * d))
    taf.attn_decode_gqa_batched(q, kc, vc, lens, out, M, H, Hkv, d, max_len, scale, ws)
    return to_host(out)


def test_slot_decode_equals_single_cache_decode():
    """Prefill K/V appended into a single cache, copied to slot 1: decoding the slot equals decoding the single cache."""
    import torch
    H, Hkv, d, S, src_max, M, max_len, slot = 16, 4, 128, 700, 1024, 3, 2048, 1
    rng = np.random.default_rng(601)
    k = rng.standard_normal((1, S, Hkv * d), dtype=np.float32)
    v = rng.standard_normal((1, S, Hkv * d), dtype=np.float32)
    q = rng.standard_normal((M, H * d), dtype=np.float32)
    scale = wl.scale_for(d)
    note("slot decode == single decode")
    dev = torch.device("cuda:0")
    sk = torch.full((1, Hkv, src_max, d), float("nan"), device=dev)
    sv = torch.full((1, Hkv, src_max, d), float("nan"), device=dev)
    taf.kv_cache_scatter(to_dev(k), to_dev(v), sk, sv, [0], 1, S, Hkv, d, src_max)
    bk = torch.full((M, Hkv, max_len, d), float("nan"), device=dev)
    bv = torch.full((M, Hkv, max_len, d), float("nan"), device=dev)
    lens = [0] * M
    taf.kv_cache_copy_to_slot(sk, sv, src_max, S, bk, bv, slot, M, Hkv, d, max_len, lens)
    assert lens == [0, S, 0]
    qd = to_dev(q)
    got = _decode(qd, bk, bv, lens, M, H, Hkv, d, max_len, scale)[slot]
    single = _decode(qd[slot:slot + 1].contiguous(), sk, sv, [S], 1, H, Hkv, d, src_max, scale)[0]
    kc = np.full((1, Hkv, src_max, d), np.nan, np.float32)
    vc = kc.copy()
    oracle.default().scatter(k, v, kc, vc, np.array([0], np.int32), 1, S, Hkv, d, src_max)
    want = oracle.default().decode(q[slot:slot + 1], kc, vc, np.array([S], np.int32), 1, H, Hkv, d, src_max, scale)[0]
    assert_attn_close(got, want, "slot decode vs oracle")
    assert_attn_close(single, want, "single decode vs oracle")
    assert np.max(np.abs(got - single)) <= 2e-6
    other = _decode(qd, bk, bv, lens, M, H, Hkv, d, max_len, scale)
    assert np.all(other[0] == 0) and np.all(other[2] == 0), "empty slots decode to zeros"


def test_rollback_restores_decode():
    """Append 3 speculative tokens, roll the lengths back: the decode equals the one from before, bit for bit."""
    import torch
    M, H, Hkv, d, max_len = 4, 8, 2, 64, 512
    rng = np.random.default_rng(602)
    kc = to_dev(rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32))
    vc = to_dev(rng.standard_normal((M, Hkv, max_len, d), dtype=np.float32))
    q = to_dev(rng.standard_normal((M, H * d), dtype=np.float32))
    lens = [100, 300, 1, 509]
    scale = wl.scale_for(d)
    note("rollback restores decode")
    before = _decode(q, kc, vc, lens, M, H, Hkv, d, max_len, scale)
    spec_k = to_dev(rng.standard_normal((M, 3, Hkv * d), dtype=np.float32))
    spec_v = to_dev(rng.standard_normal((M, 3, Hkv * d), dtype=np.float32))
    taf.kv_cache_scatter(spec_k, spec_v, kc, vc, lens, M, 3, Hkv, d, max_len)
    grown = [x + 3 for x in lens]
    during = _decode(q, kc, vc, grown, M, H, Hkv, d, max_len, scale)
    assert not np.array_equal(bits(during), bits(before))
    # Roll back per sequence to its pre-speculation length (the page's rollback
    # truncates every length to one position; apply it to each sequence alone).
    rolled = []
    for m in range(M):
        one = [grown[m]]
        taf.kv_lengths_rollback(one, 1, lens[m])
        rolled += one
    assert rolled == lens
    after = _decode(q, kc, vc, rolled, M, H, Hkv, d, max_len, scale)
    assert np.array_equal(bits(after), bits(before))
    torch.cuda.synchronize()
