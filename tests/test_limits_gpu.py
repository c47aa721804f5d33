"""The largest index spaces the entry points accept, on the GPU.

Prefill addresses [B, S, H*d] tensors up to 2^31 - 1 elements (8 GiB each):
a B=1023, S=128, H=128, d=128 problem has 2^31 - 2^21 elements per tensor, so
its last batch elements sit just below the limit.  Decode, append and slot
copy address caches beyond 2^31 elements (64-bit offsets): a
[32, 16, 65536, 128] cache holds 2^32 floats (16 GiB each), and the last
sequence lives in its top half.  Inputs are drawn on the GPU from a seeded
generator (drawing 50+ GiB on the host would take minutes); the slices the
checks need are copied to the host for the oracle, which treats batch
elements and sequences independently.
"""
import numpy as np
import pytest

import oracle
import transformer_attention_flash_amd as taf
from transformer_attention_flash_amd import workloads as wl
from gpu_common import assert_attn_close, bits, note

pytestmark = pytest.mark.gpu


def _randn(shape, seed):
    import torch
    g = torch.Generator(device="cuda:0")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device="cuda:0", dtype=torch.float32)


@pytest.mark.parametrize("causal", [False, True], ids=["full", "causal"])
def test_prefill_near_int32_element_limit(causal):
    import torch
    B, S, H, d = 1023, 128, 128, 128
    assert B * S * H * d == 2 ** 31 - 2 ** 21
    note(f"prefill near the int32 element limit causal={causal}")
    q, k, v = (_randn((B, S, H * d), 700 + i) for i in range(3))
    out = torch.full_like(q, float("nan"))
    scale = wl.scale_for(d)
    taf.attn_prefill(q, k, v, out, B, S, H, d, scale, causal)
    lowp = torch.full_like(q, float("nan"))
    taf.attn_prefill_lowp(q, k, v, lowp, B, S, H, d, scale, causal, taf.ATTN_PREC_BF16)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lowp).all()), "every element written"
    orc = oracle.default()
    for b in (0, 511, B - 1):  # every output of the first, a middle and the last batch element
        qb, kb, vb = (x[b:b + 1].cpu().numpy() for x in (q, k, v))
        want = orc.prefill(qb, kb, vb, 1, S, H, d, scale, causal)
        assert_attn_close(out[b:b + 1].cpu().numpy(), want, f"prefill b={b}")
        rq, rk, rv = (orc.round16(x, orc.BF16) for x in (qb, kb, vb))
        want_lp = orc.prefill(rq, rk, rv, 1, S, H, d, scale, causal)
        err = float(np.max(np.abs(lowp[b:b + 1].cpu().numpy() - want_lp)))
        assert err <= 2.0 * 2.0 ** -8 * float(np.max(np.abs(rv))) + 1e-5, f"reduced precision b={b}: {err:.3e}"
    del q, k, v, out, lowp
    torch.cuda.empty_cache()


def test_cache_beyond_int32_elements():
    """Append at the last row, decode, and slot copy on caches of 2^32 elements."""
    import torch
    M, Hkv, H, d, max_len = 32, 16, 16, 128, 65536
    assert M * Hkv * max_len * d == 2 ** 32
    note("caches of 2^32 elements: append, decode, slot copy")
    kc = _randn((M, Hkv, max_len, d), 710)
    vc = _randn((M, Hkv, max_len, d), 711)
    lens = [1 + 3 * m for m in range(M - 1)] + [max_len]
    k_new = _randn((M, 1, Hkv * d), 712)
    v_new = _randn((M, 1, Hkv * d), 713)
    taf.kv_cache_scatter(k_new, v_new, kc, vc, [x - 1 for x in lens], M, 1, Hkv, d, max_len)
    q = _randn((M, H * d), 714)
    ws = torch.empty(taf.attn_decode_workspace_bytes(M, H, d, max_len) // 4, device="cuda:0")
    out = torch.full((M, H * d), float("nan"), device="cuda:0")
    scale = wl.scale_for(d)
    taf.attn_decode_gqa_batched(q, kc, vc, lens, out, M, H, Hkv, d, max_len, scale, ws)
    torch.cuda.synchronize()
    orc = oracle.default()
    m = M - 1  # its rows start at element 31 * 16 * 65536 * 128 > 2^31
    k_host = kc[m:m + 1].cpu().numpy()
    v_host = vc[m:m + 1].cpu().numpy()
    # The append wrote k_new / v_new at the very last row of the very last sequence.
    assert np.array_equal(bits(k_host[0, :, max_len - 1, :].reshape(-1)), bits(k_new[m].cpu().numpy().reshape(-1)))
    assert np.array_equal(bits(v_host[0, :, max_len - 1, :].reshape(-1)), bits(v_new[m].cpu().numpy().reshape(-1)))
    want = orc.decode(q[m:m + 1].cpu().numpy(), k_host, v_host, np.array([max_len], np.int32), 1, H, Hkv, d,
                      max_len, scale)
    assert_attn_close(out[m:m + 1].cpu().numpy(), want, "decode of the last sequence")
    for s in range(M - 1):  # every other sequence, from its live rows only
        L = lens[s]
        ks = np.ascontiguousarray(kc[s:s + 1, :, :L].cpu().numpy())
        vs = np.ascontiguousarray(vc[s:s + 1, :, :L].cpu().numpy())
        want = orc.decode(q[s:s + 1].cpu().numpy(), ks, vs, np.array([L], np.int32), 1, H, Hkv, d, L, scale)
        assert_attn_close(out[s:s + 1].cpu().numpy(), want, f"decode of sequence {s}")
    # Slot copy of a single cache into the last slot (offsets beyond 2^31 elements).
    src_k = _randn((Hkv, 4096, d), 715)
    src_v = _randn((Hkv, 4096, d), 716)
    slot_lens = list(lens)
    taf.kv_cache_copy_to_slot(src_k, src_v, 4096, 4096, kc, vc, m, M, Hkv, d, max_len, slot_lens)
    torch.cuda.synchronize()
    assert slot_lens[m] == 4096
    assert torch.equal(kc[m, :, :4096], src_k) and torch.equal(vc[m, :, :4096], src_v)
    assert torch.equal(kc[m, :, max_len - 1], k_new[m, 0].view(Hkv, d)), "rows past the copy untouched"
    del kc, vc, ws, out
    torch.cuda.empty_cache()
