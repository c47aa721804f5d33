"""Independent numpy fp64 brute force for tiny attention shapes.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  A second formulation
of the same definitions as ``oracle.c``, written differently on purpose so the
two cannot share a mistake: heads are split with reshapes, scores are formed
as full matrices, the causal mask is a lower-triangular boolean mask, and the
softmax is taken over whole rows of the masked matrix.

Definitions: trueno-gpu 0.4.11 ``src/memory/resident/attention.rs``,
``batched_multihead_attention`` (softmax(Q K^T / sqrt(d_k)) V per head over
interleaved [seq, n_heads*head_dim]); trustformers-core 0.2.0
``src/gpu_ops/cuda/oxicuda/attention.rs``, ``attention_prefill_gpu_to_gpu`` and
``softmax_causal_gpu_to_gpu`` (query i sees keys 0..=i, masked cells are 0);
realizar 0.8.5 ``src/cuda/executor/cache_from_cache_from_kv_cache.rs``,
``init_batched_kv_cache_gpu`` ([M, num_kv_heads, max_len, head_dim] caches).
"""
from __future__ import annotations

import numpy as np


def _softmax_rows(s: np.ndarray, visible: np.ndarray) -> np.ndarray:
    s = np.where(visible, s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.where(visible, np.exp(s), 0.0)
    return e / e.sum(axis=-1, keepdims=True)


def prefill(q, k, v, B, S, H, d, scale, causal):
    qh = np.asarray(q, dtype=np.float64).reshape(B, S, H, d).transpose(0, 2, 1, 3)
    kh = np.asarray(k, dtype=np.float64).reshape(B, S, H, d).transpose(0, 2, 1, 3)
    vh = np.asarray(v, dtype=np.float64).reshape(B, S, H, d).transpose(0, 2, 1, 3)
    s = float(np.float32(scale)) * (qh @ kh.transpose(0, 1, 3, 2))          # [B, H, S, S]
    visible = np.tril(np.ones((S, S), dtype=bool)) if causal else np.ones((S, S), dtype=bool)
    p = _softmax_rows(s, visible[None, None])
    o = p @ vh                                                               # [B, H, S, d]
    return o.transpose(0, 2, 1, 3).reshape(B, S, H * d)


def decode(q, k_cache, v_cache, lens, M, H, Hkv, d, max_len, scale):
    g = H // Hkv
    qm = np.asarray(q, dtype=np.float64).reshape(M, H, d)
    kc = np.asarray(k_cache, dtype=np.float64).reshape(M, Hkv, max_len, d)
    vc = np.asarray(v_cache, dtype=np.float64).reshape(M, Hkv, max_len, d)
    out = np.zeros((M, H, d))
    for m in range(M):
        L = int(lens[m])
        if L == 0:
            continue
        # Repeat each KV head over its g query heads, then attend per head.
        kr = np.repeat(kc[m, :, :L, :], g, axis=0)                           # [H, L, d]
        vr = np.repeat(vc[m, :, :L, :], g, axis=0)
        s = float(np.float32(scale)) * np.einsum("hd,hld->hl", qm[m], kr)
        p = _softmax_rows(s, np.ones_like(s, dtype=bool))
        out[m] = np.einsum("hl,hld->hd", p, vr)
    return out.reshape(M, H * d)


def scatter(k_new, v_new, k_cache, v_cache, cache_lens, M, n_new, Hkv, d, max_len):
    """Fancy-index append on uint32 views (bit-exact); returns new arrays."""
    kc = np.array(k_cache, dtype=np.float32, copy=True).reshape(M, Hkv, max_len, d).view(np.uint32)
    vc = np.array(v_cache, dtype=np.float32, copy=True).reshape(M, Hkv, max_len, d).view(np.uint32)
    kn = np.asarray(k_new, dtype=np.float32).reshape(M, n_new, Hkv, d).view(np.uint32)
    vn = np.asarray(v_new, dtype=np.float32).reshape(M, n_new, Hkv, d).view(np.uint32)
    for m in range(M):
        pos = int(cache_lens[m]) + np.arange(n_new)
        kc[m][:, pos, :] = kn[m].transpose(1, 0, 2)
        vc[m][:, pos, :] = vn[m].transpose(1, 0, 2)
    return kc.view(np.float32), vc.view(np.float32)


def prefill_cached(q, k_new, v_new, k_cache, v_cache, cache_lens, M, n_new, H, Hkv, d, max_len, scale):
    """Concatenate cached rows 0..P-1 and the new rows, then a causal mask shifted by P."""
    g = H // Hkv
    qm = np.asarray(q, dtype=np.float64).reshape(M, n_new, H, d)
    kn = np.asarray(k_new, dtype=np.float64).reshape(M, n_new, Hkv, d)
    vn = np.asarray(v_new, dtype=np.float64).reshape(M, n_new, Hkv, d)
    kc = np.asarray(k_cache, dtype=np.float64).reshape(M, Hkv, max_len, d)
    vc = np.asarray(v_cache, dtype=np.float64).reshape(M, Hkv, max_len, d)
    out = np.zeros((M, n_new, H, d))
    for m in range(M):
        P = int(cache_lens[m])
        keys = np.concatenate([kc[m, :, :P, :], kn[m].transpose(1, 0, 2)], axis=1)   # [Hkv, P+n, d]
        vals = np.concatenate([vc[m, :, :P, :], vn[m].transpose(1, 0, 2)], axis=1)
        keys = np.repeat(keys, g, axis=0)
        vals = np.repeat(vals, g, axis=0)                                           # [H, P+n, d]
        s = float(np.float32(scale)) * np.einsum("rhd,hjd->hrj", qm[m], keys)      # [H, n, P+n]
        visible = np.arange(P + n_new)[None, :] <= (P + np.arange(n_new))[:, None]
        p = _softmax_rows(s, visible[None])
        out[m] = np.einsum("hrj,hjd->rhd", p, vals)
    return out.reshape(M, n_new, H * d)


def rope(x, pos, H, d, rotary_ndims, base):
    """Each pair (x_i, x_{i+half}) as the complex number x_i + 1j x_{i+half}, multiplied by e^{1j a}."""
    x = np.asarray(x, dtype=np.float64).reshape(len(pos), H, d).copy()
    half = rotary_ndims // 2
    if half == 0:
        return x.reshape(len(pos), H * d)
    i = np.arange(half, dtype=np.float64)
    a = np.asarray(pos, dtype=np.float64)[:, None] * np.float64(base) ** (-2.0 * i / rotary_ndims)  # [n, half]
    z = (x[:, :, :half] + 1j * x[:, :, half:2 * half]) * np.exp(1j * a)[:, None, :]
    x[:, :, :half] = z.real
    x[:, :, half:2 * half] = z.imag
    return x.reshape(len(pos), H * d)


def copy_to_slot(src_k, src_v, src_max_len, seq_len, dst_k, dst_v, slot, M, Hkv, d, max_len):
    """Slice assignment on uint32 views; returns new arrays."""
    out = []
    for src, dst in ((src_k, dst_k), (src_v, dst_v)):
        b = np.array(dst, dtype=np.float32, copy=True).reshape(M, Hkv, max_len, d).view(np.uint32)
        a = np.asarray(src, dtype=np.float32).reshape(Hkv, src_max_len, d).view(np.uint32)
        b[slot, :, :seq_len, :] = a[:, :seq_len, :]
        out.append(b.view(np.float32))
    return tuple(out)
