"""Independent numpy fp64 formulation of the attention definitions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  A second formulation
of the same definitions as ``oracle.c``, written differently on purpose so the
two cannot share a mistake: heads are split with reshapes, each head's scores
are formed as one full matrix by a matrix product, the causal mask is a
lower-triangular (or position-compared) boolean mask, and the softmax is
taken over whole rows of the masked matrix.  The pins check it against
``oracle.c`` on every tiny shape and on medium ones; the GPU tests use it for
whole-output checks of large results, where its matrix products (BLAS, fp64)
and one worker thread per independent head make it fast enough.  Heads are
independent, so the thread count changes no result.

Definitions: trueno-gpu 0.4.11 ``src/memory/resident/attention.rs``,
``batched_multihead_attention`` (softmax(Q K^T / sqrt(d_k)) V per head over
interleaved [seq, n_heads*head_dim]); trustformers-core 0.2.0
``src/gpu_ops/cuda/oxicuda/attention.rs``, ``attention_prefill_gpu_to_gpu`` and
``softmax_causal_gpu_to_gpu`` (query i sees keys 0..=i, masked cells are 0);
realizar 0.8.5 ``src/cuda/executor/cache_from_cache_from_kv_cache.rs``,
``init_batched_kv_cache_gpu`` ([M, num_kv_heads, max_len, head_dim] caches).
"""
from __future__ import annotations

import itertools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_WORKERS = max(1, min(16, os.cpu_count() or 1))


def _softmax_rows(s: np.ndarray, visible: np.ndarray | None) -> np.ndarray:
    if visible is None:
        e = np.exp(s - s.max(axis=-1, keepdims=True))
    else:
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=-1, keepdims=True)
        e = np.where(visible, np.exp(s), 0.0)
    return e / e.sum(axis=-1, keepdims=True)


def _attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float,
            visible: np.ndarray | None) -> np.ndarray:
    """One head: softmax(scale * q keys^T, masked) vals, with q [n, d], keys and vals [L, d]."""
    s = scale * (q.astype(np.float64) @ keys.astype(np.float64).T)          # [n, L]
    return _softmax_rows(s, visible) @ vals.astype(np.float64)              # [n, d]


def _each(fn, units) -> None:
    """fn(u) for every independent unit u, on a pool of threads (BLAS kept to one thread each)."""
    units = list(units)
    if len(units) <= 1 or _WORKERS == 1:
        for u in units:
            fn(u)
        return
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(min(_WORKERS, len(units))) as ex:
        for _ in ex.map(fn, units):
            pass


def prefill(q, k, v, B, S, H, d, scale, causal):
    qh = np.asarray(q, dtype=np.float32).reshape(B, S, H, d)
    kh = np.asarray(k, dtype=np.float32).reshape(B, S, H, d)
    vh = np.asarray(v, dtype=np.float32).reshape(B, S, H, d)
    sc = float(np.float32(scale))
    visible = np.tril(np.ones((S, S), dtype=bool)) if causal else None
    out = np.empty((B, S, H, d))

    def unit(bh):
        b, h = bh
        out[b, :, h, :] = _attend(qh[b, :, h, :], kh[b, :, h, :], vh[b, :, h, :], sc, visible)

    _each(unit, itertools.product(range(B), range(H)))
    return out.reshape(B, S, H * d)


def decode(q, k_cache, v_cache, lens, M, H, Hkv, d, max_len, scale):
    g = H // Hkv
    qm = np.asarray(q, dtype=np.float32).reshape(M, H, d)
    kc = np.asarray(k_cache, dtype=np.float32).reshape(M, Hkv, max_len, d)
    vc = np.asarray(v_cache, dtype=np.float32).reshape(M, Hkv, max_len, d)
    sc = float(np.float32(scale))
    out = np.zeros((M, H, d))

    def unit(mh):
        m, h = mh
        L = int(lens[m])
        if L > 0:  # an empty sequence keeps its zeros
            out[m, h] = _attend(qm[m, h][None, :], kc[m, h // g, :L], vc[m, h // g, :L], sc, None)[0]

    _each(unit, itertools.product(range(M), range(H)))
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
    qm = np.asarray(q, dtype=np.float32).reshape(M, n_new, H, d)
    kn = np.asarray(k_new, dtype=np.float32).reshape(M, n_new, Hkv, d)
    vn = np.asarray(v_new, dtype=np.float32).reshape(M, n_new, Hkv, d)
    kc = np.asarray(k_cache, dtype=np.float32).reshape(M, Hkv, max_len, d)
    vc = np.asarray(v_cache, dtype=np.float32).reshape(M, Hkv, max_len, d)
    sc = float(np.float32(scale))
    out = np.empty((M, n_new, H, d))

    def unit(mh):
        m, h = mh
        P, kh = int(cache_lens[m]), h // g
        keys = np.concatenate([kc[m, kh, :P], kn[m, :, kh]], axis=0)                # [P+n, d]
        vals = np.concatenate([vc[m, kh, :P], vn[m, :, kh]], axis=0)
        visible = np.arange(P + n_new)[None, :] <= (P + np.arange(n_new))[:, None]  # [n, P+n]
        out[m, :, h, :] = _attend(qm[m, :, h, :], keys, vals, sc, visible)

    _each(unit, itertools.product(range(M), range(H)))
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
