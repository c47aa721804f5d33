"""Pins that tie the CPU oracle to facts fixed by the pages and by mathematics.

Each pin takes an ``oracle.Oracle`` (so the same checks can be re-run against
deliberately broken copies of the oracle, see test_oracle_mutants.py) and
raises AssertionError when the oracle disagrees with:

* closed forms (one-hot selection, uniform/prefix means, two-key softmax),
* invariants (rows of a softmax sum to one, linearity in V, permutation
  invariance, reads only the first L_m cache rows),
* relations the pages state (decode equals the last row of a causal prefill
  -- trustformers-core 0.2.0 src/gpu_ops/cuda/oxicuda/attention.rs,
  gpu_tests ``oxicuda_resident_decode_attention_parity``; an empty sequence
  gives zeros -- trueno-gpu 0.4.11 src/memory/resident/attention.rs,
  ``incremental_attention_gpu``),
* printed offsets (tests/golden/),
* the rotary embedding's closed forms (identity at position 0, unit-vector
  images, the frequency ladder, pair lengths, composition, dependence of
  scores on relative position only), and
* an independent numpy fp64 brute force on every tiny shape.
"""
from __future__ import annotations

import itertools
import json
import math
import os
import zlib

import numpy as np

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _scale(d):
    return float(np.float32(1.0) / np.sqrt(np.float32(d)))


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite output"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _rng(tag):
    return np.random.default_rng(zlib.crc32(tag.encode()))


def _build_cache_by_scatter(orc, k_rows, v_rows, Hkv, d, max_len, fill):
    """[1, S, Hkv*d] rows appended one position at a time into a [1, Hkv, max_len, d] cache."""
    S = k_rows.shape[1]
    kc = np.full((1, Hkv, max_len, d), fill, dtype=np.float32)
    vc = np.full((1, Hkv, max_len, d), fill, dtype=np.float32)
    for t in range(S):
        orc.scatter(np.ascontiguousarray(k_rows[:, t:t + 1]), np.ascontiguousarray(v_rows[:, t:t + 1]),
                    kc, vc, np.array([t], np.int32), 1, 1, Hkv, d, max_len)
    return kc, vc


# --------------------------------------------------------------------------- prefill


def pin_rows_sum_to_one(orc):
    """V = 1 everywhere gives O = sum_j p_j = 1 (softmax rows sum to one)."""
    r = _rng("rowsum")
    for causal in (False, True):
        B, S, H, d = 2, 7, 3, 5
        q = r.standard_normal((B, S, H * d)).astype(np.float32) * 3
        k = r.standard_normal((B, S, H * d)).astype(np.float32) * 3
        v = np.ones((B, S, H * d), np.float32)
        _close(orc.prefill(q, k, v, B, S, H, d, _scale(d), causal), v, 1e-12, f"row sum causal={causal}")
    M, H, Hkv, d, max_len = 3, 4, 2, 4, 9
    q = r.standard_normal((M, H * d)).astype(np.float32)
    kc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    vc = np.ones_like(kc)
    lens = np.array([1, 5, 9], np.int32)
    _close(orc.decode(q, kc, vc, lens, M, H, Hkv, d, max_len, _scale(d)), np.ones((M, H * d)), 1e-12,
           "decode row sum")


def _onehot_case(c_times_scale, causal):
    """Key j* = e_0, all other keys 0, every query c*e_0: scores c*scale at j*, 0 elsewhere."""
    B, S, H, d = 1, 6, 2, 4
    jstar = 3
    scale = _scale(d)
    c = np.float32(c_times_scale / scale)
    q = np.zeros((B, S, H, d), np.float32)
    q[..., 0] = c
    k = np.zeros((B, S, H, d), np.float32)
    k[:, jstar, :, 0] = 1.0
    v = _rng("onehot-v").standard_normal((B, S, H, d)).astype(np.float32)
    return B, S, H, d, jstar, scale, q.reshape(B, S, H * d), k.reshape(B, S, H * d), v


def pin_one_hot_selects_row(orc):
    """A dominant score reproduces the selected V row (error ~ S*e^-200)."""
    for causal in (False, True):
        B, S, H, d, jstar, scale, q, k, v = _onehot_case(200.0, causal)
        o = orc.prefill(q, k, v, B, S, H, d, scale, causal).reshape(B, S, H, d)
        v4 = v.reshape(B, S, H, d)
        for i in range(S):
            if causal and i < jstar:
                # Row i does not see j*: every visible score is 0 -> prefix mean.
                want = v4[0, : i + 1].astype(np.float64).mean(axis=0)
            else:
                want = v4[0, jstar]
            _close(o[0, i], want, 1e-12, f"one-hot row {i} causal={causal}")


def pin_large_logits_stay_finite(orc):
    """Scores of 1000 overflow exp() in double unless the row max is subtracted first."""
    for causal in (False, True):
        B, S, H, d, jstar, scale, q, k, v = _onehot_case(1000.0, causal)
        o = orc.prefill(q, k, v, B, S, H, d, scale, causal).reshape(B, S, H, d)
        v4 = v.reshape(B, S, H, d)
        _close(o[0, S - 1], v4[0, jstar], 1e-12, f"large logits causal={causal}")


def pin_uniform_prefix_mean(orc):
    """q = 0: all visible scores equal -> mean of visible V rows (prefix mean when causal)."""
    r = _rng("uniform")
    B, S, H, d = 2, 9, 3, 4
    q = np.zeros((B, S, H * d), np.float32)
    k = r.standard_normal((B, S, H * d)).astype(np.float32)
    v = r.standard_normal((B, S, H * d)).astype(np.float32)
    v64 = v.astype(np.float64)
    o = orc.prefill(q, k, v, B, S, H, d, _scale(d), False)
    _close(o, np.broadcast_to(v64.mean(axis=1, keepdims=True), o.shape), 1e-12, "uniform non-causal")
    o = orc.prefill(q, k, v, B, S, H, d, _scale(d), True)
    prefix = np.cumsum(v64, axis=1) / np.arange(1, S + 1)[None, :, None]
    _close(o, prefix, 1e-12, "uniform causal prefix mean")


def pin_two_key_closed_form(orc):
    """d = 1, S = 2, causal: o_0 = v_0; o_1 = sigmoid(s11 - s10) v_1 + sigmoid(s10 - s11) v_0."""
    q = np.array([[[0.7], [-1.3]]], np.float32)
    k = np.array([[[0.4], [1.9]]], np.float32)
    v = np.array([[[2.5], [-0.75]]], np.float32)
    scale = np.float32(0.8)
    o = orc.prefill(q, k, v, 1, 2, 1, 1, float(scale), True)
    s10 = float(scale) * float(q[0, 1, 0]) * float(k[0, 0, 0])
    s11 = float(scale) * float(q[0, 1, 0]) * float(k[0, 1, 0])
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    want1 = sig(s11 - s10) * float(v[0, 1, 0]) + sig(s10 - s11) * float(v[0, 0, 0])
    _close(o[0, 0, 0], float(v[0, 0, 0]), 1e-15, "two-key row 0")
    _close(o[0, 1, 0], want1, 1e-14, "two-key row 1")
    # Non-causal: row 0 now also sees key 1.
    o = orc.prefill(q, k, v, 1, 2, 1, 1, float(scale), False)
    s00 = float(scale) * float(q[0, 0, 0]) * float(k[0, 0, 0])
    s01 = float(scale) * float(q[0, 0, 0]) * float(k[0, 1, 0])
    want0 = sig(s01 - s00) * float(v[0, 1, 0]) + sig(s00 - s01) * float(v[0, 0, 0])
    _close(o[0, 0, 0], want0, 1e-14, "two-key non-causal row 0")


def pin_linear_in_v(orc):
    """O(Q, K, a V + b W) = a O(Q, K, V) + b O(Q, K, W); constant V rows give that constant."""
    r = _rng("linear")
    B, S, H, d = 1, 8, 2, 6
    q, k, v, w = (r.standard_normal((B, S, H * d)).astype(np.float32) for _ in range(4))
    # Disjoint column supports and power-of-two weights keep a*v + b*w exact in f32.
    v[..., 1::2] = 0.0
    w[..., 0::2] = 0.0
    a, b = np.float32(0.5), np.float32(-2.0)
    for causal in (False, True):
        lhs = orc.prefill(q, k, (a * v + b * w).astype(np.float32), B, S, H, d, _scale(d), causal)
        rhs = float(a) * orc.prefill(q, k, v, B, S, H, d, _scale(d), causal) + \
            float(b) * orc.prefill(q, k, w, B, S, H, d, _scale(d), causal)
        _close(lhs, rhs, 1e-12, f"linearity causal={causal}")
        const = np.full((B, S, H * d), 3.25, np.float32)
        _close(orc.prefill(q, k, const, B, S, H, d, _scale(d), causal), const, 1e-12, "constant V")


def pin_permutation(orc):
    """Non-causal: jointly permuting K and V rows changes nothing; permuting Q permutes O."""
    r = _rng("perm")
    B, S, H, d = 1, 10, 2, 4
    q, k, v = (r.standard_normal((B, S, H * d)).astype(np.float32) for _ in range(3))
    perm = r.permutation(S)
    o = orc.prefill(q, k, v, B, S, H, d, _scale(d), False)
    _close(orc.prefill(q, k[:, perm], v[:, perm], B, S, H, d, _scale(d), False), o, 1e-12,
           "joint K/V permutation")
    _close(orc.prefill(q[:, perm], k, v, B, S, H, d, _scale(d), False), o[:, perm], 1e-12,
           "query permutation")


def pin_heads_and_batches_independent(orc):
    """Each (b, h) output depends only on that batch element's head-h columns."""
    r = _rng("indep")
    B, S, H, d = 2, 5, 3, 4
    q, k, v = (r.standard_normal((B, S, H * d)).astype(np.float32) for _ in range(3))
    o = orc.prefill(q, k, v, B, S, H, d, _scale(d), True)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    # Perturb head 1 of batch 0 only.
    for t in (q2, k2, v2):
        t[0, :, d:2 * d] += 1.0
    o2 = orc.prefill(q2, k2, v2, B, S, H, d, _scale(d), True)
    mask = np.ones((B, S, H * d), bool)
    mask[0, :, d:2 * d] = False
    _close(o2[mask], o[mask], 0.0, "untouched heads unchanged")
    assert np.max(np.abs(o2[0, :, d:2 * d] - o[0, :, d:2 * d])) > 1e-3, "perturbed head must change"


def pin_prefill_rows_match(orc):
    """The sampled-row entry point equals the full computation at those rows."""
    r = _rng("rows")
    B, S, H, d = 2, 11, 3, 4
    q, k, v = (r.standard_normal((B, S, H * d)).astype(np.float32) for _ in range(3))
    for causal in (False, True):
        full = orc.prefill(q, k, v, B, S, H, d, _scale(d), causal)
        sel = np.array([[0, 0, 0], [1, 10, 2], [0, 5, 1], [1, 3, 0]], np.int64)
        rows = orc.prefill_rows(q, k, v, sel, B, S, H, d, _scale(d), causal)
        want = np.stack([full[b, i, h * d:(h + 1) * d] for b, i, h in sel])
        _close(rows, want, 0.0, f"prefill_rows causal={causal}")


# --------------------------------------------------------------------------- decode


def pin_decode_equals_causal_prefill_row(orc):
    """Decode at step t over a cache filled by appends equals row t of a causal prefill."""
    r = _rng("dec=pre")
    S, H, d, max_len = 6, 3, 4, 8
    q, k, v = (r.standard_normal((1, S, H * d)).astype(np.float32) for _ in range(3))
    pre = orc.prefill(q, k, v, 1, S, H, d, _scale(d), True)
    kc, vc = _build_cache_by_scatter(orc, k, v, H, d, max_len, np.nan)
    for t in range(S):
        # Cache holds rows 0..S-1; attending over L = t+1 reads rows 0..t only.
        out = orc.decode(np.ascontiguousarray(q[:, t]), kc, vc, np.array([t + 1], np.int32),
                         1, H, H, d, max_len, _scale(d))
        _close(out[0], pre[0, t], 1e-12, f"decode step {t}")


def pin_gqa_head_map(orc):
    """Query head h reads KV head floor(h / (H/Hkv)): V rows of KV head kh hold kh+1."""
    r = _rng("gqa-map")
    M, H, Hkv, d, max_len = 2, 8, 2, 4, 5
    q = r.standard_normal((M, H * d)).astype(np.float32)
    kc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    vc = np.zeros_like(kc)
    for kh in range(Hkv):
        vc[:, kh] = kh + 1
    out = orc.decode(q, kc, vc, np.array([5, 3], np.int32), M, H, Hkv, d, max_len, _scale(d))
    g = H // Hkv
    want = np.repeat((np.arange(H) // g + 1).astype(np.float64), d)[None].repeat(M, axis=0)
    _close(out, want, 1e-12, "GQA head map")


def pin_gqa_equals_mha_on_repeated_cache(orc):
    """GQA over Hkv heads equals MHA (Hkv = H) over a cache with each KV head repeated g times."""
    r = _rng("gqa=mha")
    M, H, Hkv, d, max_len = 3, 6, 2, 4, 7
    q = r.standard_normal((M, H * d)).astype(np.float32)
    kc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    vc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    lens = np.array([7, 1, 4], np.int32)
    g = H // Hkv
    gqa = orc.decode(q, kc, vc, lens, M, H, Hkv, d, max_len, _scale(d))
    mha = orc.decode(q, np.ascontiguousarray(np.repeat(kc, g, axis=1)),
                     np.ascontiguousarray(np.repeat(vc, g, axis=1)), lens, M, H, H, d, max_len, _scale(d))
    _close(gqa, mha, 0.0, "GQA vs repeated-cache MHA")


def pin_decode_reads_only_live_rows(orc):
    """Rows at positions >= L_m (NaN / 1e30 here) and other sequences never reach out[m]."""
    r = _rng("live")
    M, H, Hkv, d, max_len = 3, 4, 2, 4, 10
    q = r.standard_normal((M, H * d)).astype(np.float32)
    kc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    vc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    lens = np.array([4, 10, 1], np.int32)
    base = orc.decode(q, kc, vc, lens, M, H, Hkv, d, max_len, _scale(d))
    for fill in (np.nan, 1e30):
        kc2, vc2 = kc.copy(), vc.copy()
        for m in range(M):
            kc2[m, :, lens[m]:] = fill
            vc2[m, :, lens[m]:] = fill
        _close(orc.decode(q, kc2, vc2, lens, M, H, Hkv, d, max_len, _scale(d)), base, 0.0,
               f"rows beyond L filled with {fill}")
    kc3 = kc.copy()
    kc3[1] += 5.0
    o3 = orc.decode(q, kc3, vc, lens, M, H, Hkv, d, max_len, _scale(d))
    _close(o3[[0, 2]], base[[0, 2]], 0.0, "other sequences unchanged")


def pin_empty_sequence_gives_zeros(orc):
    """L_m = 0 yields zeros for that sequence only."""
    r = _rng("empty")
    M, H, Hkv, d, max_len = 2, 2, 1, 4, 3
    q = r.standard_normal((M, H * d)).astype(np.float32)
    kc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    vc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    out = orc.decode(q, kc, vc, np.array([0, 2], np.int32), M, H, Hkv, d, max_len, _scale(d))
    _close(out[0], np.zeros(H * d), 0.0, "empty sequence")
    assert np.max(np.abs(out[1])) > 0


def pin_decode_rows_match(orc):
    r = _rng("decrows")
    M, H, Hkv, d, max_len = 3, 8, 4, 4, 6
    q = r.standard_normal((M, H * d)).astype(np.float32)
    kc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    vc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    lens = np.array([6, 0, 3], np.int32)
    full = orc.decode(q, kc, vc, lens, M, H, Hkv, d, max_len, _scale(d))
    sel = np.array([[0, 7], [1, 0], [2, 3], [2, 4]], np.int64)
    rows = orc.decode_rows(q, kc, vc, lens, sel, M, H, Hkv, d, max_len, _scale(d))
    _close(rows, np.stack([full[m, h * d:(h + 1) * d] for m, h in sel]), 0.0, "decode_rows")


# --------------------------------------------------------------------------- chunked prefill behind a cache


def _cached_case(r, M, n_new, H, Hkv, d, max_len, lens):
    q = r.standard_normal((M, n_new, H * d)).astype(np.float32)
    kn = r.standard_normal((M, n_new, Hkv * d)).astype(np.float32)
    vn = r.standard_normal((M, n_new, Hkv * d)).astype(np.float32)
    kc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    vc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    for m in range(M):  # rows at or past P are not part of the cache yet
        kc[m, :, lens[m]:] = np.nan
        vc[m, :, lens[m]:] = np.nan
    return q, kn, vn, kc, vc


def pin_cached_from_empty_is_causal_prefill(orc):
    """With nothing cached (P = 0) and Hkv = H, a chunk is a plain causal prefill."""
    r = _rng("cached-empty")
    M, n, H, d, max_len = 2, 7, 3, 4, 9
    lens = np.zeros(M, np.int32)
    q, kn, vn, kc, vc = _cached_case(r, M, n, H, H, d, max_len, lens)
    got = orc.prefill_cached(q, kn, vn, kc, vc, lens, M, n, H, H, d, max_len, _scale(d))
    _close(got, orc.prefill(q, kn, vn, M, n, H, d, _scale(d), True), 1e-13, "P=0 chunk vs causal prefill")


def pin_cached_single_token_is_decode(orc):
    """A one-token chunk behind P cached rows is a decode over the appended cache (L = P + 1)."""
    r = _rng("cached-one")
    M, H, Hkv, d, max_len = 3, 8, 2, 4, 10
    lens = np.array([0, 4, 9], np.int32)
    q, kn, vn, kc, vc = _cached_case(r, M, 1, H, Hkv, d, max_len, lens)
    got = orc.prefill_cached(q, kn, vn, kc, vc, lens, M, 1, H, Hkv, d, max_len, _scale(d))
    kc2, vc2 = kc.copy(), vc.copy()
    orc.scatter(kn, vn, kc2, vc2, lens, M, 1, Hkv, d, max_len)
    want = orc.decode(q.reshape(M, H * d), kc2, vc2, lens + 1, M, H, Hkv, d, max_len, _scale(d))
    _close(got.reshape(M, H * d), want, 1e-13, "one-token chunk vs decode")


def pin_cached_chunks_compose(orc):
    """Prefilling S tokens in two chunks (the second behind the first's appended rows) equals one causal prefill."""
    r = _rng("cached-compose")
    M, S, s1, H, Hkv, d, max_len = 2, 9, 4, 6, 3, 4, 12
    zero = np.zeros(M, np.int32)
    q, kn, vn, kc, vc = _cached_case(r, M, S, H, Hkv, d, max_len, zero)
    whole = orc.prefill_cached(q, kn, vn, kc, vc, zero, M, S, H, Hkv, d, max_len, _scale(d))
    first = orc.prefill_cached(np.ascontiguousarray(q[:, :s1]), np.ascontiguousarray(kn[:, :s1]),
                               np.ascontiguousarray(vn[:, :s1]), kc, vc, zero, M, s1, H, Hkv, d, max_len, _scale(d))
    kc2, vc2 = kc.copy(), vc.copy()
    orc.scatter(np.ascontiguousarray(kn[:, :s1]), np.ascontiguousarray(vn[:, :s1]), kc2, vc2, zero, M, s1, Hkv, d,
                max_len)
    second = orc.prefill_cached(np.ascontiguousarray(q[:, s1:]), np.ascontiguousarray(kn[:, s1:]),
                                np.ascontiguousarray(vn[:, s1:]), kc2, vc2, np.full(M, s1, np.int32), M, S - s1, H,
                                Hkv, d, max_len, _scale(d))
    _close(np.concatenate([first, second], axis=1), whole, 1e-13, "two chunks vs one")


def pin_cached_brute_force(orc):
    """C oracle == numpy concatenate-and-mask formulation on ragged cache lengths and GQA groups."""
    r = _rng("cached-brute")
    for M, n, H, Hkv, d, max_len in [(3, 5, 4, 2, 3, 9), (2, 1, 6, 3, 4, 6), (4, 3, 2, 1, 2, 7), (1, 6, 3, 3, 5, 6)]:
        lens = r.integers(0, max_len - n + 1, size=M).astype(np.int32)
        q, kn, vn, kc, vc = _cached_case(r, M, n, H, Hkv, d, max_len, lens)
        _close(orc.prefill_cached(q, kn, vn, kc, vc, lens, M, n, H, Hkv, d, max_len, _scale(d)),
               brute.prefill_cached(q, kn, vn, np.nan_to_num(kc), np.nan_to_num(vc), lens, M, n, H, Hkv, d, max_len,
                                    _scale(d)), 1e-12, f"cached brute {M, n, H, Hkv, d}")


def _rotated_rows(orc, x, pos, heads, d, rot, base):
    """Rows [n, heads*d] turned to positions pos by the oracle's own rotation, handed over as f32."""
    return orc.rope(np.ascontiguousarray(x, np.float32).reshape(len(pos), heads * d), np.asarray(pos, np.int32),
                    heads, d, rot, base).astype(np.float32)


def pin_cached_rope_zero_width_is_plain(orc):
    """rotary_ndims = 0 rotates nothing: the plain chunked prefill, exactly."""
    r = _rng("cached-rope-zero")
    M, n, H, Hkv, d, max_len = 3, 5, 4, 2, 8, 16
    lens = np.array([0, 7, 11], np.int32)
    q, kn, vn, kc, vc = _cached_case(r, M, n, H, Hkv, d, max_len, lens)
    _close(orc.prefill_cached_rope(q, kn, vn, kc, vc, lens, M, n, H, Hkv, d, max_len, _scale(d), 0, 1e4),
           orc.prefill_cached(q, kn, vn, kc, vc, lens, M, n, H, Hkv, d, max_len, _scale(d)), 0.0, "rotary width 0")


def pin_cached_rope_chunks_compose(orc):
    """Two rotary chunks equal one: the first chunk's keys appended rotated to rows 0..P-1, the second chunk
    behind them must turn its queries and keys to P + r (not r) to match the whole sequence from empty."""
    r = _rng("cached-rope-chunks")
    for M, S, P, H, Hkv, d, rot, base in [(2, 12, 7, 4, 2, 8, 8, 100.0), (1, 9, 4, 2, 2, 16, 8, 10.0)]:
        max_len = S + 3
        q = r.standard_normal((M, S, H * d)).astype(np.float32)
        kn = r.standard_normal((M, S, Hkv * d)).astype(np.float32)
        vn = r.standard_normal((M, S, Hkv * d)).astype(np.float32)
        empty = np.full((M, Hkv, max_len, d), np.nan, np.float32)
        zero = np.zeros(M, np.int32)
        whole = orc.prefill_cached_rope(q, kn, vn, empty, empty, zero, M, S, H, Hkv, d, max_len, _scale(d), rot, base)
        pos = np.tile(np.arange(P), M)
        k_rot = _rotated_rows(orc, kn[:, :P], pos, Hkv, d, rot, base).reshape(M, P, Hkv * d)
        kc, vc = empty.copy(), empty.copy()
        orc.scatter(k_rot, np.ascontiguousarray(vn[:, :P]), kc, vc, zero, M, P, Hkv, d, max_len)
        second = orc.prefill_cached_rope(np.ascontiguousarray(q[:, P:]), np.ascontiguousarray(kn[:, P:]),
                                         np.ascontiguousarray(vn[:, P:]), kc, vc, np.full(M, P, np.int32), M, S - P,
                                         H, Hkv, d, max_len, _scale(d), rot, base)
        _close(second, whole[:, P:], 1e-13, f"rotary chunk behind {P} vs whole")


def pin_cached_rope_single_token_is_rotary_decode(orc):
    """One new token behind P rotated keys: its query turned to position P, its key appended rotated to row
    P, then the plain decode over P + 1 keys."""
    r = _rng("cached-rope-decode")
    M, H, Hkv, d, max_len, rot, base = 3, 6, 2, 16, 20, 16, 1000.0
    lens = np.array([0, 5, 19], np.int32)
    q, kn, vn, kc, vc = _cached_case(r, M, 1, H, Hkv, d, max_len, lens)
    got = orc.prefill_cached_rope(q, kn, vn, kc, vc, lens, M, 1, H, Hkv, d, max_len, _scale(d), rot, base)
    kc2, vc2 = kc.copy(), vc.copy()
    orc.scatter(_rotated_rows(orc, kn, lens, Hkv, d, rot, base).reshape(M, 1, Hkv * d), vn, kc2, vc2, lens, M, 1,
                Hkv, d, max_len)
    q_rot = _rotated_rows(orc, q, lens, H, d, rot, base)
    want = orc.decode(q_rot, kc2, vc2, lens + 1, M, H, Hkv, d, max_len, _scale(d))
    _close(got.reshape(M, H * d), want, 1e-13, "rotary single token vs rotary decode")


def pin_cached_rope_brute_force(orc):
    """C composition == numpy rotation (complex multiplication) + numpy chunked prefill."""
    r = _rng("cached-rope-brute")
    for M, n, H, Hkv, d, max_len, rot, base in [(3, 4, 4, 2, 8, 12, 8, 10000.0), (2, 6, 3, 3, 16, 9, 16, 50.0)]:
        lens = r.integers(0, max_len - n + 1, size=M).astype(np.int32)
        q, kn, vn, kc, vc = _cached_case(r, M, n, H, Hkv, d, max_len, lens)
        pos = (lens[:, None] + np.arange(n)[None, :]).reshape(-1)
        qb = brute.rope(q.reshape(M * n, H * d), pos, H, d, rot, base).astype(np.float32).reshape(q.shape)
        kb = brute.rope(kn.reshape(M * n, Hkv * d), pos, Hkv, d, rot, base).astype(np.float32).reshape(kn.shape)
        _close(orc.prefill_cached_rope(q, kn, vn, kc, vc, lens, M, n, H, Hkv, d, max_len, _scale(d), rot, base),
               brute.prefill_cached(qb, kb, vn, np.nan_to_num(kc), np.nan_to_num(vc), lens, M, n, H, Hkv, d,
                                    max_len, _scale(d)), 1e-9, f"rotary chunk brute {M, n, H, Hkv, d}")


def pin_cached_rows_match(orc):
    """The sampled-row entry point of the chunked prefill equals the full computation."""
    r = _rng("cached-rows")
    M, n, H, Hkv, d, max_len = 3, 6, 4, 2, 4, 12
    lens = np.array([0, 5, 6], np.int32)
    q, kn, vn, kc, vc = _cached_case(r, M, n, H, Hkv, d, max_len, lens)
    full = orc.prefill_cached(q, kn, vn, kc, vc, lens, M, n, H, Hkv, d, max_len, _scale(d))
    sel = np.array([[0, 0, 0], [2, 5, 3], [1, 2, 1], [1, 5, 2]], np.int64)
    rows = orc.prefill_cached_rows(q, kn, vn, kc, vc, lens, sel, M, n, H, Hkv, d, max_len, _scale(d))
    _close(rows, np.stack([full[m, i, h * d:(h + 1) * d] for m, i, h in sel]), 0.0, "prefill_cached_rows")


# --------------------------------------------------------------------------- brute force


def pin_brute_force_tiny_shapes(orc):
    """C oracle == independent numpy fp64 on every S<=5, d<=4, H<=4, Hkv | H."""
    r = _rng("brute")
    for S, d, H in itertools.product(range(1, 6), range(1, 5), range(1, 5)):
        B = 2
        q, k, v = (r.standard_normal((B, S, H * d)).astype(np.float32) * 2 for _ in range(3))
        for causal in (False, True):
            _close(orc.prefill(q, k, v, B, S, H, d, _scale(d), causal),
                   brute.prefill(q, k, v, B, S, H, d, _scale(d), causal), 1e-12,
                   f"brute prefill S={S} d={d} H={H} causal={causal}")
        for Hkv in [x for x in range(1, H + 1) if H % x == 0]:
            M, max_len = 3, 5
            qd = r.standard_normal((M, H * d)).astype(np.float32) * 2
            kc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
            vc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
            lens = r.integers(0, max_len + 1, size=M).astype(np.int32)
            _close(orc.decode(qd, kc, vc, lens, M, H, Hkv, d, max_len, _scale(d)),
                   brute.decode(qd, kc, vc, lens, M, H, Hkv, d, max_len, _scale(d)), 1e-12,
                   f"brute decode H={H} Hkv={Hkv} d={d}")


def pin_brute_force_medium_shapes(orc):
    """C oracle == the numpy formulation where it runs head by head on worker threads: many heads,
    hundreds of keys, ragged lengths, GQA groups, both masks and a cache behind a chunk."""
    r = _rng("brute-medium")
    B, S, H, d = 2, 150, 5, 64
    q, k, v = (r.standard_normal((B, S, H * d)).astype(np.float32) for _ in range(3))
    for causal in (False, True):
        _close(orc.prefill(q, k, v, B, S, H, d, _scale(d), causal),
               brute.prefill(q, k, v, B, S, H, d, _scale(d), causal), 1e-12, f"brute medium prefill causal={causal}")
    M, H, Hkv, d, max_len = 4, 12, 3, 32, 400
    lens = np.array([0, 1, 257, 400], np.int32)
    qd = r.standard_normal((M, H * d)).astype(np.float32)
    kc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    vc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    _close(orc.decode(qd, kc, vc, lens, M, H, Hkv, d, max_len, _scale(d)),
           brute.decode(qd, kc, vc, lens, M, H, Hkv, d, max_len, _scale(d)), 1e-12, "brute medium decode")
    M, n, H, Hkv, d, max_len = 3, 40, 8, 2, 32, 300
    lens = np.array([0, 133, 260], np.int32)
    q, kn, vn, kc, vc = _cached_case(r, M, n, H, Hkv, d, max_len, lens)
    _close(orc.prefill_cached(q, kn, vn, kc, vc, lens, M, n, H, Hkv, d, max_len, _scale(d)),
           brute.prefill_cached(q, kn, vn, kc, vc, lens, M, n, H, Hkv, d, max_len, _scale(d)), 1e-12,
           "brute medium chunk behind a cache")


def pin_pages_inputs_brute(orc):
    """The pages' deterministic test inputs (sin/cos/linear ramps) agree with the brute force.

    trustformers-core 0.2.0 ..., gpu_tests: prefill q = sin(0.37 i), k = cos(0.53 i),
    v = 0.25 i - 1 with H=2, seq=3, d=2; decode q = sin(0.41 i), k = cos(0.29 i),
    v = 1.5 - 0.2 i.  The page prints no expected values, so these are cross-checks
    against the independent formulation only (heads-major [H, seq, d] there, so the
    arrays are re-laid out to interleaved [seq, H*d] here).
    """
    H, S, d = 2, 3, 2
    i = np.arange(H * S * d, dtype=np.float32)
    def interleave(x):
        return np.ascontiguousarray(x.reshape(H, S, d).transpose(1, 0, 2).reshape(1, S, H * d))
    for qf, kf, vf in [(np.sin(i * np.float32(0.37)), np.cos(i * np.float32(0.53)), i * np.float32(0.25) - 1),
                       (np.sin(i * np.float32(0.41)), np.cos(i * np.float32(0.29)), np.float32(1.5) - i * np.float32(0.2))]:
        q, k, v = (interleave(x.astype(np.float32)) for x in (qf, kf, vf))
        _close(orc.prefill(q, k, v, 1, S, H, d, _scale(d), True),
               brute.prefill(q, k, v, 1, S, H, d, _scale(d), True), 1e-13, "pages' inputs")


# --------------------------------------------------------------------------- scatter


def pin_scatter_printed_offsets(orc):
    """Append offsets printed on the page (tests/golden/kv_append_offsets.json)."""
    g = json.load(open(os.path.join(GOLDEN, "kv_append_offsets.json")))
    Hkv, kv_old, kv_new, d = g["num_heads"], g["kv_old"], g["kv_new"], g["head_dim"]
    max_len = kv_old + kv_new
    # Old rows first (positions 0..kv_old-1), marked with 1000 + source index.
    old = (1000 + np.arange(kv_old * Hkv * d, dtype=np.float32)).reshape(1, kv_old, Hkv * d)
    new = np.arange(kv_new * Hkv * d, dtype=np.float32).reshape(1, kv_new, Hkv * d)
    kc = np.full((1, Hkv, max_len, d), -1.0, np.float32)
    vc = kc.copy()
    orc.scatter(old, old, kc, vc, np.array([0], np.int32), 1, kv_old, Hkv, d, max_len)
    orc.scatter(new, new, kc, vc, np.array([kv_old], np.int32), 1, kv_new, Hkv, d, max_len)
    flat = kc.reshape(-1)
    for h, (src, dst) in enumerate(g["new_src_dst"]):
        assert np.array_equal(flat[dst:dst + d], new.reshape(-1)[src:src + d]), f"new row head {h}"
    for h, (_, dst) in enumerate(g["old_src_dst"]):
        # Old row 0 of head h sits at the printed destination.
        assert np.array_equal(flat[dst:dst + d], old[0, 0, h * d:(h + 1) * d]), f"old row head {h}"
    assert not np.any(flat == -1.0), "every position of the appended cache is written"
    assert np.array_equal(kc, vc)


def pin_scatter_layout_offsets(orc):
    """Slot stride and head-0 position offsets (tests/golden/kv_cache_layout.json)."""
    g = json.load(open(os.path.join(GOLDEN, "kv_cache_layout.json")))
    for c in g["cases"]:
        Hkv, max_len, d, slot, head, pos = (c[x] for x in ("num_kv_heads", "max_len", "head_dim", "slot", "head", "pos"))
        M = slot + 1
        src = np.zeros((M, 1, Hkv * d), np.float32)
        marker = np.arange(1, d + 1, dtype=np.float32)
        src[slot, 0, head * d:(head + 1) * d] = marker
        kc = np.zeros((M, Hkv, max_len, d), np.float32)
        vc = kc.copy()
        lens = np.zeros(M, np.int32)
        lens[slot] = pos
        orc.scatter(src, src, kc, vc, lens, M, 1, Hkv, d, max_len)
        flat = kc.reshape(-1)
        assert np.array_equal(flat[c["offset"]:c["offset"] + d], marker), f"case {c}"
        assert np.count_nonzero(flat) == d


def pin_scatter_matches_fancy_index(orc):
    """Bit-exact agreement with a numpy fancy-index append; untouched sentinel bytes stay."""
    r = _rng("scatter")
    for M, n_new, Hkv, d, max_len in [(3, 4, 2, 8, 9), (1, 1, 1, 4, 1), (4, 2, 3, 4, 6)]:
        kn = r.standard_normal((M, n_new, Hkv * d)).astype(np.float32)
        vn = r.standard_normal((M, n_new, Hkv * d)).astype(np.float32)
        kn.view(np.uint32)[0, 0, 0] = 0x7FA00001  # a NaN payload must survive bit for bit
        lens = r.integers(0, max_len - n_new + 1, size=M).astype(np.int32)
        sent = np.full((M, Hkv, max_len, d), 0x7FC0DEAD, np.uint32).view(np.float32)
        kc, vc = sent.copy(), sent.copy()
        orc.scatter(kn, vn, kc, vc, lens, M, n_new, Hkv, d, max_len)
        bk, bv = brute.scatter(kn, vn, sent, sent, lens, M, n_new, Hkv, d, max_len)
        assert np.array_equal(kc.view(np.uint32), bk.reshape(kc.shape).view(np.uint32))
        assert np.array_equal(vc.view(np.uint32), bv.reshape(vc.shape).view(np.uint32))
        written = M * n_new * Hkv * d
        assert np.count_nonzero(kc.view(np.uint32) != 0x7FC0DEAD) == written


def pin_scatter_rejects_overflow(orc):
    """A write at or past max_len is refused and leaves the caches untouched."""
    kn = np.ones((1, 2, 4), np.float32)
    kc = np.zeros((1, 1, 3, 4), np.float32)
    vc = kc.copy()
    try:
        orc.scatter(kn, kn, kc, vc, np.array([2], np.int32), 1, 2, 1, 4, 3)
    except ValueError:
        pass
    else:
        raise AssertionError("append past max_len accepted")
    assert not kc.any() and not vc.any()


# --------------------------------------------------------------------------- reduced precision
#
# trueno-gpu 0.4.11 ..., ``batched_gemm``: for k >= 64 the attention GEMMs run on
# fp16 tensor-core operands.  Reading: the reduced-precision prefill is the
# attention of the inputs rounded (nearest, ties to even) to the 16-bit format.


def _bf16_by_bits(x):
    """bfloat16 rounding by integer arithmetic on the f32 bit pattern (finite inputs)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def _rounding_samples():
    r = _rng("round16")
    parts = [r.standard_normal(20000) * s for s in (1e-6, 1e-3, 1.0, 30.0, 3e4)]
    parts.append(r.uniform(-7e4, 7e4, 5000))
    # Ties and near-ties at several binades, both formats' subnormals, overflow edges.
    ties = []
    for e in range(-30, 20):
        base = 2.0 ** e
        for m in range(1, 9):
            ties += [base * (1 + m * 2.0 ** -11), base * (1 + (2 * m + 1) * 2.0 ** -12),
                     base * (1 + (2 * m + 1) * 2.0 ** -9), base * (1 + m * 2.0 ** -8)]
    parts.append(np.array(ties))
    parts.append(np.array([0.0, -0.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 65504, 65519.99, 65520,
                           -65520, 3.0e38, 3.4e38, 2.0 ** -126, 2.0 ** -133, 2.0 ** -134, 1e-40]))
    x = np.concatenate(parts).astype(np.float32)
    return np.concatenate([x, -x])


def pin_round16_binary16_matches_numpy(orc):
    """binary16 rounding equals numpy's float16 conversion (its own implementation), value by value."""
    x = _rounding_samples()
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).astype(np.float32)
    got = orc.round16(x, orc.FP16)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
        f"{np.count_nonzero(got.view(np.uint32) != want.view(np.uint32))} values differ"


def pin_round16_bfloat16_matches_bit_rounding(orc):
    """bfloat16 rounding equals round-to-nearest-even on the f32 bit pattern (a second formulation)."""
    x = _rounding_samples()
    got = orc.round16(x, orc.BF16)
    want = _bf16_by_bits(x)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), \
        f"{np.count_nonzero(got.view(np.uint32) != want.view(np.uint32))} values differ"


def pin_round16_hand_cases(orc):
    """Ties go to even, subnormals keep their spacing, overflow goes to infinity, NaN stays NaN."""
    cases = [
        (orc.BF16, 1 + 2.0 ** -8, 1.0), (orc.BF16, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6),
        (orc.BF16, 1 + 2.0 ** -7, 1 + 2.0 ** -7), (orc.BF16, 2.0 ** -133, 2.0 ** -133),
        (orc.BF16, 3.4e38, np.inf), (orc.BF16, -(2 - 2.0 ** -7) * 2.0 ** 127, -(2 - 2.0 ** -7) * 2.0 ** 127),
        (orc.FP16, 1 + 2.0 ** -11, 1.0), (orc.FP16, 1 + 3 * 2.0 ** -11, 1 + 2.0 ** -9),
        (orc.FP16, 65519.0, 65504.0), (orc.FP16, 65520.0, np.inf), (orc.FP16, -65520.0, -np.inf),
        (orc.FP16, 2.0 ** -25, 0.0), (orc.FP16, 3 * 2.0 ** -26, 2.0 ** -24), (orc.FP16, 2.0 ** -24, 2.0 ** -24),
        (orc.FP16, 0.1, 0.0999755859375), (orc.BF16, 0.1, 0.10009765625),
    ]
    for fmt, x, want in cases:
        got = float(orc.round16(np.array([x], np.float32), fmt)[0])
        assert got == np.float32(want), f"fmt {fmt}: {x!r} -> {got!r}, want {want!r}"
    for fmt in (orc.FP16, orc.BF16):
        assert np.isnan(orc.round16(np.array([np.nan], np.float32), fmt)[0])
        x = _rounding_samples()
        once = orc.round16(x, fmt)
        with np.errstate(invalid="ignore"):
            assert np.array_equal(orc.round16(once, fmt).view(np.uint32), once.view(np.uint32)), "not idempotent"


def pin_prefill_lowp_is_prefill_of_rounded_inputs(orc):
    """Exactly the plain attention of the rounded inputs (brute force on numpy-rounded fp16 inputs too),
    and equal to plain attention when the inputs are already representable."""
    r = _rng("lowp")
    for B, S, H, d, causal in [(1, 7, 2, 8, True), (2, 5, 3, 4, False), (1, 9, 1, 16, True)]:
        q, k, v = (r.standard_normal((B, S, H * d)).astype(np.float32) for _ in range(3))
        for fmt in (orc.FP16, orc.BF16):
            got = orc.prefill_lowp(q, k, v, B, S, H, d, _scale(d), causal, fmt)
            rq, rk, rv = (orc.round16(x, fmt) for x in (q, k, v))
            _close(got, orc.prefill(rq, rk, rv, B, S, H, d, _scale(d), causal), 0.0, f"lowp fmt {fmt}")
        hq, hk, hv = (x.astype(np.float16).astype(np.float32) for x in (q, k, v))
        _close(orc.prefill_lowp(q, k, v, B, S, H, d, _scale(d), causal, orc.FP16),
               brute.prefill(hq, hk, hv, B, S, H, d, _scale(d), causal), 1e-12, "lowp fp16 brute")
        g = (np.round(r.standard_normal((B, S, H * d)) * 8) / 8).astype(np.float32)  # exact in both formats
        _close(orc.prefill_lowp(g, g, g, B, S, H, d, _scale(d), causal, orc.BF16),
               orc.prefill(g, g, g, B, S, H, d, _scale(d), causal), 0.0, "representable inputs")


# --------------------------------------------------------------------------- slot copy
#
# realizar 0.8.5 ...cache_from_kv_cache.rs, ``scatter_single_kv_to_batched``:
# a prefilled single cache goes to batch slot k at offset k * stride.


def pin_slot_copy_golden_offsets(orc):
    """A row copied into a slot lands at the slot / head / position offsets of tests/golden/kv_cache_layout.json."""
    g = json.load(open(os.path.join(GOLDEN, "kv_cache_layout.json")))
    for c in g["cases"]:
        Hkv, max_len, d, slot, head, pos = (c[x] for x in ("num_kv_heads", "max_len", "head_dim", "slot", "head", "pos"))
        M = slot + 1
        src = np.zeros((Hkv, max_len, d), np.float32)
        marker = np.arange(1, d + 1, dtype=np.float32)
        src[head, pos] = marker
        kc = np.zeros((M, Hkv, max_len, d), np.float32)
        vc = kc.copy()
        orc.copy_to_slot(src, src, max_len, pos + 1, kc, vc, slot, M, Hkv, d, max_len)
        flat = kc.reshape(-1)
        assert np.array_equal(flat[c["offset"]:c["offset"] + d], marker), f"case {c}"
        assert np.count_nonzero(flat) == d


def pin_slot_copy_then_decode_equals_single(orc):
    """Decoding the slot after the copy gives exactly what decoding the single cache gave.

    The single cache has its own max_len (20) and only 13 live rows of 3 KV
    heads; a copy of Hkv * seq_len * d consecutive floats from the start of the
    single cache (one block, as the page's D2D copy is written) would move head
    0's rows 13..38 instead of heads 1 and 2: that reading fails here.
    """
    r = _rng("slotdecode")
    Hkv, H, d, src_max, seq_len, M, max_len, slot = 3, 6, 4, 20, 13, 4, 16, 2
    sk = r.standard_normal((Hkv, src_max, d)).astype(np.float32)
    sv = r.standard_normal((Hkv, src_max, d)).astype(np.float32)
    kc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    vc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
    orc.copy_to_slot(sk, sv, src_max, seq_len, kc, vc, slot, M, Hkv, d, max_len)
    q = r.standard_normal((M, H * d)).astype(np.float32)
    lens = np.array([16, 5, seq_len, 0], np.int32)
    got = orc.decode(q, kc, vc, lens, M, H, Hkv, d, max_len, _scale(d))[slot]
    want = orc.decode(q[slot:slot + 1], sk, sv, np.array([seq_len], np.int32), 1, H, Hkv, d, src_max, _scale(d))[0]
    assert np.array_equal(got, want), "slot decode differs from the single-cache decode"


def pin_slot_copy_touches_only_the_slot_prefix(orc):
    """Exactly Hkv * seq_len * d elements change: rows >= seq_len and other slots keep their bytes."""
    r = _rng("slotuntouched")
    for Hkv, d, src_max, seq_len, M, max_len, slot in [(2, 8, 10, 7, 3, 12, 1), (1, 4, 5, 5, 1, 5, 0),
                                                        (4, 2, 30, 1, 5, 3, 4)]:
        sk = r.standard_normal((Hkv, src_max, d)).astype(np.float32)
        sent = np.full((M, Hkv, max_len, d), 0x7FC0DEAD, np.uint32).view(np.float32)
        kc, vc = sent.copy(), sent.copy()
        orc.copy_to_slot(sk, sk, src_max, seq_len, kc, vc, slot, M, Hkv, d, max_len)
        changed = kc.view(np.uint32) != 0x7FC0DEAD
        assert np.count_nonzero(changed) == Hkv * seq_len * d
        assert changed[slot, :, :seq_len].all()
        assert np.array_equal(kc.view(np.uint32), vc.view(np.uint32))


def pin_slot_copy_brute(orc):
    """Bit-exact agreement with numpy slice assignment (NaN payloads kept), and seq_len 0 is a no-op."""
    r = _rng("slotbrute")
    for Hkv, d, src_max, seq_len, M, max_len, slot in [(3, 4, 9, 6, 2, 7, 0), (2, 8, 4, 4, 6, 9, 5),
                                                        (5, 2, 12, 0, 3, 12, 2), (1, 1, 1, 1, 1, 1, 0)]:
        sk = r.standard_normal((Hkv, src_max, d)).astype(np.float32)
        sv = r.standard_normal((Hkv, src_max, d)).astype(np.float32)
        sk.view(np.uint32).reshape(-1)[0] = 0x7FA00001
        kc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
        vc = r.standard_normal((M, Hkv, max_len, d)).astype(np.float32)
        bk, bv = brute.copy_to_slot(sk, sv, src_max, seq_len, kc, vc, slot, M, Hkv, d, max_len)
        k0, v0 = kc.copy(), vc.copy()
        orc.copy_to_slot(sk, sv, src_max, seq_len, kc, vc, slot, M, Hkv, d, max_len)
        assert np.array_equal(kc.view(np.uint32), bk.reshape(kc.shape).view(np.uint32))
        assert np.array_equal(vc.view(np.uint32), bv.reshape(vc.shape).view(np.uint32))
        if seq_len == 0:
            assert np.array_equal(kc.view(np.uint32), k0.view(np.uint32))


def pin_slot_copy_rejects(orc):
    """A slot outside the batch or more rows than either cache holds is refused, caches untouched."""
    sk = np.ones((2, 4, 2), np.float32)
    for seq_len, slot, M, max_len in ((5, 0, 1, 8), (4, 0, 1, 3), (1, 1, 1, 4), (1, -1, 2, 4), (-1, 0, 1, 4)):
        kc = np.zeros((M, 2, max_len, 2), np.float32)
        vc = kc.copy()
        try:
            orc.copy_to_slot(sk, sk, 4, seq_len, kc, vc, slot, M, 2, 2, max_len)
        except ValueError:
            assert not kc.any() and not vc.any()
            continue
        raise AssertionError(f"seq_len {seq_len} slot {slot} M {M} max_len {max_len} accepted")


# --------------------------------------------------------------------------- rope
#
# GPT-NeoX half-split partial rotary embedding: trustformers-core 0.2.0
# src/gpu_ops/cuda/oxicuda/attention.rs, ``rope_neox_gpu_to_gpu`` and its CPU
# helper ``rope_reference``; realizar 0.8.5 ...cache_from_kv_cache.rs,
# ``apply_rope_to_buffer`` (the rotary_ndims = head_dim case, base = theta).


def pin_rope_position_zero_is_identity(orc):
    """At position 0 every angle is 0, so the rotation is exactly the identity."""
    r = _rng("rope0")
    n, H, d = 3, 2, 8
    x = r.standard_normal((n, H * d)).astype(np.float32)
    for rot in (0, 2, 4, 8):
        y = orc.rope(x, np.zeros(n, np.int32), H, d, rot, 10000.0)
        assert np.array_equal(y, x.astype(np.float64)), f"position 0, rotary {rot}"


def pin_rope_untouched_dims(orc):
    """Dims at or past rotary_ndims pass through unchanged; rotary_ndims = 0 is the identity."""
    r = _rng("ropetail")
    n, H, d = 4, 3, 10
    x = r.standard_normal((n, H * d)).astype(np.float32)
    pos = np.array([1, 7, 100, 12345], np.int32)
    assert np.array_equal(orc.rope(x, pos, H, d, 0, 500.0), x.astype(np.float64)), "rotary 0"
    for rot in (2, 4, 6):
        y = orc.rope(x, pos, H, d, rot, 500.0).reshape(n, H, d)
        assert np.array_equal(y[:, :, rot:], x.reshape(n, H, d)[:, :, rot:].astype(np.float64)), f"tail rot={rot}"
        assert not np.allclose(y[:, :, :rot], x.reshape(n, H, d)[:, :, :rot]), f"head rot={rot} not rotated"


def pin_rope_basis_vectors(orc):
    """Pair 0 turns at base^0 = 1 radian per position, counter-clockwise, pairing dim 0 with dim half.

    e_0 at position p goes to cos(p) e_0 + sin(p) e_half and e_half to
    -sin(p) e_0 + cos(p) e_half; no other dim is touched.
    """
    H, d, rot = 1, 8, 8
    half = rot // 2
    for p in (1, 2, 5, 33):
        for src, want in ((0, {0: math.cos(p), half: math.sin(p)}), (half, {0: -math.sin(p), half: math.cos(p)})):
            x = np.zeros((1, d), np.float32)
            x[0, src] = 1.0
            y = orc.rope(x, np.array([p], np.int32), H, d, rot, 10000.0)[0]
            exp = np.zeros(d)
            for k, val in want.items():
                exp[k] = val
            _close(y, exp, 1e-15, f"basis e_{src} at position {p}")


def pin_rope_frequency_ladder(orc):
    """Pair i turns at base^(-2i/rotary_ndims) radians per position.

    With base 10000 and rotary 4 (the sizes of the pages' RoPE parity test,
    head_dim 6) pair 1 turns at 10000^(-1/2) = 1/100, so position 100 turns
    e_1 by exactly one radian; with base 10000 and rotary 8 the four pairs turn
    at 1, 1/10, 1/100, 1/1000: position 1000 turns pair i by 1000 / 10^i.
    """
    x = np.zeros((1, 6), np.float32)
    x[0, 1] = 1.0
    y = orc.rope(x, np.array([100], np.int32), 1, 6, 4, 10000.0)[0]
    _close(y, [0, math.cos(1.0), 0, math.sin(1.0), 0, 0], 1e-14, "rotary 4 of head_dim 6, pair 1")
    for i, turns in enumerate((1000.0, 100.0, 10.0, 1.0)):
        x = np.zeros((1, 8), np.float32)
        x[0, i] = 1.0
        y = orc.rope(x, np.array([1000], np.int32), 1, 8, 8, 10000.0)[0]
        exp = np.zeros(8)
        exp[i], exp[i + 4] = math.cos(turns), math.sin(turns)
        _close(y, exp, 1e-12, f"rotary 8 pair {i}")


def pin_rope_pair_norms_preserved(orc):
    """Each rotated pair keeps its length."""
    r = _rng("ropenorm")
    n, H, d, rot = 5, 2, 16, 12
    x = r.standard_normal((n, H * d)).astype(np.float32)
    pos = r.integers(0, 40000, size=n).astype(np.int32)
    y = orc.rope(x, pos, H, d, rot, 1e6).reshape(n, H, d)
    xs = x.reshape(n, H, d).astype(np.float64)
    h = rot // 2
    _close(np.hypot(y[:, :, :h], y[:, :, h:rot]), np.hypot(xs[:, :, :h], xs[:, :, h:rot]), 1e-12, "pair norms")


def pin_rope_composes(orc):
    """Rotating to p1 and then by p2 equals rotating to p1 + p2 (up to the f32 hand-over)."""
    r = _rng("ropecomp")
    n, H, d, rot = 4, 2, 8, 8
    x = r.standard_normal((n, H * d)).astype(np.float32)
    p1 = np.array([3, 50, 700, 9000], np.int32)
    p2 = np.array([4, 1, 300, 11], np.int32)
    two = orc.rope(orc.rope(x, p1, H, d, rot, 10000.0).astype(np.float32), p2, H, d, rot, 10000.0)
    _close(two, orc.rope(x, p1 + p2, H, d, rot, 10000.0), 2e-6, "R(p2) R(p1) = R(p1 + p2)")


def pin_rope_relative_position(orc):
    """q at position p and k at position p' score the same for every equal offset p - p'."""
    r = _rng("roperel")
    H, d, rot = 2, 8, 8
    q = r.standard_normal((1, H * d)).astype(np.float32)
    k = r.standard_normal((1, H * d)).astype(np.float32)
    for off in (0, 1, 7, 250):
        scores = []
        for base_pos in (0, 13, 1000, 31000):
            rq = orc.rope(q, np.array([base_pos + off], np.int32), H, d, rot, 10000.0).reshape(H, d)
            rk = orc.rope(k, np.array([base_pos], np.int32), H, d, rot, 10000.0).reshape(H, d)
            scores.append((rq * rk).sum(axis=1))
        for sc in scores[1:]:
            _close(sc, scores[0], 1e-9, f"offset {off}")


def pin_rope_brute(orc):
    """Complex-number formulation (oracle/brute.py) on random rows, partial rotary and several bases."""
    r = _rng("ropebrute")
    for n, H, d, rot, base in [(5, 3, 8, 8, 10000.0), (3, 2, 12, 4, 10000.0), (6, 4, 32, 16, 1e6),
                               (2, 1, 6, 2, 500.0), (4, 2, 128, 128, 10000.0), (4, 2, 128, 32, 10000.0)]:
        x = r.standard_normal((n, H * d)).astype(np.float32)
        pos = r.integers(0, 33000, size=n).astype(np.int32)
        _close(orc.rope(x, pos, H, d, rot, base), brute.rope(x, pos, H, d, rot, base), 1e-9,
               f"rope brute n={n} H={H} d={d} rot={rot}")


def pin_rope_pages_case(orc):
    """The sizes and inputs of the pages' RoPE parity test, at position offsets 0 and 3.

    trustformers-core 0.2.0 ..., gpu_tests ``oxicuda_resident_rope_parity_with_offset``:
    seq 2, 2 heads, head_dim 6, rotary 4, base 10000, element t of the input
    = 0.31 t - 1.5 (f32).  No expected values are printed; pair 0 turns by the
    position and pair 1 by a hundredth of it, so each output is written out here.
    """
    seq, H, d, rot = 2, 2, 6, 4
    x = (np.arange(seq * H * d, dtype=np.float32) * np.float32(0.31) - np.float32(1.5)).reshape(seq, H * d)
    for offset in (0, 3):
        pos = np.arange(seq, dtype=np.int32) + offset
        y = orc.rope(x, pos, H, d, rot, 10000.0).reshape(seq, H, d)
        xs = x.reshape(seq, H, d).astype(np.float64)
        for t in range(seq):
            p = float(pos[t])
            for h in range(H):
                a0, a1 = p, p / 100.0
                e = [xs[t, h, 0] * math.cos(a0) - xs[t, h, 2] * math.sin(a0),
                     xs[t, h, 1] * math.cos(a1) - xs[t, h, 3] * math.sin(a1),
                     xs[t, h, 0] * math.sin(a0) + xs[t, h, 2] * math.cos(a0),
                     xs[t, h, 1] * math.sin(a1) + xs[t, h, 3] * math.cos(a1),
                     xs[t, h, 4], xs[t, h, 5]]
                _close(y[t, h], e, 1e-12, f"offset {offset} row {t} head {h}")
        _close(y.reshape(seq, H * d), brute.rope(x, pos, H, d, rot, 10000.0), 1e-12, f"brute offset {offset}")


def pin_rope_rejects_bad_sizes(orc):
    """Odd rotary_ndims, rotary_ndims > head_dim and a non-positive base are refused."""
    x = np.ones((1, 8), np.float32)
    for rot, base in ((3, 10000.0), (10, 10000.0), (8, 0.0), (-2, 10000.0)):
        try:
            orc.rope(x, np.array([1], np.int32), 1, 8, rot, base)
        except ValueError:
            continue
        raise AssertionError(f"rotary {rot} base {base} accepted")


ALL_PINS = [(name, fn) for name, fn in sorted(globals().items()) if name.startswith("pin_")]
