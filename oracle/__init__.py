"""CPU oracle for GPU-resident attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it.

``liboracle.so`` (plain C, fp64, OpenMP over independent (batch, head) or
(sequence, head) units) is built from ``oracle.c`` by :func:`build`.  The
functions here only marshal numpy arrays; the arithmetic is in ``oracle.c``
and follows the definitions cited there:

* prefill -- trueno-gpu 0.4.11 ``src/memory/resident/attention.rs``,
  ``batched_multihead_attention``; trustformers-core 0.2.0
  ``src/gpu_ops/cuda/oxicuda/attention.rs``, ``attention_prefill_gpu_to_gpu``
  and ``prefill_reference``;
* decode -- trueno-gpu ``incremental_attention_gpu``; realizar 0.8.5
  ``src/cuda/executor/cache_from_cache_from_kv_cache.rs``,
  ``init_kv_cache_gpu`` / ``init_batched_kv_cache_gpu`` (GQA cache layout);
* scatter -- trueno-gpu ``kv_cache_scatter_gpu``;
* chunked prefill behind a cache -- trustformers-core ``attention_prefill_gpu_to_gpu``
  (the offset mask its nothing-cached mask leaves to other paths);
* reduced-precision prefill -- trueno-gpu ``batched_gemm`` (fp16 tensor-core
  operands): attention of the inputs rounded to binary16 / bfloat16;
* copy of a prefilled cache into a batch slot -- realizar
  ``scatter_single_kv_to_batched``;
* rotary position embedding -- trustformers-core ``rope_neox_gpu_to_gpu`` /
  ``rope_reference``; realizar ``apply_rope_to_buffer``; also composed with the
  chunked prefill (rotation at each new token's absolute position).

``brute.py`` is a second, independent numpy fp64 formulation, checked
against this one by the pins and used by the GPU tests for whole-output
checks of large results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(src: str = _SRC, out: str = _LIB_PATH, extra_flags: list[str] | None = None) -> str:
    """Compile oracle.c into a shared library (gcc, -O2, OpenMP, no fast-math); ``extra_flags``
    (e.g. sanitizers, for the CPU checks) are added to the command."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", *(extra_flags or []), src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_prefill.argtypes = [p, p, p, p, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int]
    lib.oracle_prefill.restype = ctypes.c_int
    lib.oracle_prefill_rows.argtypes = [p, p, p, p, i64, p, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int]
    lib.oracle_prefill_rows.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, ctypes.c_float]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode_rows.argtypes = [p, p, p, p, p, i64, p, i64, i64, i64, i64, i64, ctypes.c_float]
    lib.oracle_decode_rows.restype = ctypes.c_int
    lib.oracle_scatter.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64]
    lib.oracle_scatter.restype = ctypes.c_int
    lib.oracle_prefill_cached.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, ctypes.c_float]
    lib.oracle_prefill_cached.restype = ctypes.c_int
    lib.oracle_prefill_cached_rows.argtypes = [p, p, p, p, p, p, p, i64, p, i64, i64, i64, i64, i64, i64,
                                               ctypes.c_float]
    lib.oracle_prefill_cached_rows.restype = ctypes.c_int
    lib.oracle_copy_to_slot.argtypes = [p, p, i64, i64, p, p, i64, i64, i64, i64, i64]
    lib.oracle_copy_to_slot.restype = ctypes.c_int
    lib.oracle_round16.argtypes = [p, p, i64, ctypes.c_int]
    lib.oracle_round16.restype = ctypes.c_int
    lib.oracle_prefill_lowp.argtypes = [p, p, p, p, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int, ctypes.c_int]
    lib.oracle_prefill_lowp.restype = ctypes.c_int
    lib.oracle_prefill_cached_rope.argtypes = [p, p, p, p, p, p, p, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                                               i64, ctypes.c_double]
    lib.oracle_prefill_cached_rope.restype = ctypes.c_int
    lib.oracle_rope.argtypes = [p, p, p, i64, i64, i64, i64, ctypes.c_double]
    lib.oracle_rope.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    return lib


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library; ``path`` loads another copy."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError(f"oracle inputs are the exact f32 values given to the GPU, got {a.dtype}")
    return a


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


class Oracle:
    """Thin numpy-facing wrapper over one loaded copy of the oracle library."""

    def __init__(self, lib: ctypes.CDLL | None = None):
        self.lib = lib if lib is not None else load()

    def prefill(self, q, k, v, B, S, H, d, scale, causal):
        """O[b, i, h*d:(h+1)*d] for every (b, i, h); q/k/v are [B, S, H*d] f32."""
        q, k, v = _f32(q), _f32(k), _f32(v)
        n = B * S * H * d
        assert q.size == n and k.size == n and v.size == n
        out = np.empty(n, dtype=np.float64)
        rc = self.lib.oracle_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S, H, d,
                                     float(np.float32(scale)), int(bool(causal)))
        if rc != 0:
            raise ValueError("oracle_prefill rejected its arguments")
        return out.reshape(B, S, H * d)

    def prefill_rows(self, q, k, v, sel, B, S, H, d, scale, causal):
        """Selected rows; ``sel`` is an (n, 3) int array of (b, i, h)."""
        q, k, v = _f32(q), _f32(k), _f32(v)
        sel = np.ascontiguousarray(sel, dtype=np.int64).reshape(-1, 3)
        out = np.empty((sel.shape[0], d), dtype=np.float64)
        rc = self.lib.oracle_prefill_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(sel), sel.shape[0],
                                          _ptr(out), B, S, H, d, float(np.float32(scale)),
                                          int(bool(causal)))
        if rc != 0:
            raise ValueError("oracle_prefill_rows rejected its arguments")
        return out

    def decode(self, q, k_cache, v_cache, lens, M, H, Hkv, d, max_len, scale):
        """out[m, h*d:(h+1)*d]; q is [M, H*d], caches [M, Hkv, max_len, d]."""
        q, k_cache, v_cache = _f32(q), _f32(k_cache), _f32(v_cache)
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        assert lens.size == M and q.size == M * H * d
        assert k_cache.size == M * Hkv * max_len * d and v_cache.size == k_cache.size
        out = np.empty(M * H * d, dtype=np.float64)
        rc = self.lib.oracle_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens), _ptr(out),
                                    M, H, Hkv, d, max_len, float(np.float32(scale)))
        if rc != 0:
            raise ValueError("oracle_decode rejected its arguments")
        return out.reshape(M, H * d)

    def decode_rows(self, q, k_cache, v_cache, lens, sel, M, H, Hkv, d, max_len, scale):
        """Selected (m, h) outputs; ``sel`` is an (n, 2) int array."""
        q, k_cache, v_cache = _f32(q), _f32(k_cache), _f32(v_cache)
        lens = np.ascontiguousarray(lens, dtype=np.int32)
        sel = np.ascontiguousarray(sel, dtype=np.int64).reshape(-1, 2)
        out = np.empty((sel.shape[0], d), dtype=np.float64)
        rc = self.lib.oracle_decode_rows(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens),
                                         _ptr(sel), sel.shape[0], _ptr(out), M, H, Hkv, d,
                                         max_len, float(np.float32(scale)))
        if rc != 0:
            raise ValueError("oracle_decode_rows rejected its arguments")
        return out

    def scatter(self, k_new, v_new, k_cache, v_cache, cache_lens, M, n_new, Hkv, d, max_len):
        """In-place append into numpy caches (modified); returns them."""
        k_new, v_new = _f32(k_new), _f32(v_new)
        if not (k_cache.flags.c_contiguous and v_cache.flags.c_contiguous):
            raise ValueError("caches must be C-contiguous (updated in place)")
        cache_lens = np.ascontiguousarray(cache_lens, dtype=np.int32)
        rc = self.lib.oracle_scatter(_ptr(k_new), _ptr(v_new), _ptr(_f32(k_cache)),
                                     _ptr(_f32(v_cache)), _ptr(cache_lens), M, n_new, Hkv, d,
                                     max_len)
        if rc != 0:
            raise ValueError("oracle_scatter rejected its arguments")
        return k_cache, v_cache

    def prefill_cached(self, q, k_new, v_new, k_cache, v_cache, cache_lens, M, n_new, H, Hkv, d, max_len,
                       scale):
        """Chunk of n_new tokens behind cache_lens[m] cached rows; out is [M, n_new, H*d]."""
        q, k_new, v_new = _f32(q), _f32(k_new), _f32(v_new)
        k_cache, v_cache = _f32(k_cache), _f32(v_cache)
        cache_lens = np.ascontiguousarray(cache_lens, dtype=np.int32)
        assert q.size == M * n_new * H * d and k_new.size == M * n_new * Hkv * d == v_new.size
        assert k_cache.size == M * Hkv * max_len * d == v_cache.size and cache_lens.size == M
        out = np.empty(M * n_new * H * d, dtype=np.float64)
        rc = self.lib.oracle_prefill_cached(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(cache_lens), _ptr(out), M, n_new, H, Hkv, d, max_len,
                                            float(np.float32(scale)))
        if rc != 0:
            raise ValueError("oracle_prefill_cached rejected its arguments")
        return out.reshape(M, n_new, H * d)

    def prefill_cached_rows(self, q, k_new, v_new, k_cache, v_cache, cache_lens, sel, M, n_new, H, Hkv, d,
                            max_len, scale):
        """Selected rows of prefill_cached; ``sel`` is an (n, 3) int array of (m, r, h)."""
        q, k_new, v_new = _f32(q), _f32(k_new), _f32(v_new)
        k_cache, v_cache = _f32(k_cache), _f32(v_cache)
        cache_lens = np.ascontiguousarray(cache_lens, dtype=np.int32)
        sel = np.ascontiguousarray(sel, dtype=np.int64).reshape(-1, 3)
        out = np.empty((sel.shape[0], d), dtype=np.float64)
        rc = self.lib.oracle_prefill_cached_rows(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                                 _ptr(cache_lens), _ptr(sel), sel.shape[0], _ptr(out), M, n_new,
                                                 H, Hkv, d, max_len, float(np.float32(scale)))
        if rc != 0:
            raise ValueError("oracle_prefill_cached_rows rejected its arguments")
        return out

    def prefill_cached_rope(self, q, k_new, v_new, k_cache, v_cache, cache_lens, M, n_new, H, Hkv, d, max_len,
                            scale, rotary_ndims, base):
        """prefill_cached with query and new key row r of sequence m rotated to cache_lens[m] + r."""
        q, k_new, v_new = _f32(q), _f32(k_new), _f32(v_new)
        k_cache, v_cache = _f32(k_cache), _f32(v_cache)
        cache_lens = np.ascontiguousarray(cache_lens, dtype=np.int32)
        assert q.size == M * n_new * H * d and k_new.size == M * n_new * Hkv * d == v_new.size
        assert k_cache.size == M * Hkv * max_len * d == v_cache.size and cache_lens.size == M
        out = np.empty(M * n_new * H * d, dtype=np.float64)
        rc = self.lib.oracle_prefill_cached_rope(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                                 _ptr(cache_lens), _ptr(out), M, n_new, H, Hkv, d, max_len,
                                                 float(np.float32(scale)), int(rotary_ndims), float(base))
        if rc != 0:
            raise ValueError("oracle_prefill_cached_rope rejected its arguments")
        return out.reshape(M, n_new, H * d)

    def copy_to_slot(self, src_k, src_v, src_max_len, seq_len, dst_k, dst_v, slot, M, Hkv, d, max_len):
        """In-place copy of a single cache [Hkv, src_max_len, d] into slot `slot` of [M, Hkv, max_len, d]."""
        src_k, src_v = _f32(src_k), _f32(src_v)
        if not (dst_k.flags.c_contiguous and dst_v.flags.c_contiguous):
            raise ValueError("caches must be C-contiguous (updated in place)")
        assert src_k.size == Hkv * src_max_len * d and dst_k.size == M * Hkv * max_len * d
        rc = self.lib.oracle_copy_to_slot(_ptr(src_k), _ptr(src_v), src_max_len, seq_len, _ptr(_f32(dst_k)),
                                          _ptr(_f32(dst_v)), slot, M, Hkv, d, max_len)
        if rc != 0:
            raise ValueError("oracle_copy_to_slot rejected its arguments")
        return dst_k, dst_v

    FP16, BF16 = 1, 2

    def round16(self, x, fmt):
        """f32 values rounded (nearest, ties to even) to binary16 (fmt 1) or bfloat16 (fmt 2), as f32."""
        x = _f32(x)
        y = np.empty_like(x)
        if self.lib.oracle_round16(_ptr(x), _ptr(y), x.size, int(fmt)) != 0:
            raise ValueError("oracle_round16 rejected its arguments")
        return y

    def prefill_lowp(self, q, k, v, B, S, H, d, scale, causal, fmt):
        """Attention (fp64) of q, k, v rounded to the 16-bit format fmt; [B, S, H*d]."""
        q, k, v = _f32(q), _f32(k), _f32(v)
        out = np.empty(B * S * H * d, dtype=np.float64)
        rc = self.lib.oracle_prefill_lowp(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S, H, d,
                                          float(np.float32(scale)), 1 if causal else 0, int(fmt))
        if rc != 0:
            raise ValueError("oracle_prefill_lowp rejected its arguments")
        return out.reshape(B, S, H * d)

    def rope(self, x, pos, H, d, rotary_ndims, base):
        """NeoX half-split partial RoPE of rows [n, H*d] at positions pos[n]; returns f64 [n, H*d]."""
        x = _f32(x)
        pos = np.ascontiguousarray(pos, dtype=np.int32).reshape(-1)
        n = pos.size
        assert x.size == n * H * d
        out = np.empty(n * H * d, dtype=np.float64)
        rc = self.lib.oracle_rope(_ptr(x), _ptr(pos), _ptr(out), n, H, d, rotary_ndims, float(base))
        if rc != 0:
            raise ValueError("oracle_rope rejected its arguments")
        return out.reshape(n, H * d)

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        """Threads of the following calls (timing only; results do not depend on it)."""
        self.lib.oracle_set_num_threads(int(n))


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
