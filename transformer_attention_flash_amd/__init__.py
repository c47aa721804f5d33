"""GPU-resident scaled-dot-product attention for MI355X (gfx950).

Thin Python binding over the C ABI of ``libattn.so`` (``include/attn.h``).
Each function has the name of the C entry point it calls and only marshals
arguments: it checks the torch tensors' device, dtype, contiguity and element
counts (which the C layer cannot see behind raw pointers), passes their data
pointers and the current HIP stream of their device, and turns a non-zero
status into :class:`AttnError`.  All computation happens in the HIP kernels.

The library is built ahead of time (``python -m
transformer_attention_flash_amd.build`` or ``__graft_entry__.build()``); if it
is missing, every call raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

__all__ = [
    "AttnError",
    "ATTN_MAX_SEQS",
    "attn_prefill",
    "attn_prefill_cached",
    "attn_prefill_cached_rope",
    "attn_prefill_lowp",
    "ATTN_PREC_FP16",
    "ATTN_PREC_BF16",
    "attn_decode_workspace_bytes",
    "attn_decode_gqa_batched",
    "attn_decode_gqa_batched_noalloc",
    "ATTN_DECODE_SCRATCH_BYTES",
    "kv_cache_scatter",
    "kv_cache_scatter_rope",
    "attn_decode_gqa_batched_rope",
    "kv_cache_copy_to_slot",
    "kv_lengths_reset",
    "kv_lengths_rollback",
    "attn_status_string",
    "library",
    "library_path",
]

ATTN_MAX_SEQS = 32
ATTN_PREC_FP16 = 1
ATTN_PREC_BF16 = 2
ATTN_DECODE_SCRATCH_BYTES = 64 << 20
_STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_INVALID_DIM", 3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_OVERFLOW", 5: "ATTN_ERR_WORKSPACE", 6: "ATTN_ERR_HIP", 7: "ATTN_ERR_ALIAS",
}

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libattn.so")
_lib = None


class AttnError(RuntimeError):
    """A non-zero attn_status returned by libattn.so."""

    def __init__(self, status: int, func: str):
        self.status = status
        super().__init__(f"{func}: {_STATUS.get(status, status)} ({attn_status_string(status)})")


def library_path() -> str:
    return _LIB_PATH


def library() -> ctypes.CDLL:
    """The loaded libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m transformer_attention_flash_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        p, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
        lib.attn_prefill.argtypes = [p, p, p, p, i32, i32, i32, i32, f32, i32, p]
        lib.attn_prefill.restype = ctypes.c_int
        lib.attn_prefill_lowp.argtypes = [p, p, p, p, i32, i32, i32, i32, f32, i32, i32, p]
        lib.attn_prefill_lowp.restype = ctypes.c_int
        lib.attn_prefill_cached.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p]
        lib.attn_prefill_cached.restype = ctypes.c_int
        lib.attn_prefill_cached_rope.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, i32, f32,
                                                 p]
        lib.attn_prefill_cached_rope.restype = ctypes.c_int
        lib.attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
        lib.attn_decode_workspace_bytes.restype = sz
        lib.attn_decode_gqa_batched.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, f32, p, sz, p]
        lib.attn_decode_gqa_batched.restype = ctypes.c_int
        lib.attn_decode_gqa_batched_noalloc.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, f32, p]
        lib.attn_decode_gqa_batched_noalloc.restype = ctypes.c_int
        lib.kv_cache_scatter.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, p]
        lib.kv_cache_scatter.restype = ctypes.c_int
        lib.kv_cache_scatter_rope.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, p]
        lib.kv_cache_scatter_rope.restype = ctypes.c_int
        lib.attn_decode_gqa_batched_rope.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, f32, i32, f32, p,
                                                     sz, p]
        lib.attn_decode_gqa_batched_rope.restype = ctypes.c_int
        lib.kv_cache_copy_to_slot.argtypes = [p, p, i32, i32, p, p, i32, i32, i32, i32, i32, p, p]
        lib.kv_cache_copy_to_slot.restype = ctypes.c_int
        lib.kv_lengths_reset.argtypes = [p, i32]
        lib.kv_lengths_reset.restype = ctypes.c_int
        lib.kv_lengths_rollback.argtypes = [p, i32, i32]
        lib.kv_lengths_rollback.restype = ctypes.c_int
        lib.attn_status_string.argtypes = [ctypes.c_int]
        lib.attn_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def attn_status_string(status: int) -> str:
    return library().attn_status_string(int(status)).decode()


# ----------------------------------------------------------------- marshalling


def _check_tensor(name, t, numel, device=None):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live in GPU memory, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _host_ints(name, values, count) -> ctypes.Array:
    vals = [int(x) for x in (values.tolist() if hasattr(values, "tolist") else values)]
    if len(vals) != count:
        raise ValueError(f"{name} has {len(vals)} entries, expected {count}")
    for x in vals:
        if not -(2**31) <= x < 2**31:
            raise ValueError(f"{name} value {x} does not fit int32")
    return (ctypes.c_int32 * count)(*vals)


def _stream_ptr(device, stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _call(func_name, status):
    if status != 0:
        raise AttnError(status, func_name)


# ----------------------------------------------------------------- entry points


def attn_prefill(q, k, v, out, batch: int, seq_len: int, n_heads: int, head_dim: int,
                 scale: float, causal: bool, stream=None) -> None:
    """out[b, i, h*d:(h+1)*d] = softmax(scale q k^T [causal]) v for [batch, seq_len, n_heads*head_dim] f32."""
    n = batch * seq_len * n_heads * head_dim
    dev = q.device
    ptrs = [_check_tensor(nm, t, n, dev) for nm, t in (("q", q), ("k", k), ("v", v), ("out", out))]
    _call("attn_prefill", library().attn_prefill(*ptrs, batch, seq_len, n_heads, head_dim, scale,
                                                 1 if causal else 0, _stream_ptr(dev, stream)))


def attn_prefill_lowp(q, k, v, out, batch: int, seq_len: int, n_heads: int, head_dim: int,
                      scale: float, causal: bool, precision: int, stream=None) -> None:
    """attn_prefill on 16-bit MFMA operands; precision ATTN_PREC_FP16 or ATTN_PREC_BF16 (f32 in and out)."""
    n = batch * seq_len * n_heads * head_dim
    dev = q.device
    ptrs = [_check_tensor(nm, t, n, dev) for nm, t in (("q", q), ("k", k), ("v", v), ("out", out))]
    _call("attn_prefill_lowp", library().attn_prefill_lowp(*ptrs, batch, seq_len, n_heads, head_dim, scale,
                                                           1 if causal else 0, int(precision),
                                                           _stream_ptr(dev, stream)))


def attn_prefill_cached(q, k_new, v_new, k_cache, v_cache, cache_lens: Sequence[int], out, num_seqs: int,
                        n_new: int, num_heads: int, num_kv_heads: int, head_dim: int, max_len: int,
                        scale: float, stream=None) -> None:
    """Append a chunk's K/V at cache_lens[m] and attend its queries over cache rows 0..cache_lens[m]+r."""
    dev = q.device
    qn = num_seqs * n_new * num_heads * head_dim
    nn = num_seqs * n_new * num_kv_heads * head_dim
    cn = num_seqs * num_kv_heads * max_len * head_dim
    ptrs = [_check_tensor("q", q, qn, dev), _check_tensor("k_new", k_new, nn, dev),
            _check_tensor("v_new", v_new, nn, dev), _check_tensor("k_cache", k_cache, cn, dev),
            _check_tensor("v_cache", v_cache, cn, dev)]
    lens = _host_ints("cache_lens", cache_lens, num_seqs)
    po = _check_tensor("out", out, qn, dev)
    _call("attn_prefill_cached",
          library().attn_prefill_cached(*ptrs, lens, po, num_seqs, n_new, num_heads, num_kv_heads, head_dim,
                                        max_len, scale, _stream_ptr(dev, stream)))


def attn_prefill_cached_rope(q, k_new, v_new, k_cache, v_cache, cache_lens: Sequence[int], out, num_seqs: int,
                             n_new: int, num_heads: int, num_kv_heads: int, head_dim: int, max_len: int,
                             scale: float, rotary_ndims: int, rope_theta: float, stream=None) -> None:
    """attn_prefill_cached with keys appended rotated to P + r and query r rotated to P + r."""
    dev = q.device
    qn = num_seqs * n_new * num_heads * head_dim
    nn = num_seqs * n_new * num_kv_heads * head_dim
    cn = num_seqs * num_kv_heads * max_len * head_dim
    ptrs = [_check_tensor("q", q, qn, dev), _check_tensor("k_new", k_new, nn, dev),
            _check_tensor("v_new", v_new, nn, dev), _check_tensor("k_cache", k_cache, cn, dev),
            _check_tensor("v_cache", v_cache, cn, dev)]
    lens = _host_ints("cache_lens", cache_lens, num_seqs)
    po = _check_tensor("out", out, qn, dev)
    _call("attn_prefill_cached_rope",
          library().attn_prefill_cached_rope(*ptrs, lens, po, num_seqs, n_new, num_heads, num_kv_heads, head_dim,
                                             max_len, scale, rotary_ndims, rope_theta, _stream_ptr(dev, stream)))


def attn_decode_workspace_bytes(num_seqs: int, num_heads: int, head_dim: int, max_len: int) -> int:
    return int(library().attn_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_len))


def _decode_ptrs(q, k_cache, v_cache, out, workspace, num_seqs, num_heads, num_kv_heads, head_dim, max_len):
    import torch

    dev = q.device
    qn = num_seqs * num_heads * head_dim
    cn = num_seqs * num_kv_heads * max_len * head_dim
    ptrs = [_check_tensor("q", q, qn, dev), _check_tensor("k_cache", k_cache, cn, dev),
            _check_tensor("v_cache", v_cache, cn, dev)]
    po = _check_tensor("out", out, qn, dev)
    if not isinstance(workspace, torch.Tensor) or workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the same GPU")
    return dev, ptrs, po, workspace.data_ptr(), workspace.numel() * workspace.element_size()


def attn_decode_gqa_batched(q, k_cache, v_cache, seq_lens: Sequence[int], out, num_seqs: int,
                            num_heads: int, num_kv_heads: int, head_dim: int, max_len: int,
                            scale: float, workspace, stream=None) -> None:
    """Batched GQA decode; ``seq_lens`` is a host sequence of M ints; ``workspace`` a device tensor."""
    dev, ptrs, po, pw, ws_bytes = _decode_ptrs(q, k_cache, v_cache, out, workspace, num_seqs, num_heads,
                                               num_kv_heads, head_dim, max_len)
    lens = _host_ints("seq_lens", seq_lens, num_seqs)
    _call("attn_decode_gqa_batched",
          library().attn_decode_gqa_batched(*ptrs, lens, po, num_seqs, num_heads, num_kv_heads, head_dim,
                                            max_len, scale, pw, ws_bytes, _stream_ptr(dev, stream)))


def attn_decode_gqa_batched_noalloc(q, k_cache, v_cache, seq_lens: Sequence[int], out, num_seqs: int,
                                    num_heads: int, num_kv_heads: int, head_dim: int, max_len: int,
                                    scale: float, stream=None) -> None:
    """attn_decode_gqa_batched on the library's built-in scratch (no workspace, nothing allocated)."""
    dev = q.device
    qn = num_seqs * num_heads * head_dim
    cn = num_seqs * num_kv_heads * max_len * head_dim
    ptrs = [_check_tensor("q", q, qn, dev), _check_tensor("k_cache", k_cache, cn, dev),
            _check_tensor("v_cache", v_cache, cn, dev)]
    po = _check_tensor("out", out, qn, dev)
    lens = _host_ints("seq_lens", seq_lens, num_seqs)
    _call("attn_decode_gqa_batched_noalloc",
          library().attn_decode_gqa_batched_noalloc(*ptrs, lens, po, num_seqs, num_heads, num_kv_heads, head_dim,
                                                    max_len, scale, _stream_ptr(dev, stream)))


def attn_decode_gqa_batched_rope(q, k_cache, v_cache, seq_lens: Sequence[int], out, num_seqs: int,
                                 num_heads: int, num_kv_heads: int, head_dim: int, max_len: int,
                                 scale: float, rotary_ndims: int, rope_theta: float, workspace,
                                 stream=None) -> None:
    """attn_decode_gqa_batched with each query rotated to position seq_lens[m] - 1 first."""
    dev, ptrs, po, pw, ws_bytes = _decode_ptrs(q, k_cache, v_cache, out, workspace, num_seqs, num_heads,
                                               num_kv_heads, head_dim, max_len)
    lens = _host_ints("seq_lens", seq_lens, num_seqs)
    _call("attn_decode_gqa_batched_rope",
          library().attn_decode_gqa_batched_rope(*ptrs, lens, po, num_seqs, num_heads, num_kv_heads, head_dim,
                                                 max_len, scale, rotary_ndims, rope_theta, pw, ws_bytes,
                                                 _stream_ptr(dev, stream)))


def _scatter_ptrs(k_new, v_new, k_cache, v_cache, num_seqs, n_new, num_kv_heads, head_dim, max_len):
    dev = k_new.device
    sn = num_seqs * n_new * num_kv_heads * head_dim
    cn = num_seqs * num_kv_heads * max_len * head_dim
    return dev, [_check_tensor("k_new", k_new, sn, dev), _check_tensor("v_new", v_new, sn, dev),
                 _check_tensor("k_cache", k_cache, cn, dev), _check_tensor("v_cache", v_cache, cn, dev)]


def kv_cache_scatter(k_new, v_new, k_cache, v_cache, cache_lens: Sequence[int], num_seqs: int,
                     n_new: int, num_kv_heads: int, head_dim: int, max_len: int, stream=None) -> None:
    """cache[m, kh, cache_lens[m] + r, :] = new[m, r, kh*d:(kh+1)*d] for K and V."""
    dev, ptrs = _scatter_ptrs(k_new, v_new, k_cache, v_cache, num_seqs, n_new, num_kv_heads, head_dim, max_len)
    lens = _host_ints("cache_lens", cache_lens, num_seqs)
    _call("kv_cache_scatter", library().kv_cache_scatter(*ptrs, lens, num_seqs, n_new, num_kv_heads,
                                                         head_dim, max_len, _stream_ptr(dev, stream)))


def kv_cache_scatter_rope(k_new, v_new, k_cache, v_cache, cache_lens: Sequence[int], num_seqs: int,
                          n_new: int, num_kv_heads: int, head_dim: int, max_len: int, rotary_ndims: int,
                          rope_theta: float, stream=None) -> None:
    """kv_cache_scatter with key row r rotated to position cache_lens[m] + r."""
    dev, ptrs = _scatter_ptrs(k_new, v_new, k_cache, v_cache, num_seqs, n_new, num_kv_heads, head_dim, max_len)
    lens = _host_ints("cache_lens", cache_lens, num_seqs)
    _call("kv_cache_scatter_rope",
          library().kv_cache_scatter_rope(*ptrs, lens, num_seqs, n_new, num_kv_heads, head_dim, max_len,
                                          rotary_ndims, rope_theta, _stream_ptr(dev, stream)))


def kv_cache_copy_to_slot(src_k, src_v, src_max_len: int, seq_len: int, k_cache, v_cache, slot: int,
                          num_seqs: int, num_kv_heads: int, head_dim: int, max_len: int, slot_lens=None,
                          stream=None) -> None:
    """Rows 0..seq_len-1 of each KV head of a single cache go to batch slot `slot`.

    ``slot_lens``, if given, is a mutable host sequence of num_seqs lengths whose
    entry ``slot`` is set to seq_len on success.
    """
    dev = k_cache.device
    sn = num_kv_heads * src_max_len * head_dim
    cn = num_seqs * num_kv_heads * max_len * head_dim
    ptrs = [_check_tensor("src_k", src_k, sn, dev), _check_tensor("src_v", src_v, sn, dev)]
    cptrs = [_check_tensor("k_cache", k_cache, cn, dev), _check_tensor("v_cache", v_cache, cn, dev)]
    lens = _host_ints("slot_lens", slot_lens, num_seqs) if slot_lens is not None else None
    _call("kv_cache_copy_to_slot",
          library().kv_cache_copy_to_slot(*ptrs, src_max_len, seq_len, *cptrs, slot, num_seqs, num_kv_heads,
                                          head_dim, max_len, lens, _stream_ptr(dev, stream)))
    if lens is not None:
        slot_lens[slot] = lens[slot]


def _lengths_call(name, lens, num_seqs, *extra):
    arr = _host_ints("lens", lens, num_seqs)
    _call(name, getattr(library(), name)(arr, num_seqs, *extra))
    for m in range(num_seqs):
        lens[m] = arr[m]


def kv_lengths_reset(lens, num_seqs: int) -> None:
    """Every length of the mutable host sequence ``lens`` becomes 0."""
    _lengths_call("kv_lengths_reset", lens, num_seqs)


def kv_lengths_rollback(lens, num_seqs: int, position: int) -> None:
    """Every length of ``lens`` above ``position`` becomes ``position``."""
    _lengths_call("kv_lengths_rollback", lens, num_seqs, position)
