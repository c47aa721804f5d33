"""The C ABI on the CPU: the library loads, exports what include/attn.h declares,
and rejects every invalid call with its documented status before touching HIP.

No call here reaches a kernel launch: every argument set is invalid, and the
library validates on the host before any HIP call (include/attn.h, conventions).
"""
import ctypes
import os
import re
import subprocess

import pytest

import transformer_attention_flash_amd as taf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULL, DIM, UNSUP, OVF, WS, HIP, ALIAS = range(8)
A = 0x10000          # fake, 16-byte aligned "device" addresses, never dereferenced
B_ = 0x20000000
C_ = 0x40000000
O_ = 0x60000000
W_ = 0x80000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return taf.library()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "attn_prefill", "attn_prefill_cached", "attn_decode_workspace_bytes", "attn_decode_gqa_batched",
        "kv_cache_scatter", "attn_status_string", "kv_cache_scatter_rope", "attn_decode_gqa_batched_rope",
        "kv_cache_copy_to_slot", "kv_lengths_reset", "kv_lengths_rollback", "attn_prefill_lowp",
        "attn_decode_gqa_batched_noalloc", "attn_prefill_cached_rope"])


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", taf.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert exported == set(declared_functions()), f"undeclared exports: {sorted(exported - set(declared_functions()))}"


def test_status_strings(lib):
    for s in range(8):
        assert taf.attn_status_string(s) and taf.attn_status_string(s) != "unknown status"
    assert taf.attn_status_string(99) == "unknown status"


def prefill(lib, q=A, k=B_, v=C_, out=O_, b=1, s=64, h=4, d=32, scale=0.125, causal=0):
    return lib.attn_prefill(q, k, v, out, b, s, h, d, scale, causal, None)


def test_prefill_validation(lib):
    assert prefill(lib, q=0) == NULL
    assert prefill(lib, out=0) == NULL
    assert prefill(lib, b=0) == DIM
    assert prefill(lib, s=-1) == DIM
    assert prefill(lib, h=0) == DIM
    assert prefill(lib, causal=2) == DIM
    assert prefill(lib, scale=float("nan")) == DIM
    assert prefill(lib, scale=float("inf")) == DIM
    assert prefill(lib, d=48) == UNSUP
    assert prefill(lib, d=256) == UNSUP
    assert prefill(lib, q=A + 4) == UNSUP
    assert prefill(lib, b=64, s=65536, h=64, d=128) == OVF
    assert prefill(lib, out=A + 64) == ALIAS      # out starts inside q
    assert prefill(lib, out=C_ - 16) == ALIAS     # out runs into v


def test_prefill_lowp_validation(lib):
    def call(q=A, out=O_, b=1, s=64, h=4, d=32, scale=0.125, causal=0, prec=2):
        return lib.attn_prefill_lowp(q, B_, C_, out, b, s, h, d, scale, causal, prec, None)
    assert call(q=0) == NULL
    assert call(b=0) == DIM
    assert call(causal=3) == DIM
    assert call(scale=float("nan")) == DIM
    assert call(d=96) == UNSUP
    assert call(prec=0) == UNSUP
    assert call(prec=3) == UNSUP
    assert call(q=A + 8) == UNSUP
    assert call(b=64, s=65536, h=64, d=128) == OVF
    assert call(out=A + 64) == ALIAS


def decode(lib, q=A, k=B_, v=C_, lens=None, out=O_, M=2, H=8, Hkv=2, d=64, max_len=100, scale=0.125,
           ws=W_, ws_bytes=None):
    if lens is None:
        lens = [5, 100][:M] + [1] * max(0, M - 2)
    arr = (ctypes.c_int32 * max(1, len(lens)))(*lens) if lens != "null" else None
    if ws_bytes is None:
        ws_bytes = lib.attn_decode_workspace_bytes(max(1, min(M, 32)), max(1, H), d if d in (32, 64, 128) else 64,
                                                   max(1, max_len))
    return lib.attn_decode_gqa_batched(q, k, v, arr, out, M, H, Hkv, d, max_len, scale, ws, ws_bytes, None)


def test_decode_validation(lib):
    assert decode(lib, q=0) == NULL
    assert decode(lib, lens="null") == NULL
    assert decode(lib, ws=0) == NULL
    assert decode(lib, M=0, lens=[1]) == DIM
    assert decode(lib, M=33, lens=[1] * 33) == DIM
    assert decode(lib, Hkv=3) == DIM           # 8 % 3 != 0
    assert decode(lib, Hkv=16) == DIM          # more KV heads than query heads
    assert decode(lib, lens=[101, 3]) == DIM   # longer than the cache
    assert decode(lib, lens=[-1, 3]) == DIM
    assert decode(lib, max_len=0, lens=[0, 0]) == DIM
    assert decode(lib, scale=float("nan")) == DIM
    assert decode(lib, d=96) == UNSUP
    assert decode(lib, k=B_ + 8) == UNSUP
    assert decode(lib, ws=W_ + 4) == UNSUP
    assert decode(lib, ws_bytes=16) == WS
    assert decode(lib, out=A) == ALIAS                       # out is q
    assert decode(lib, ws=B_ + 1024) == ALIAS                # workspace inside the K cache


def test_decode_workspace_bytes(lib):
    # acc [M, H, splits, d] + (max, sum) [M, H, splits, 2] floats.  A split is
    # one key block of at least a floor of keys, a power-of-two multiple of 128
    # that keeps a sequence at <= 64 blocks; calls with M * ceil(H / 16) < 16
    # may take 128, 256 or 512 blocks (doubled while M * ceil(H / 16) * n < 1024).
    assert lib.attn_decode_workspace_bytes(32, 32, 128, 4096) == 32 * 32 * 32 * 130 * 4
    assert lib.attn_decode_workspace_bytes(16, 64, 128, 32768) == 16 * 64 * 64 * 130 * 4
    assert lib.attn_decode_workspace_bytes(1, 1, 32, 1) == 1 * 1 * 1 * 34 * 4
    assert lib.attn_decode_workspace_bytes(2, 4, 64, 300) == 2 * 4 * 3 * 66 * 4
    assert lib.attn_decode_workspace_bytes(8, 32, 128, 32768) == 8 * 32 * 64 * 130 * 4    # 16 units: 64
    assert lib.attn_decode_workspace_bytes(4, 32, 128, 32768) == 4 * 32 * 128 * 130 * 4   # 8 units: 128
    assert lib.attn_decode_workspace_bytes(1, 32, 128, 32768) == 1 * 32 * 256 * 130 * 4   # 512 at most; 128-key floor
    assert lib.attn_decode_workspace_bytes(2, 8, 128, 60000) == 2 * 8 * 469 * 130 * 4     # 512 at most; 128-key floor
    assert lib.attn_decode_workspace_bytes(0, 8, 128, 16) == 0
    assert lib.attn_decode_workspace_bytes(33, 8, 128, 16) == 0
    assert lib.attn_decode_workspace_bytes(2, 8, 80, 16) == 0
    # The largest supported cache: 2^30 rows, 64 key blocks of 2^24 keys, or for
    # a single head 512 blocks of 2^21 keys.
    assert lib.attn_decode_workspace_bytes(16, 1, 32, 2**30) == 16 * 64 * 34 * 4
    assert lib.attn_decode_workspace_bytes(1, 1, 32, 2**30) == 512 * 34 * 4
    # Beyond it, up to the int32 limit, the size is refused rather than overflowing.
    assert lib.attn_decode_workspace_bytes(1, 1, 32, 2**30 + 1) == 0
    assert lib.attn_decode_workspace_bytes(1, 1, 32, 2**31 - 1) == 0


def decode_noalloc(lib, q=A, k=B_, v=C_, lens=None, out=O_, M=2, H=8, Hkv=2, d=64, max_len=100, scale=0.125):
    if lens is None:
        lens = [5, 100][:M] + [1] * max(0, M - 2)
    arr = (ctypes.c_int32 * max(1, len(lens)))(*lens) if lens != "null" else None
    return lib.attn_decode_gqa_batched_noalloc(q, k, v, arr, out, M, H, Hkv, d, max_len, scale, None)


def test_decode_noalloc_validation(lib):
    """Every refusal happens on the host, before the scratch is looked up."""
    assert taf.ATTN_DECODE_SCRATCH_BYTES == 64 * 2**20
    assert decode_noalloc(lib, q=0) == NULL
    assert decode_noalloc(lib, lens="null") == NULL
    assert decode_noalloc(lib, M=0, lens=[1]) == DIM
    assert decode_noalloc(lib, M=33, lens=[1] * 33) == DIM
    assert decode_noalloc(lib, Hkv=3) == DIM
    assert decode_noalloc(lib, lens=[101, 3]) == DIM
    assert decode_noalloc(lib, scale=float("inf")) == DIM
    assert decode_noalloc(lib, d=96) == UNSUP
    assert decode_noalloc(lib, out=O_ + 4) == UNSUP
    assert decode_noalloc(lib, max_len=2**30 + 1) == OVF
    assert decode_noalloc(lib, out=A) == ALIAS
    # Sizes whose workspace exceeds the built-in scratch: 32 x 64 heads at d 128 over
    # 64 key blocks need 68.2 MB; 2016 sequence-heads is the most that fits.
    need = lib.attn_decode_workspace_bytes(32, 64, 128, 32768)
    assert need > taf.ATTN_DECODE_SCRATCH_BYTES
    far = dict(q=A, k=2**36, v=2**37, out=3 * 2**36)  # 4.3 GB caches that overlap nothing
    assert decode_noalloc(lib, M=32, H=64, Hkv=8, d=128, max_len=32768, lens=[1] * 32, **far) == WS
    assert decode_noalloc(lib, M=32, H=63, Hkv=7, d=128, max_len=32768, lens=[1] * 32, q=0, k=far["k"],
                          v=far["v"], out=far["out"]) == NULL
    assert lib.attn_decode_workspace_bytes(32, 63, 128, 32768) <= taf.ATTN_DECODE_SCRATCH_BYTES
    assert lib.attn_decode_workspace_bytes(16, 64, 128, 32768) <= taf.ATTN_DECODE_SCRATCH_BYTES


def test_decode_refuses_max_len_past_limit(lib):
    # Validated before any size arithmetic that could overflow; nothing is launched.
    assert decode(lib, max_len=2**31 - 1, ws_bytes=2**40) == OVF
    assert decode(lib, max_len=2**30 + 1, ws_bytes=2**40) == OVF


def scatter(lib, kn=A, vn=B_, kc=C_, vc=O_, lens=(0, 3), M=2, n_new=2, Hkv=2, d=64, max_len=8):
    arr = (ctypes.c_int32 * max(1, len(lens)))(*lens) if lens is not None else None
    return lib.kv_cache_scatter(kn, vn, kc, vc, arr, M, n_new, Hkv, d, max_len, None)


def test_scatter_validation(lib):
    assert scatter(lib, kn=0) == NULL
    assert scatter(lib, lens=None) == NULL
    assert scatter(lib, M=0, lens=(0,)) == DIM
    assert scatter(lib, M=33, lens=(0,) * 33) == DIM
    assert scatter(lib, n_new=0) == DIM
    assert scatter(lib, lens=(0, 7)) == DIM     # 7 + 2 > 8: the pages reject pos >= max_seq_len
    assert scatter(lib, lens=(-1, 0)) == DIM
    assert scatter(lib, d=16) == UNSUP
    assert scatter(lib, vc=O_ + 8) == UNSUP
    assert scatter(lib, n_new=2**20, Hkv=2**10, d=128, max_len=2**21, lens=(0, 0)) == OVF
    assert scatter(lib, vc=C_ + 256) == ALIAS   # the two caches overlap
    assert scatter(lib, kc=A) == ALIAS          # cache over the source


def cached(lib, q=A, kn=B_, vn=B_ + 0x1000000, kc=C_, vc=C_ + 0x8000000, lens=(0, 3), out=O_, M=2, n=4,
           H=8, Hkv=2, d=64, max_len=64, scale=0.125):
    arr = (ctypes.c_int32 * max(1, len(lens)))(*lens) if lens is not None else None
    return lib.attn_prefill_cached(q, kn, vn, kc, vc, arr, out, M, n, H, Hkv, d, max_len, scale, None)


def test_prefill_cached_validation(lib):
    assert cached(lib, q=0) == NULL
    assert cached(lib, lens=None) == NULL
    assert cached(lib, M=0, lens=(0,)) == DIM
    assert cached(lib, M=33, lens=(0,) * 33) == DIM
    assert cached(lib, n=0) == DIM
    assert cached(lib, Hkv=3) == DIM                 # 8 % 3 != 0
    assert cached(lib, lens=(0, 61)) == DIM          # 61 + 4 > 64
    assert cached(lib, lens=(-2, 0)) == DIM
    assert cached(lib, scale=float("inf")) == DIM
    assert cached(lib, d=48) == UNSUP
    assert cached(lib, kc=C_ + 4) == UNSUP
    assert cached(lib, n=2**16, H=2**10, Hkv=2**10, d=128, max_len=2**17, lens=(0, 0)) == OVF
    assert cached(lib, out=A + 64) == ALIAS          # out over q
    assert cached(lib, vc=C_ + 1024) == ALIAS        # the caches overlap
    assert cached(lib, kc=B_) == ALIAS               # cache over k_new


def cached_rope(lib, rot=32, theta=1e4, **kw):
    args = dict(q=A, kn=B_, vn=B_ + 0x1000000, kc=C_, vc=C_ + 0x8000000, lens=(0, 3), out=O_, M=2, n=4, H=8,
                Hkv=2, d=64, max_len=64, scale=0.125)
    args.update(kw)
    lens = args["lens"]
    arr = (ctypes.c_int32 * max(1, len(lens)))(*lens) if lens is not None else None
    return lib.attn_prefill_cached_rope(args["q"], args["kn"], args["vn"], args["kc"], args["vc"], arr, args["out"],
                                        args["M"], args["n"], args["H"], args["Hkv"], args["d"], args["max_len"],
                                        args["scale"], rot, theta, None)


def test_prefill_cached_rope_validation(lib):
    """The chunked prefill's refusals, then the rotary ones; nothing reaches HIP."""
    assert cached_rope(lib, q=0) == NULL
    assert cached_rope(lib, lens=None) == NULL
    assert cached_rope(lib, lens=(0, 61)) == DIM
    assert cached_rope(lib, d=48) == UNSUP
    assert cached_rope(lib, out=A + 64) == ALIAS
    assert cached_rope(lib, rot=-8) == DIM
    assert cached_rope(lib, rot=72) == DIM             # wider than head_dim 64
    assert cached_rope(lib, theta=0.0) == DIM
    assert cached_rope(lib, theta=float("nan")) == DIM
    assert cached_rope(lib, rot=12) == UNSUP           # not a multiple of 8


def test_scatter_rope_validation(lib):
    def call(rot=64, theta=10000.0, d=64, **kw):
        lens = kw.pop("lens", (0, 3))
        arr = (ctypes.c_int32 * len(lens))(*lens)
        args = dict(kn=A, vn=B_, kc=C_, vc=O_, M=2, n_new=2, Hkv=2, max_len=8)
        args.update(kw)
        return lib.kv_cache_scatter_rope(args["kn"], args["vn"], args["kc"], args["vc"], arr, args["M"],
                                         args["n_new"], args["Hkv"], d, args["max_len"], rot, theta, None)
    assert call(kn=0) == NULL
    assert call(lens=(0, 7)) == DIM              # the plain append's checks come first
    assert call(d=48) == UNSUP
    assert call(rot=-8) == DIM
    assert call(rot=72) == DIM                   # wider than head_dim 64
    assert call(theta=0.0) == DIM
    assert call(theta=-10000.0) == DIM
    assert call(theta=float("inf")) == DIM
    assert call(theta=float("nan")) == DIM
    assert call(rot=12) == UNSUP                 # not a multiple of 8
    assert call(rot=6) == UNSUP
    assert call(kc=A) == ALIAS


def test_decode_rope_validation(lib):
    def call(rot=128, theta=1e6, d=128, lens=(5, 100), ws_bytes=None, **kw):
        arr = (ctypes.c_int32 * len(lens))(*lens)
        M, H, Hkv, max_len = 2, 8, 2, 100
        if ws_bytes is None:
            ws_bytes = lib.attn_decode_workspace_bytes(M, H, 128, max_len)
        args = dict(q=A, k=B_, v=C_, out=O_, ws=W_)
        args.update(kw)
        return lib.attn_decode_gqa_batched_rope(args["q"], args["k"], args["v"], arr, args["out"], M, H, Hkv, d,
                                                max_len, 0.088, rot, theta, args["ws"], ws_bytes, None)
    assert call(q=0) == NULL
    assert call(lens=(101, 3)) == DIM
    assert call(d=96) == UNSUP
    assert call(ws_bytes=16) == WS
    assert call(out=A) == ALIAS
    assert call(rot=136) == DIM
    assert call(rot=-1) == DIM
    assert call(theta=0.0) == DIM
    assert call(theta=float("nan")) == DIM
    assert call(rot=4) == UNSUP
    assert call(rot=100) == UNSUP


def test_copy_to_slot_validation(lib):
    def call(sk=A, sv=B_, src_max=64, seq_len=10, kc=C_, vc=O_, slot=1, M=2, Hkv=4, d=64, max_len=32, lens=None):
        return lib.kv_cache_copy_to_slot(sk, sv, src_max, seq_len, kc, vc, slot, M, Hkv, d, max_len, lens, None)
    assert call(sk=0) == NULL
    assert call(vc=0) == NULL
    assert call(M=0) == DIM
    assert call(M=33, slot=0) == DIM
    assert call(slot=2) == DIM
    assert call(slot=-1) == DIM
    assert call(seq_len=33) == DIM             # more rows than the batched cache holds
    assert call(src_max=8) == DIM              # more rows than the single cache holds
    assert call(seq_len=-1) == DIM
    assert call(Hkv=0) == DIM
    assert call(d=80) == UNSUP
    assert call(kc=C_ + 8) == UNSUP
    assert call(Hkv=2**12, max_len=2**20, d=128, M=32, seq_len=1, src_max=1) == OVF
    assert call(vc=C_ + 64) == ALIAS           # caches overlap
    assert call(kc=A) == ALIAS                 # cache over the source
    lens = (ctypes.c_int32 * 2)(7, 7)
    assert call(slot=5, lens=lens) == DIM and list(lens) == [7, 7]


def test_lengths_reset_and_rollback(lib):
    """realizar reset_batched_kv_cache_gpu (all lengths 0) and rollback_kv_cache_gpu (lengths above
    `position` drop to it, shorter ones stay), on the host arrays the other entry points take."""
    lens = (ctypes.c_int32 * 5)(10, 3, 0, 7, 4096)
    assert lib.kv_lengths_rollback(lens, 5, 7) == OK
    assert list(lens) == [7, 3, 0, 7, 7]
    assert lib.kv_lengths_rollback(lens, 5, 0) == OK
    assert list(lens) == [0, 0, 0, 0, 0]
    lens = (ctypes.c_int32 * 3)(5, 6, 7)
    assert lib.kv_lengths_rollback(lens, 3, -1) == DIM and list(lens) == [5, 6, 7]
    assert lib.kv_lengths_rollback(lens, 0, 1) == DIM
    assert lib.kv_lengths_rollback(None, 3, 1) == NULL
    assert lib.kv_lengths_reset(lens, 3) == OK and list(lens) == [0, 0, 0]
    assert lib.kv_lengths_reset(lens, 33) == DIM
    assert lib.kv_lengths_reset(None, 1) == NULL
    # The Python binding updates a list in place.
    py = [9, 2, 11]
    taf.kv_lengths_rollback(py, 3, 4)
    assert py == [4, 2, 4]
    taf.kv_lengths_reset(py, 3)
    assert py == [0, 0, 0]


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4 * 32, dtype=torch.float32)
    with pytest.raises(ValueError):
        taf.attn_prefill(x, x, x, x, 1, 1, 4, 32, 0.1, False)
