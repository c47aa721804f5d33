"""Property-based fuzz of the C ABI's host validation (CPU only, no GPU call).

Every generated call carries at least one argument that makes it invalid (a NULL
pointer, a head_dim outside {32, 64, 128}, a non-finite scale, a zero or negative
size, a sequence count outside [1, 32], ...), while every other argument is drawn
freely, including the int32 extremes and misaligned or overlapping pointers.  The
header promises that every argument is validated on the host before anything is
enqueued, so each call must return one of the validation statuses: never OK and
never ATTN_ERR_HIP (which would mean it got as far as the HIP runtime), and it must
not crash.  Pointers are fake addresses that are never dereferenced; host length
arrays hold 64 entries, more than any valid sequence count.
"""
import ctypes

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import transformer_attention_flash_amd as taf  # noqa: E402

OK, NULL, DIM, UNSUP, OVF, WS, HIP, ALIAS = range(8)
REFUSALS = {NULL, DIM, UNSUP, OVF, WS, ALIAS}

SETTINGS = settings(max_examples=300, deadline=None, derandomize=True, database=None)

ints = st.one_of(st.sampled_from([0, 1, 2, 3, 4, 8, 31, 32, 33, 64, 100, 128, 4096, 2**30, 2**31 - 1, -1,
                                  -2**31]),
                 st.integers(min_value=-2**31, max_value=2**31 - 1))
small = st.integers(min_value=1, max_value=40)
dims = st.sampled_from([32, 64, 128, 0, 16, 48, 96, 256, -64])
ptrs = st.sampled_from([0x10000, 0x20000000, 0x40000000, 0x60000000, 0x80000000, 0x10004, 0x20000008, 0x10040])
floats = st.one_of(st.sampled_from([0.125, 1.0, -0.5, 0.0, float("inf"), -float("inf"), float("nan"), 1e38]),
                   st.floats(allow_nan=True, allow_infinity=True, width=32))


@pytest.fixture(scope="module")
def lib():
    return taf.library()


def lens_array(values):
    vals = list(values)[:64]
    return (ctypes.c_int32 * 64)(*(vals + [0] * (64 - len(vals))))


def refused(status, what):
    assert status in REFUSALS, f"{what}: status {status} ({taf.attn_status_string(status)})"


# Each poison makes a call invalid whatever the other arguments are.
PREFILL_POISONS = ["q", "k", "v", "out", "batch", "seq", "heads", "dim", "causal", "scale"]


@SETTINGS
@given(data=st.data())
def test_prefill_refuses_invalid_calls(lib, data):
    a = dict(q=data.draw(ptrs), k=data.draw(ptrs), v=data.draw(ptrs), out=data.draw(ptrs), b=data.draw(ints),
             s=data.draw(ints), h=data.draw(ints), d=data.draw(dims), scale=data.draw(floats),
             causal=data.draw(st.sampled_from([0, 1, 2, -1])))
    poison = data.draw(st.sampled_from(PREFILL_POISONS + ["precision"]))
    lowp = poison == "precision" or data.draw(st.booleans())
    prec = data.draw(st.sampled_from([1, 2]))
    if poison in ("q", "k", "v", "out"):
        a[poison] = 0
    elif poison == "batch":
        a["b"] = data.draw(st.integers(min_value=-2**31, max_value=0))
    elif poison == "seq":
        a["s"] = data.draw(st.integers(min_value=-2**31, max_value=0))
    elif poison == "heads":
        a["h"] = data.draw(st.integers(min_value=-2**31, max_value=0))
    elif poison == "dim":
        a["d"] = data.draw(st.sampled_from([0, 16, 48, 96, 256, -128]))
    elif poison == "causal":
        a["causal"] = data.draw(st.sampled_from([2, -1, 7]))
    elif poison == "scale":
        a["scale"] = data.draw(st.sampled_from([float("nan"), float("inf"), -float("inf")]))
    else:
        prec = data.draw(st.sampled_from([0, 3, -1]))
    if lowp:
        st_ = lib.attn_prefill_lowp(a["q"], a["k"], a["v"], a["out"], a["b"], a["s"], a["h"], a["d"], a["scale"],
                                    a["causal"], prec, None)
    else:
        st_ = lib.attn_prefill(a["q"], a["k"], a["v"], a["out"], a["b"], a["s"], a["h"], a["d"], a["scale"],
                               a["causal"], None)
    refused(st_, f"prefill (lowp={lowp}) poisoned by {poison}: {a}")


@SETTINGS
@given(data=st.data())
def test_decode_refuses_invalid_calls(lib, data):
    M = data.draw(st.one_of(small, ints))
    a = dict(q=data.draw(ptrs), k=data.draw(ptrs), v=data.draw(ptrs), out=data.draw(ptrs), ws=data.draw(ptrs),
             H=data.draw(st.one_of(small, ints)), Hkv=data.draw(st.one_of(small, ints)), d=data.draw(dims),
             max_len=data.draw(st.one_of(st.integers(1, 5000), ints)), scale=data.draw(floats),
             ws_bytes=data.draw(st.sampled_from([0, 16, 2**20, 2**30, 2**40])), rot=data.draw(st.sampled_from(
                 [0, 8, 64, 128, -8, 12])), theta=data.draw(floats))
    lens = data.draw(st.lists(st.one_of(st.integers(0, 5000), ints), min_size=0, max_size=64))
    poison = data.draw(st.sampled_from(["q", "k", "v", "out", "ws", "lens_ptr", "M", "H", "Hkv", "max_len",
                                        "dim", "scale", "len"]))
    arr = lens_array(lens)
    if poison in ("q", "k", "v", "out", "ws"):
        a[poison] = 0
    elif poison == "lens_ptr":
        arr = None
    elif poison == "M":
        M = data.draw(st.sampled_from([0, -1, 33, 2**31 - 1, -2**31]))
    elif poison == "H":
        a["H"] = data.draw(st.integers(min_value=-2**31, max_value=0))
    elif poison == "Hkv":
        a["Hkv"] = data.draw(st.integers(min_value=-2**31, max_value=0))
    elif poison == "max_len":
        a["max_len"] = data.draw(st.integers(min_value=-2**31, max_value=0))
    elif poison == "dim":
        a["d"] = data.draw(st.sampled_from([0, 16, 48, 96, 256]))
    elif poison == "scale":
        a["scale"] = data.draw(st.sampled_from([float("nan"), float("inf")]))
    else:  # one length out of [0, max_len]: M must be valid for the lengths to be read
        M = data.draw(st.integers(1, 32))
        i = data.draw(st.integers(0, M - 1))
        arr[i] = data.draw(st.sampled_from([-1, -2**31])) if a["max_len"] > 2**31 - 2 or data.draw(
            st.booleans()) else a["max_len"] + 1
    which = data.draw(st.sampled_from(["plain", "rope", "noalloc"]))
    if which == "plain":
        st_ = lib.attn_decode_gqa_batched(a["q"], a["k"], a["v"], arr, a["out"], M, a["H"], a["Hkv"], a["d"],
                                          a["max_len"], a["scale"], a["ws"], a["ws_bytes"], None)
    elif which == "rope":
        st_ = lib.attn_decode_gqa_batched_rope(a["q"], a["k"], a["v"], arr, a["out"], M, a["H"], a["Hkv"], a["d"],
                                               a["max_len"], a["scale"], a["rot"], a["theta"], a["ws"],
                                               a["ws_bytes"], None)
    else:
        if poison == "ws":  # no workspace argument: poison the query instead
            a["q"] = 0
        st_ = lib.attn_decode_gqa_batched_noalloc(a["q"], a["k"], a["v"], arr, a["out"], M, a["H"], a["Hkv"],
                                                  a["d"], a["max_len"], a["scale"], None)
    refused(st_, f"decode ({which}) poisoned by {poison}: M={M} {a}")


@SETTINGS
@given(data=st.data())
def test_append_and_chunked_prefill_refuse_invalid_calls(lib, data):
    M = data.draw(st.one_of(small, ints))
    a = dict(q=data.draw(ptrs), kn=data.draw(ptrs), vn=data.draw(ptrs), kc=data.draw(ptrs), vc=data.draw(ptrs),
             out=data.draw(ptrs), n=data.draw(st.one_of(small, ints)), H=data.draw(st.one_of(small, ints)),
             Hkv=data.draw(st.one_of(small, ints)), d=data.draw(dims),
             max_len=data.draw(st.one_of(st.integers(1, 5000), ints)), scale=data.draw(floats),
             rot=data.draw(st.sampled_from([0, 8, 64, -8, 12])), theta=data.draw(floats))
    lens = data.draw(st.lists(st.one_of(st.integers(0, 5000), ints), min_size=0, max_size=64))
    poison = data.draw(st.sampled_from(["kn", "vn", "kc", "vc", "lens_ptr", "M", "n", "Hkv", "max_len", "dim",
                                        "len"]))
    arr = lens_array(lens)
    if poison in ("kn", "vn", "kc", "vc"):
        a[poison] = 0
    elif poison == "lens_ptr":
        arr = None
    elif poison == "M":
        M = data.draw(st.sampled_from([0, -1, 33, 2**31 - 1, -2**31]))
    elif poison in ("n", "Hkv", "max_len"):
        a[poison] = data.draw(st.integers(min_value=-2**31, max_value=0))
    elif poison == "dim":
        a["d"] = data.draw(st.sampled_from([0, 16, 48, 96, 256]))
    else:  # one write start negative: M must be valid for the lengths to be read
        M = data.draw(st.integers(1, 32))
        arr[data.draw(st.integers(0, M - 1))] = data.draw(st.sampled_from([-1, -2**31]))
    which = data.draw(st.sampled_from(["scatter", "scatter_rope", "cached", "cached_rope"]))
    if which == "scatter":
        st_ = lib.kv_cache_scatter(a["kn"], a["vn"], a["kc"], a["vc"], arr, M, a["n"], a["Hkv"], a["d"],
                                   a["max_len"], None)
    elif which == "scatter_rope":
        st_ = lib.kv_cache_scatter_rope(a["kn"], a["vn"], a["kc"], a["vc"], arr, M, a["n"], a["Hkv"], a["d"],
                                        a["max_len"], a["rot"], a["theta"], None)
    elif which == "cached":
        st_ = lib.attn_prefill_cached(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], arr, a["out"], M, a["n"], a["H"],
                                      a["Hkv"], a["d"], a["max_len"], a["scale"], None)
    else:
        st_ = lib.attn_prefill_cached_rope(a["q"], a["kn"], a["vn"], a["kc"], a["vc"], arr, a["out"], M, a["n"],
                                           a["H"], a["Hkv"], a["d"], a["max_len"], a["scale"], a["rot"],
                                           a["theta"], None)
    refused(st_, f"{which} poisoned by {poison}: M={M} {a}")
