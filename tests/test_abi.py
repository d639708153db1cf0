"""The C ABI without a GPU: libpa.so loads, exports every function include/pa.h
declares, and rejects bad arguments on the host before any HIP call.

A rejected call returns its status before touching the device, so these run
in a container without a GPU.  Valid calls are never made here.
"""

import ctypes
import os
import re

import pytest

from paged_kv_cache_hkv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libpa.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ["pa_metadata_build", "pa_cache_write", "pa_decode", "pa_prefill_varlen"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(B.EXPORTED)


def test_status_strings():
    assert B.status_string(B.PA_OK) == "PA_OK"
    assert B.status_string(B.PA_ERR_WORKSPACE_TOO_SMALL) == "PA_ERR_WORKSPACE_TOO_SMALL"


def _desc(**kw):
    base = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, act_dtype=B.PA_BF16)
    base.update(kw)
    return B.make_desc(**base)


FAKE = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: every call below fails its checks


def _write(desc, num_tokens=4, key=FAKE, stride=1024, kc=FAKE):
    lib = B.load()
    return lib.pa_cache_write(ctypes.byref(desc), num_tokens, key, stride, FAKE, stride, FAKE,
                              kc, FAKE, 100, None)


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=30, num_kv_heads=8), B.PA_ERR_INVALID_ARG),   # Hq % Hkv != 0
    (dict(num_kv_heads=0), B.PA_ERR_INVALID_ARG),
    (dict(head_dim=96), B.PA_ERR_UNSUPPORTED),
    (dict(block_size=32), B.PA_ERR_UNSUPPORTED),
    (dict(act_dtype=B.PA_FP8_E4M3), B.PA_ERR_UNSUPPORTED),
    (dict(act_dtype=7), B.PA_ERR_INVALID_ARG),
    (dict(act_dtype=B.PA_F16, cache_dtype=B.PA_BF16), B.PA_ERR_UNSUPPORTED),
    (dict(cache_dtype=B.PA_FP8_E4M3, k_scale=0.0), B.PA_ERR_INVALID_ARG),
    (dict(cache_dtype=B.PA_FP8_E4M3, v_scale=float("nan")), B.PA_ERR_INVALID_ARG),
    (dict(act_dtype=B.PA_INT8), B.PA_ERR_UNSUPPORTED),
    (dict(cache_dtype=B.PA_INT8, k_scale=-1.0), B.PA_ERR_INVALID_ARG),
    (dict(cache_dtype=B.PA_INT8, v_scale=float("inf")), B.PA_ERR_INVALID_ARG),
    (dict(cache_dtype=4), B.PA_ERR_INVALID_ARG),
    (dict(decode_workers=-1), B.PA_ERR_INVALID_ARG),
    (dict(softmax_scale=float("inf")), B.PA_ERR_INVALID_ARG),
    # masked scores are -inf before the scale: 0 * -inf is NaN, a negative scale gives +inf
    (dict(softmax_scale=0.0), B.PA_ERR_INVALID_ARG),
    (dict(softmax_scale=-0.125), B.PA_ERR_INVALID_ARG),
    (dict(softmax_scale=-0.0), B.PA_ERR_INVALID_ARG),
])
def test_desc_rejections(kw, status):
    assert _write(_desc(**kw)) == status


class _Ptr:
    """A fake device array: only its address is passed (the calls fail first)."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


@pytest.mark.parametrize("kw", [
    dict(k_scales=_Ptr(1 << 20)),                                   # per-head scales, 16-bit cache
    dict(v_scales=_Ptr(1 << 20)),
    dict(cache_dtype=B.PA_INT8, k_scales=_Ptr((1 << 20) + 2)),      # not float32-aligned
    dict(cache_dtype=B.PA_FP8_E4M3, v_scales=_Ptr((1 << 20) + 1)),
])
def test_head_scale_rejections(kw):
    assert _write(_desc(**kw)) == B.PA_ERR_INVALID_ARG


def test_head_scales_accepted_with_quantized_cache():
    # aligned per-head scales on an 8-bit cache pass the descriptor checks (the
    # call then stops at its own argument check: a null key)
    d = _desc(cache_dtype=B.PA_INT8, k_scales=_Ptr(1 << 20), v_scales=_Ptr(1 << 21))
    assert _write(d, key=None) == B.PA_ERR_INVALID_ARG
    assert _write(d, num_tokens=0) == B.PA_OK


def test_cache_write_argument_checks():
    d = _desc()
    assert _write(d, key=None) == B.PA_ERR_INVALID_ARG
    assert _write(d, key=ctypes.c_void_p((1 << 20) + 2)) == B.PA_ERR_INVALID_ARG  # misaligned
    assert _write(d, stride=1000) == B.PA_ERR_INVALID_ARG                        # < Hkv*D
    assert _write(d, stride=1028) == B.PA_ERR_INVALID_ARG                        # not 16-byte
    assert _write(d, num_tokens=-1) == B.PA_ERR_INVALID_ARG
    assert _write(d, num_tokens=0) == B.PA_OK                                    # nothing to do


def test_metadata_argument_checks():
    lib = B.load()
    f = lambda R, qsl_len, T=4, qsl=FAKE: lib.pa_metadata_build(
        R, 16, 8, T, qsl_len, FAKE, FAKE, FAKE, qsl, FAKE, FAKE, FAKE, None)
    assert f(3, 3) == B.PA_ERR_INVALID_ARG        # qsl buffer shorter than R + 1
    assert f(-1, 4) == B.PA_ERR_INVALID_ARG
    assert f(3, 4, qsl=None) == B.PA_ERR_INVALID_ARG
    assert f(3, 4, T=-2) == B.PA_ERR_INVALID_ARG


def test_decode_checks_and_workspace_query():
    lib = B.load()
    d = _desc()
    # size query is host-only
    assert B.pa_decode_workspace_size(d, 256, 8193, 513) > 0
    # fixed worker count: prefix (int64, R+1), 2 slots per workgroup (4 workers each for a
    # 16-bit cache) of G*(D+2) floats, 1 per worker of G*D floats, in 256-aligned parts
    d8 = _desc(decode_workers=8)
    rup = lambda x: (x + 255) // 256 * 256
    G, D = 4, 128
    wg_slots, w_slots = 2 * 2, 8
    assert B.pa_decode_workspace_size(d8, 4, 100, 8) == (
        rup(5 * 8) + rup(wg_slots * G * D * 4) + rup(wg_slots * G * 2 * 4) + rup(w_slots * G * D * 4))
    assert B.pa_decode_workspace_size(d8, 0, 100, 8) == 0
    big = _desc(num_q_heads=64, num_kv_heads=1)
    with pytest.raises(B.PaError) as e:
        B.pa_decode_workspace_size(big, 4, 100, 8)
    assert e.value.status == B.PA_ERR_UNSUPPORTED              # G = 64 > 32
    call = lambda ws, ws_bytes, q=FAKE: lib.pa_decode(
        ctypes.byref(d), 0, 256, q, 4096, FAKE, FAKE, FAKE, 513, FAKE, FAKE, 1000, 8193,
        ws, ws_bytes, FAKE, 4096, None)
    assert call(None, 0) == B.PA_ERR_WORKSPACE_TOO_SMALL
    assert call(FAKE, 16) == B.PA_ERR_WORKSPACE_TOO_SMALL
    assert call(FAKE, 1 << 40, q=None) == B.PA_ERR_INVALID_ARG
    bad_range = lib.pa_decode(ctypes.byref(d), 5, 2, FAKE, 4096, FAKE, FAKE, FAKE, 8, FAKE, FAKE,
                              10, 100, None, 0, FAKE, 4096, None)
    assert bad_range == B.PA_ERR_INVALID_ARG


def test_decode_noalloc_checks():
    """The no-allocation decode validates like pa_decode and refuses, before any
    device work, a call whose workspace would not fit the library's array."""
    lib = B.load()
    d = _desc()
    call = lambda desc, q=FAKE, begin=0, end=256, stride=8192: lib.pa_decode_noalloc(
        ctypes.byref(desc), begin, end, q, stride, FAKE, FAKE, FAKE, 513, FAKE, FAKE, 1000, 8193,
        FAKE, stride, None)
    assert call(d, q=None) == B.PA_ERR_INVALID_ARG
    assert call(d, begin=5, end=2) == B.PA_ERR_INVALID_ARG
    assert call(d, begin=7, end=7) == B.PA_OK                      # empty range: nothing to do
    # 2^20 workers' slots of G = 4 x (128 + 2) floats: far beyond the 64 MiB array
    huge = _desc(decode_workers=1 << 20)
    assert B.pa_decode_workspace_size(huge, 256, 8193, 513) > (64 << 20)
    assert call(huge) == B.PA_ERR_WORKSPACE_TOO_SMALL
    assert call(_desc(num_q_heads=64, num_kv_heads=1)) == B.PA_ERR_UNSUPPORTED   # G > 32


def test_prefill_checks():
    lib = B.load()
    d = _desc()
    f = lambda q_stride=4096, out_stride=4096, mq=10: lib.pa_prefill_varlen(
        ctypes.byref(d), 0, 3, FAKE, q_stride, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 100, mq, 100,
        FAKE, out_stride, None)
    assert f(q_stride=4000) == B.PA_ERR_INVALID_ARG
    assert f(out_stride=4092) == B.PA_ERR_INVALID_ARG
    assert f(mq=-1) == B.PA_ERR_INVALID_ARG
    assert f(mq=0) == B.PA_OK                                 # no query rows: nothing launched
    # positions must stay below 2^30 (a window of 2^30 or more keys is then no window)
    long = lambda ms: lib.pa_prefill_varlen(
        ctypes.byref(d), 0, 3, FAKE, 4096, FAKE, FAKE, FAKE, 8, FAKE, FAKE, 100, 10, ms,
        FAKE, 4096, None)
    assert long((1 << 30) + 1) == B.PA_ERR_UNSUPPORTED
    dlong = lib.pa_decode(ctypes.byref(d), 0, 3, FAKE, 4096, FAKE, FAKE, FAKE, 8, FAKE, FAKE,
                          100, (1 << 30) + 1, FAKE, 1 << 40, FAKE, 4096, None)
    assert dlong == B.PA_ERR_UNSUPPORTED


def test_rope_cache_write_checks():
    lib = B.load()
    d = _desc()

    def f(T=4, rd=128, neox=1, maxpos=4096, cs=FAKE, q=FAKE, qs=4096, ks=1024, dd=d):
        return lib.pa_rope_cache_write(ctypes.byref(dd), T, FAKE, cs, maxpos, rd, neox, q, qs,
                                       FAKE, ks, FAKE, ks, FAKE, FAKE, FAKE, 100, None)
    assert f(rd=0) == B.PA_ERR_INVALID_ARG
    assert f(rd=7) == B.PA_ERR_INVALID_ARG          # odd
    assert f(rd=256) == B.PA_ERR_INVALID_ARG        # > head_dim
    assert f(rd=40) == B.PA_ERR_UNSUPPORTED         # even but not a multiple of 16
    assert f(neox=2) == B.PA_ERR_INVALID_ARG
    assert f(maxpos=0) == B.PA_ERR_INVALID_ARG
    assert f(T=-1) == B.PA_ERR_INVALID_ARG
    assert f(cs=None) == B.PA_ERR_INVALID_ARG
    assert f(cs=ctypes.c_void_p((1 << 20) + 4)) == B.PA_ERR_INVALID_ARG   # table not 16-byte aligned
    assert f(q=None) == B.PA_ERR_INVALID_ARG
    assert f(qs=1024) == B.PA_ERR_INVALID_ARG       # query row stride < Hq*D
    assert f(ks=100) == B.PA_ERR_INVALID_ARG
    assert f(dd=_desc(head_dim=96)) == B.PA_ERR_UNSUPPORTED
    assert f(T=0) == B.PA_OK                        # nothing to do


def test_copy_blocks_checks():
    lib = B.load()
    d = _desc()

    def f(sk=FAKE, dk=FAKE, pairs=FAKE, n=4, snb=100, dnb=100, dd=d):
        return lib.pa_copy_blocks(ctypes.byref(dd), sk, FAKE, snb, dk, FAKE, dnb, pairs, n, None)
    assert f(n=-1) == B.PA_ERR_INVALID_ARG
    assert f(snb=-1) == B.PA_ERR_INVALID_ARG
    assert f(dnb=-5) == B.PA_ERR_INVALID_ARG
    assert f(sk=None) == B.PA_ERR_INVALID_ARG
    assert f(pairs=None) == B.PA_ERR_INVALID_ARG
    assert f(dk=ctypes.c_void_p((1 << 20) + 8)) == B.PA_ERR_INVALID_ARG   # cache not 16-byte aligned
    assert f(pairs=ctypes.c_void_p((1 << 20) + 4)) == B.PA_ERR_INVALID_ARG  # pairs not 8-byte aligned
    assert f(n=1 << 31) == B.PA_ERR_UNSUPPORTED
    assert f(dd=_desc(num_kv_heads=0)) == B.PA_ERR_INVALID_ARG
    assert f(n=0, sk=None) == B.PA_OK             # nothing to do: no pointer is looked at
    # an address no allocation owns: rejected by the pointer query, nothing launched
    assert f() == B.PA_ERR_INVALID_ARG
