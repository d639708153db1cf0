"""Thin Python binding of libpa.so (include/pa.h).

Argument marshalling only: torch tensors become device pointers and the
current HIP stream; every step of the path runs in the library's kernels.  The
functions keep the C names and raise ``PaError`` on any status other than
PA_OK.  There is no fallback: if libpa.so is missing, loading raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE_TOO_SMALL, PA_ERR_HIP = range(5)
PA_F16, PA_BF16, PA_FP8_E4M3, PA_INT8 = 0, 1, 2, 3

DTYPE_CODE = {torch.float16: PA_F16, torch.bfloat16: PA_BF16, torch.float8_e4m3fn: PA_FP8_E4M3,
              torch.uint8: PA_FP8_E4M3, torch.int8: PA_INT8}


class PaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("cache_dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("decode_workers", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32),
        ("alibi_slopes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
    ]


def make_desc(num_q_heads, num_kv_heads, head_dim, block_size=16, act_dtype=PA_BF16,
              cache_dtype=None, softmax_scale=None, k_scale=1.0, v_scale=1.0,
              decode_workers=0, sliding_window=0, alibi_slopes=None, k_scales=None,
              v_scales=None):
    """alibi_slopes: float32 device tensor [num_q_heads] or None; k_scales /
    v_scales: float32 device tensors [num_kv_heads] (per-head scales of a
    quantized cache) or None.  The descriptor keeps references so the memory
    outlives it."""
    if cache_dtype is None:
        cache_dtype = act_dtype
    if softmax_scale is None:
        softmax_scale = head_dim ** -0.5
    ptr = lambda t: None if t is None else t.data_ptr()
    d = AttnDesc(num_q_heads, num_kv_heads, head_dim, block_size, act_dtype, cache_dtype,
                 softmax_scale, k_scale, v_scale, decode_workers, sliding_window,
                 ptr(alibi_slopes), ptr(k_scales), ptr(v_scales))
    d._refs = (alibi_slopes, k_scales, v_scales)
    return d


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

# name -> (argtypes)
_SIGS = {
    "pa_status_string": [ctypes.c_int],
    "pa_metadata_build": [_I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P],
    "pa_cache_write": [ctypes.POINTER(AttnDesc), _I64, _P, _I64, _P, _I64, _P, _P, _P, _I64, _P],
    "pa_rope_cache_write": [ctypes.POINTER(AttnDesc), _I64, _P, _P, _I64, _I32, _I32, _P, _I64, _P,
                            _I64, _P, _I64, _P, _P, _P, _I64, _P],
    "pa_copy_blocks": [ctypes.POINTER(AttnDesc), _P, _P, _I64, _P, _P, _I64, _P, _I64, _P],
    "pa_decode": [ctypes.POINTER(AttnDesc), _I32, _I32, _P, _I64, _P, _P, _P, _I32, _P, _P, _I64,
                  _I32, _P, _SZ, _P, _I64, _P],
    "pa_decode_noalloc": [ctypes.POINTER(AttnDesc), _I32, _I32, _P, _I64, _P, _P, _P, _I32, _P, _P,
                          _I64, _I32, _P, _I64, _P],
    "pa_decode_workspace_size": [ctypes.POINTER(AttnDesc), _I32, _I32, _I32, ctypes.POINTER(_SZ)],
    "pa_prefill_varlen": [ctypes.POINTER(AttnDesc), _I32, _I32, _P, _I64, _P, _P, _P, _I32, _P, _P,
                          _I64, _I32, _I32, _P, _I64, _P],
}
EXPORTED = tuple(_SIGS)


def load(path=LIB_PATH):
    """Load libpa.so once; raise if it is missing (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m paged_kv_cache_hkv_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "pa_status_string" else ctypes.c_int
    _lib = lib
    return lib


def status_string(status):
    return load().pa_status_string(status).decode()


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, where):
    if status != PA_OK:
        raise PaError(status, where)


def _row_stride(t):
    """Row stride in elements of a [rows, heads, D] (or [rows, heads*D]) view."""
    return t.stride(0)


def pa_metadata_build(num_computed_tokens, query_lens, block_tables, query_start_loc, seq_lens,
                      positions, slot_mapping, block_size=16, stream=None):
    num_reqs = query_lens.shape[0]
    _check(load().pa_metadata_build(
        num_reqs, block_size, block_tables.shape[1], positions.shape[0], query_start_loc.shape[0],
        _ptr(num_computed_tokens), _ptr(query_lens), _ptr(block_tables),
        _ptr(query_start_loc), _ptr(seq_lens), _ptr(positions), _ptr(slot_mapping),
        _stream(stream)), "pa_metadata_build")


def pa_cache_write(desc, key, value, slot_mapping, key_cache, value_cache, num_tokens=None,
                   stream=None):
    if num_tokens is None:
        num_tokens = key.shape[0]
    _check(load().pa_cache_write(
        ctypes.byref(desc), num_tokens, _ptr(key), _row_stride(key), _ptr(value),
        _row_stride(value), _ptr(slot_mapping), _ptr(key_cache), _ptr(value_cache),
        key_cache.shape[0], _stream(stream)), "pa_cache_write")


def pa_rope_cache_write(desc, positions, cos_sin_cache, rotary_dim, is_neox, query, key, value,
                        slot_mapping, key_cache, value_cache, num_tokens=None, stream=None):
    """Rotate query (in place) and key by position, write rotated key and value to the cache."""
    if num_tokens is None:
        num_tokens = key.shape[0]
    _check(load().pa_rope_cache_write(
        ctypes.byref(desc), num_tokens, _ptr(positions), _ptr(cos_sin_cache),
        cos_sin_cache.shape[0], rotary_dim, 1 if is_neox else 0, _ptr(query), _row_stride(query),
        _ptr(key), _row_stride(key), _ptr(value), _row_stride(value), _ptr(slot_mapping),
        _ptr(key_cache), _ptr(value_cache), key_cache.shape[0], _stream(stream)),
        "pa_rope_cache_write")


def pa_copy_blocks(desc, src_key_cache, src_value_cache, dst_key_cache, dst_value_cache,
                   block_pairs, num_pairs=None, stream=None):
    """Copy block s of the source pool to block d of the destination pool for each
    (s, d) row of block_pairs (int64 [n, 2]); pools on the device or in pinned host memory."""
    if num_pairs is None:
        num_pairs = block_pairs.shape[0]
    _check(load().pa_copy_blocks(
        ctypes.byref(desc), _ptr(src_key_cache), _ptr(src_value_cache), src_key_cache.shape[0],
        _ptr(dst_key_cache), _ptr(dst_value_cache), dst_key_cache.shape[0], _ptr(block_pairs),
        num_pairs, _stream(stream)), "pa_copy_blocks")


def pa_decode_workspace_size(desc, num_reqs, max_seq_len, max_blocks_per_req):
    need = _SZ(0)
    _check(load().pa_decode_workspace_size(ctypes.byref(desc), num_reqs, max_seq_len,
                                           max_blocks_per_req, ctypes.byref(need)),
           "pa_decode_workspace_size")
    return need.value


def pa_decode(desc, req_begin, req_end, q, query_start_loc, seq_lens, block_tables, key_cache,
              value_cache, max_seq_len, workspace, out, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().pa_decode(
        ctypes.byref(desc), req_begin, req_end, _ptr(q), _row_stride(q), _ptr(query_start_loc),
        _ptr(seq_lens), _ptr(block_tables), block_tables.shape[1], _ptr(key_cache),
        _ptr(value_cache), key_cache.shape[0], max_seq_len, _ptr(workspace), ws_bytes,
        _ptr(out), _row_stride(out), _stream(stream)), "pa_decode")


def pa_decode_noalloc(desc, req_begin, req_end, q, query_start_loc, seq_lens, block_tables,
                      key_cache, value_cache, max_seq_len, out, stream=None):
    """pa_decode on the library's own per-GPU scratch array (no workspace argument)."""
    _check(load().pa_decode_noalloc(
        ctypes.byref(desc), req_begin, req_end, _ptr(q), _row_stride(q), _ptr(query_start_loc),
        _ptr(seq_lens), _ptr(block_tables), block_tables.shape[1], _ptr(key_cache),
        _ptr(value_cache), key_cache.shape[0], max_seq_len, _ptr(out), _row_stride(out),
        _stream(stream)), "pa_decode_noalloc")


def pa_prefill_varlen(desc, req_begin, req_end, q, query_start_loc, seq_lens, block_tables,
                      key_cache, value_cache, max_query_len, max_seq_len, out, stream=None):
    _check(load().pa_prefill_varlen(
        ctypes.byref(desc), req_begin, req_end, _ptr(q), _row_stride(q), _ptr(query_start_loc),
        _ptr(seq_lens), _ptr(block_tables), block_tables.shape[1], _ptr(key_cache),
        _ptr(value_cache), key_cache.shape[0], max_query_len, max_seq_len, _ptr(out),
        _row_stride(out), _stream(stream)), "pa_prefill_varlen")
