"""Paged causal attention of the oracle (test infrastructure only).

What is computed (the plain definition; float64 throughout):

For request ``r`` with ``n_r = query_start_loc[r+1] - query_start_loc[r]`` new
tokens and ``s_r = seq_lens[r]`` keys in total, the ``c_r = s_r - n_r`` tokens
cached before this step come first ("Tour: One forward pass", stop 3:
``seq_lens = num_computed_tokens + query_len``, positions start at
``num_computed_tokens``).  Its logical key ``j`` lives in physical block
``block_table[r][j // block_size]`` at offset ``j % block_size`` of the global
cache ``[num_blocks, block_size, num_kv_heads, head_size]`` ("vLLM MHA Code
Path", "Cache write and cache read use different maps": the block table is the
request-to-page gather map; "vLLM 推理全流程深度解析", the PagedAttention decode
kernel reads each sequence's blocks through ``block_tables``).

Query ``i`` of the request sits at position ``c_r + i`` and attends to keys
``j = 0 .. c_r + i``: the current token attends to itself and future positions
are masked ("vLLM MHA Code Path", Worked Trace step 10 remark; "Tour: One
forward pass", stop 10: R1 reads 541 keys, R2 130, R3's rows together 298).
Query head ``h`` reads K/V head ``h // G`` with ``G = Hq / Hkv`` ("vLLM MHA Code
Path", "One Path Covers MHA, GQA, and MQA": Hq must be a multiple of Hkv, so
each K/V head serves G query heads).  Scores are ``q . k * scale`` and the row
is ``softmax(scores) @ V``.

Readings where the pages are silent: the alignment of the causal mask for a
cached prefix is bottom-right (it follows from the positions); ``scale`` is
``1/sqrt(head_size)`` unless the caller passes another; query head ``h`` maps to
K/V head ``h // G`` (contiguous groups).

Mask variants.  "Tour: One forward pass", stop 10, shows the kernel call with
``alibi_slopes`` and ``window_size`` arguments, and "vLLM MHA Code Path"
(Worked Trace step 10) speaks of the causal/window rules; "vLLM 推理全流程深度解析"
lists ALiBi beside RoPE as a position encoding that uses the token positions.
The pages define neither, so the plain readings are taken:
* sliding window ``W`` (0 = none): query at position ``p`` attends keys
  ``j`` with ``p - W < j <= p`` -- the ``W`` most recent positions, itself
  included;
* ALiBi: query head ``h`` adds ``slope[h] * (j - p)`` (zero for the key at the
  query's own position, more negative the older the key) to the scaled score
  ``q . k * scale`` before the softmax; the caller gives the slopes.

Absent blocks (a defensive reading; the pages only ever hand out pool blocks):
a block-table entry that is not a block of the pool (negative, or not below
``num_blocks``) holds no keys -- its keys take no part in any softmax, and a
query row left with no visible key is zero.
"""

import math

import numpy as np

from . import codecs


def gather_request_kv(key_cache_f64, value_cache_f64, block_table_row, seq_len, block_size):
    """Logical K/V of one request: [seq_len, Hkv, D] each, through its block-table row."""
    hkv, d = key_cache_f64.shape[2], key_cache_f64.shape[3]
    k = np.empty((seq_len, hkv, d), dtype=np.float64)
    v = np.empty((seq_len, hkv, d), dtype=np.float64)
    for j in range(0, seq_len, block_size):
        blk = int(block_table_row[j // block_size])
        cnt = min(block_size, seq_len - j)
        k[j:j + cnt] = key_cache_f64[blk, :cnt]
        v[j:j + cnt] = value_cache_f64[blk, :cnt]
    return k, v


def causal_attention(q, k, v, num_computed, scale, sliding_window=0, alibi_slopes=None,
                     key_present=None):
    """Dense causal attention of one request in float64.

    q: [n, Hq, D]; k, v: [s, Hkv, D] with s = num_computed + n.
    Row i (position p = num_computed + i) attends keys 0 .. p, or only
    p - sliding_window + 1 .. p when sliding_window > 0; with alibi_slopes
    ([Hq]) head h adds slope[h] * (j - p) to the score of key j.
    key_present: bool [s] or None; keys marked False are left out, and a row
    with no key left is zero.
    Returns [n, Hq, D].
    """
    n, hq, d = q.shape
    s, hkv, _ = k.shape
    g = hq // hkv
    out = np.empty((n, hq, d), dtype=np.float64)
    if n == 0:
        return out
    key_idx = np.arange(s)[None, :]
    last_key = (num_computed + np.arange(n))[:, None]
    allowed = key_idx <= last_key                         # [n, s]
    if sliding_window > 0:
        allowed &= key_idx > last_key - sliding_window
    if key_present is not None:
        allowed &= np.asarray(key_present, dtype=bool)[None, :]
    empty = ~allowed.any(axis=1)                          # rows with no visible key
    for h in range(hq):
        kv = h // g
        scores = (q[:, h, :] @ k[:, kv, :].T) * scale     # [n, s]
        if alibi_slopes is not None:
            scores = scores + float(alibi_slopes[h]) * (key_idx - last_key)
        scores = np.where(allowed, scores, -np.inf)
        mx = scores.max(axis=1, keepdims=True)
        mx = np.where(empty[:, None], 0.0, mx)
        p = np.exp(scores - mx)
        p = np.where(allowed, p, 0.0)
        den = p.sum(axis=1, keepdims=True)
        p /= np.where(empty[:, None], 1.0, den)
        out[:, h, :] = p @ v[:, kv, :]
    return out


def decode_cache(cache_bits, cache_dtype, scale=1.0):
    """Stored cache bits [..., Hkv, D] -> float64 values (fp8 and int8 codes
    are multiplied by the tensor's scale, or by their K/V head's when ``scale``
    is an array [Hkv])."""
    vals = codecs.decode(cache_bits, cache_dtype)
    if cache_dtype in ("fp8_e4m3", "int8"):
        sc = np.asarray(scale, dtype=np.float64)
        vals = vals * (sc[:, None] if sc.ndim == 1 else sc)
    return vals


def paged_attention(q, key_cache, value_cache, block_tables, query_start_loc, seq_lens,
                    block_size, scale=None, requests=None, cache_dtype=None,
                    k_scale=1.0, v_scale=1.0, sliding_window=0, alibi_slopes=None,
                    num_blocks=None):
    """Attention of a batch over the paged cache, one request at a time.

    q: float64 [T, Hq, D] (already decoded).
    key_cache/value_cache: float64 [num_blocks, block_size, Hkv, D] (decoded), or
      raw bits when ``cache_dtype`` is given ('f16' | 'bf16' | 'fp8_e4m3' | 'int8'); raw
      bits are decoded per request, so a large pool is never widened at once.
    requests: iterable of request indices to compute (default: all).
    k_scale/v_scale: the quantized formats' scale of the tensor, or one per
      K/V head (array [Hkv]).
    sliding_window, alibi_slopes: the mask variants of ``causal_attention``.
    num_blocks: pool size; when given, table entries outside [0, num_blocks)
      are absent blocks (their keys are left out; K/V read as zeros).
    Returns {r: float64 [n_r, Hq, D]}.
    """
    d = q.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    num_reqs = len(seq_lens)
    if requests is None:
        requests = range(num_reqs)
    result = {}
    for r in requests:
        start, end = int(query_start_loc[r]), int(query_start_loc[r + 1])
        n = end - start
        s = int(seq_lens[r])
        c = s - n
        nb = -(-s // block_size)
        ids = np.asarray(list(block_tables[r][:nb]), dtype=np.int64)
        present_blk = np.ones(nb, dtype=bool)
        if num_blocks is not None:
            present_blk = (ids >= 0) & (ids < num_blocks)
        safe = np.where(present_blk, ids, 0)
        if not present_blk.any():
            kb = vb = np.zeros((nb,) + tuple(key_cache.shape[1:]), dtype=np.float64)
        elif cache_dtype is None:
            kb, vb = key_cache[safe], value_cache[safe]
        else:
            kb = decode_cache(key_cache[safe], cache_dtype, k_scale)
            vb = decode_cache(value_cache[safe], cache_dtype, v_scale)
        kb = np.where(present_blk[:, None, None, None], kb, 0.0)
        vb = np.where(present_blk[:, None, None, None], vb, 0.0)
        k, v = gather_request_kv(kb, vb, np.arange(nb), s, block_size)
        key_present = None
        if num_blocks is not None:
            key_present = np.repeat(present_blk, block_size)[:s]
        result[r] = causal_attention(q[start:end], k, v, c, scale, sliding_window, alibi_slopes,
                                     key_present)
    return result
