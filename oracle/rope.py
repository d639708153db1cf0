"""Rotary position embedding fused with the cache write, in the oracle
(test infrastructure only).

"Tour: One forward pass", stop 9 ("QKVParallelLinear and the rotary
embedding"): once the fused QKV output is split, q and k are turned by
RoPE using each token's position from stop 3; the per-position cosines and
sines come from the ``cos_sin_cache`` table and every head's pairs are rotated
by them.  The model takes the unscaled ``RotaryEmbedding``.  "vLLM MHA Code Path"
(worked decode trace, step 4) and the ``LlamaAttention`` listing of
"vLLM 推理全流程深度解析" give the same order: RoPE on Q and K, then
``reshape_and_cache`` of K and V, then attention.

Readings taken where the pages are silent (each is a parameter here):
* the table ``cos_sin_cache[position]`` holds ``rotary_dim/2`` cosines then
  ``rotary_dim/2`` sines (float32), built by the caller; ``cos_sin_table``
  builds the plain one, angle ``position * base**(-2j/rotary_dim)``;
* the rotated pairs are ``(j, j + rotary_dim/2)`` (``is_neox``, the
  half-split layout Llama uses) or ``(2j, 2j+1)`` (interleaved); dimensions at
  or past ``rotary_dim`` are left as they are;
* precision: the GPU computes in float32 with each product and each sum
  rounded once -- ``a' = (a*c) - (b*s)``, ``b' = (b*c) + (a*s)`` -- and rounds
  the result to the activation dtype (nearest even).  ``rotate_f32`` does
  exactly those float32 steps (NumPy float32 arithmetic is IEEE, and NumPy
  does not fuse multiply-add); ``rotate_f64`` is the exact rotation used to
  pin it;
* fusing does not change what is stored: the cache receives the rotated key
  rounded to the activation dtype (then fp8-encoded, for an fp8 cache), i.e.
  exactly "rotate, then ``cache.scatter``";
* a token whose position is outside ``[0, max_position)`` is left alone: its
  query row is not rotated and its K/V are not written.
"""

import numpy as np

from . import cache, codecs


def cos_sin_table(max_position, rotary_dim, base):
    """[max_position, rotary_dim] float32: cos(p*f_j) for j < rotary_dim/2, then
    sin(p*f_j), with f_j = base**(-2j/rotary_dim), computed in float64."""
    j = np.arange(rotary_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * j / rotary_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def pair_index(rotary_dim, is_neox):
    """Indices (first, second) of the rotated pairs within a head."""
    half = rotary_dim // 2
    j = np.arange(half)
    if is_neox:
        return j, j + half
    return 2 * j, 2 * j + 1


def rotate_f32(x, cos, sin, rotary_dim, is_neox):
    """Rotate float32 rows x [..., D] by float32 cos/sin [..., rotary_dim/2]
    (broadcast over heads) with the float32 steps of the GPU."""
    x = np.asarray(x, dtype=np.float32)
    i1, i2 = pair_index(rotary_dim, is_neox)
    a = x[..., i1]
    b = x[..., i2]
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    out = np.array(x, copy=True)
    with np.errstate(over="ignore", invalid="ignore"):
        out[..., i1] = (a * c) - (b * s)
        out[..., i2] = (b * c) + (a * s)
    return out


def rotate_f64(x, cos, sin, rotary_dim, is_neox):
    """The same rotation in float64 (exact products of the float32 inputs)."""
    x = np.asarray(x, dtype=np.float64)
    i1, i2 = pair_index(rotary_dim, is_neox)
    a = x[..., i1]
    b = x[..., i2]
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    out = np.array(x, copy=True)
    out[..., i1] = a * c - b * s
    out[..., i2] = b * c + a * s
    return out


def apply_rope(bits, act_dtype, positions, table, rotary_dim, is_neox):
    """Rotate rows of activation bits [T, H, D] by their positions; rows whose
    position is outside the table are returned unchanged.  Returns bits."""
    bits = np.asarray(bits)
    out = np.array(bits, copy=True)
    half = rotary_dim // 2
    pos = np.asarray(positions, dtype=np.int64)
    ok = (pos >= 0) & (pos < table.shape[0])
    if not ok.any():
        return out
    rows = np.nonzero(ok)[0]
    x = codecs.decode(bits[rows], act_dtype).astype(np.float32)    # exact widening
    cs = table[pos[rows]]
    cos = cs[:, None, :half]
    sin = cs[:, None, half:rotary_dim]
    y = rotate_f32(x, cos, sin, rotary_dim, is_neox)
    out[rows] = codecs.f32_to_act_bits(y, act_dtype)
    return out


def rope_cache_write(query, key, value, positions, table, rotary_dim, is_neox,
                     slot_mapping, key_cache, value_cache, block_size,
                     act_dtype, cache_dtype, k_inv_scale=1.0, v_inv_scale=1.0, num_tokens=None):
    """Rotated query rows, and the caches after writing the rotated keys and the
    values of the first num_tokens rows (tokens with an out-of-table position
    write nothing).  Returns (query_bits, key_cache, value_cache)."""
    if num_tokens is None:
        num_tokens = key.shape[0]
    pos = np.asarray(positions, dtype=np.int64)[:num_tokens]
    q_rot = np.array(query, copy=True)
    q_rot[:num_tokens] = apply_rope(query[:num_tokens], act_dtype, pos, table, rotary_dim, is_neox)
    k_rot = apply_rope(key[:num_tokens], act_dtype, pos, table, rotary_dim, is_neox)
    ok = (pos >= 0) & (pos < table.shape[0])
    slots = np.where(ok, np.asarray(slot_mapping, dtype=np.int64)[:num_tokens], -1)
    kc, vc = cache.scatter(key_cache, value_cache, k_rot, value[:num_tokens], slots, block_size,
                           act_dtype, cache_dtype, k_inv_scale, v_inv_scale, num_tokens)
    return q_rot, kc, vc
