"""The slot_mapping scatter of the oracle (test infrastructure only).

Follows the ``reshape_and_cache`` description in "vLLM 推理全流程深度解析": for
each new token ``t`` with ``slot_mapping[t] >= 0`` (negative slots are skipped),
``block = slot // block_size``, ``offset = slot % block_size``, and the token's
``[num_kv_heads, head_size]`` key and value rows go to
``key_cache[block, offset]`` / ``value_cache[block, offset]`` of the global pool
``[num_blocks, block_size, num_kv_heads, head_size]``.  "Tour: One forward
pass", stop 10, and the worked decode trace of "vLLM MHA Code Path" (step 8)
place this write before the attention read of the same layer.

Caches are handled as raw bit patterns (uint16 for fp16/bf16, uint8 for fp8
and int8), so a write is a byte copy and can be compared bit for bit.  The fp8
and int8 paths encode with ``codecs.e4m3fn_encode`` / ``codecs.int8_encode``
from the float32 value of the input.
"""

import numpy as np

from . import codecs


def _to_f32(bits, act_dtype):
    return codecs.decode(bits, act_dtype).astype(np.float32)


def _per_head(inv):
    """A tensor's inverse scale as is; one per head as [Hkv, 1] (broadcasts over [T, Hkv, D])."""
    a = np.asarray(inv, dtype=np.float32)
    return a[:, None] if a.ndim == 1 else a


def scatter(key_cache, value_cache, key, value, slot_mapping, block_size,
            act_dtype="f16", cache_dtype="f16", k_inv_scale=1.0, v_inv_scale=1.0,
            num_tokens=None):
    """Write new K/V rows into copies of the caches; return the new caches.

    key_cache/value_cache: uint arrays [num_blocks, block_size, Hkv, D] (bits).
    key/value: uint16 arrays [T, Hkv, D] of the activation dtype (bits).
    slot_mapping: int sequence of length >= num_tokens.
    k_inv_scale/v_inv_scale: the float32 inverse scale of the tensor, or one
    per K/V head (a float32 array [Hkv]: head h is encoded with its own).
    A slot that is negative, or past the pool, is skipped.
    """
    k_inv = _per_head(k_inv_scale)
    v_inv = _per_head(v_inv_scale)
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    num_blocks = kc.shape[0]
    if num_tokens is None:
        num_tokens = key.shape[0]
    if cache_dtype == act_dtype:
        new_k, new_v = key, value
    elif cache_dtype == "fp8_e4m3":
        new_k = codecs.e4m3fn_encode(_to_f32(key[:num_tokens], act_dtype), k_inv)
        new_v = codecs.e4m3fn_encode(_to_f32(value[:num_tokens], act_dtype), v_inv)
    elif cache_dtype == "int8":
        new_k = codecs.int8_encode(_to_f32(key[:num_tokens], act_dtype), k_inv).view(np.uint8)
        new_v = codecs.int8_encode(_to_f32(value[:num_tokens], act_dtype), v_inv).view(np.uint8)
    else:
        raise ValueError((act_dtype, cache_dtype))
    for t in range(num_tokens):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        block = slot // block_size
        offset = slot % block_size
        if block >= num_blocks:
            continue
        kc[block, offset] = new_k[t]
        vc[block, offset] = new_v[t]
    return kc, vc
