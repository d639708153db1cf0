"""Block copy and swap of the paged cache, in the oracle (test infrastructure only).

"vLLM 推理全流程深度解析": the scheduler's output carries three lists of block
pairs -- ``blocks_to_swap_in`` (CPU to GPU), ``blocks_to_swap_out`` (GPU to
CPU) and ``blocks_to_copy`` (sharing for parallel sampling and beam search).
The same page explains why the lists exist: when GPU memory runs short the
scheduler evicts some sequences' KV blocks to host memory (swapping), and
because the cache is one global ``[num_blocks, block_size, Hkv, D]`` pool and
not a per-sequence buffer, several sequences may point at one block (beam
candidates share the prompt's blocks), so a shared block that one of them is
about to extend is first copied to a block of its own.

All three lists are the same operation between a source pool and a
destination pool (the same pool for ``blocks_to_copy``): for each pair
``(src, dst)``, block ``dst`` of the destination K and V caches receives the
bytes of block ``src`` of the source caches.

Readings taken where the pages are silent:
* every read sees the source pool as it was before the call (for a copy
  inside one pool the caller gives destinations that are distinct and are not
  sources; then the order of the pairs does not matter);
* a pair whose source or destination is outside its pool is skipped;
* a block moves as raw bytes whatever the cache dtype, K and V alike.
"""

import numpy as np


def copy_blocks(src_key, src_value, dst_key, dst_value, pairs):
    """Return new (dst_key, dst_value) after copying block ``s`` of the source
    caches to block ``d`` of the destination caches for each pair (s, d).

    Pools are arrays [num_blocks, ...] of any element type (bits); the source
    is read as it was before the call, even when it is the destination.
    """
    sk = np.array(src_key, copy=True)
    sv = np.array(src_value, copy=True)
    dk = np.array(dst_key, copy=True)
    dv = np.array(dst_value, copy=True)
    for s, d in pairs:
        s, d = int(s), int(d)
        if 0 <= s < sk.shape[0] and 0 <= d < dk.shape[0]:
            dk[d] = sk[s]
            dv[d] = sv[s]
    return dk, dv
