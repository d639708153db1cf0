"""Reference oracle for paged KV-cache attention (test infrastructure only).

This package is a plain, slow, CPU implementation of what the paged-attention
hot path computes.  It exists to check the HIP kernels and nothing else: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product path (the C-ABI library and its Python
binding) never imports, links or calls anything in here, and this package never
imports the product path.

Sources (web pages; every function cites the part it follows):

* "Tour: One forward pass" (explainvllm), stops 1-5 (request rows, batch order,
  ``query_start_loc``, positions, ``seq_lens``, block tables, slot mappings,
  ``PAD_SLOT_ID``) and stop 10 (cache write, then varlen causal attention that
  reads keys through the block table).
* "vLLM MHA Code Path: From QKV to Paged KV Cache", sections "One Path Covers
  MHA, GQA, and MQA", "Worked Trace: One Decode Token", "Cache write and cache
  read use different maps".
* "vLLM 推理全流程深度解析" (vLLM inference deep dive): the BlockManager block
  allocation example, the ``prepare_input_tensors`` slot-mapping example, the
  ``reshape_and_cache`` kernel description, the PagedAttention decode kernel
  signature, the KV-cache quantization remark and the ``LlamaAttention``
  listing (RoPE on Q and K before the cache write).
* "Tour: One forward pass", stop 9 (RoPE on q and k: per-position cosines
  and sines from ``cos_sin_cache`` turn every head's pairs).
* "vLLM 推理全流程深度解析": the scheduler output's ``blocks_to_swap_in``,
  ``blocks_to_swap_out`` and ``blocks_to_copy`` lists, swapping to host memory
  and block sharing between sequences.

Arithmetic is float64 unless the format itself fixes the precision (the fp8
and int8 encoders' single float32 multiply) or the reading of the pages fixes it (the
rotary embedding's float32 steps, pinned to the float64 rotation).  Modules:

* ``codecs``     fp16 / bf16 / OCP e4m3fn / int8 bit decoders, the e4m3fn and int8 encoders.
* ``metadata``   query_start_loc, seq_lens, positions, slot_mapping.
* ``cache``      the slot_mapping scatter into ``[num_blocks, block_size, Hkv, D]``.
* ``attention``  gather through the block table + dense causal softmax(QK^T*scale)V.
* ``rope``       rotary position embedding of Q and K fused with the cache write.
* ``blocks``     block copy and swap between block pools.

Every function here is pinned by ``tests/test_oracle_*.py`` against values the
pages print, closed forms, library routines or brute force; none is
"parity unpinned".
"""

from . import codecs, metadata, cache, attention, rope, blocks  # noqa: F401
