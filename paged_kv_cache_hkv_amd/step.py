"""One step of the paged-attention path on one attention layer.

The order of calls is the one "Tour: One forward pass" walks through: the
batch metadata once per step (stops 3-4), then per layer the cache write
followed by attention that reads the cache (stop 10).  Decode requests come
first in the batch (stop 2's batch order), so attention is one ``pa_decode``
over requests [0, num_decodes) and one ``pa_prefill_varlen`` over the rest;
the two write disjoint output rows.

Every buffer is allocated once here (fixed addresses, so the sequence can be
replayed); ``run()`` only enqueues library calls on the current stream.
"""

import torch

from . import binding as B

_ACT = {torch.float16: B.PA_F16, torch.bfloat16: B.PA_BF16}


class PagedAttentionStep:
    def __init__(self, wl, tensors, decode_workers=0, qsl_len=None, sliding_window=0,
                 alibi_slopes=None):
        self.wl = wl
        self.t = tensors
        dev = tensors.q.device
        act = _ACT[wl.act_dtype]
        cache = {"act": act, "fp8_e4m3": B.PA_FP8_E4M3, "int8": B.PA_INT8}[wl.cache_kind]
        self.desc = B.make_desc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size,
                                act, cache, k_scale=tensors.k_scale, v_scale=tensors.v_scale,
                                decode_workers=decode_workers, sliding_window=sliding_window,
                                alibi_slopes=alibi_slopes, k_scales=tensors.k_scales,
                                v_scales=tensors.v_scales)
        R = wl.num_reqs
        self.T_pad = tensors.q.shape[0]
        self.qsl = torch.empty(qsl_len or (R + 1), dtype=torch.int32, device=dev)
        self.seq_lens = torch.empty(R, dtype=torch.int32, device=dev)
        self.positions = torch.zeros(self.T_pad, dtype=torch.int64, device=dev)
        self.slot_mapping = torch.empty(self.T_pad, dtype=torch.int64, device=dev)
        self.out = torch.zeros((self.T_pad, wl.num_q_heads, wl.head_dim), dtype=wl.act_dtype,
                               device=dev)
        self.max_seq_len = wl.max_seq_len
        self.num_decodes = wl.num_decodes
        self.max_prefill_len = int(wl.query_lens[wl.num_decodes:].max()) if R > wl.num_decodes else 0
        ws = B.pa_decode_workspace_size(self.desc, self.num_decodes, self.max_seq_len,
                                        wl.block_tables.shape[1])
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=dev) if ws else None

    def metadata(self, stream=None):
        t = self.t
        B.pa_metadata_build(t.num_computed, t.query_lens, t.block_tables, self.qsl, self.seq_lens,
                            self.positions, self.slot_mapping, self.wl.block_size, stream)

    def cache_write(self, stream=None):
        t = self.t
        B.pa_cache_write(self.desc, t.k_new, t.v_new, self.slot_mapping, t.key_cache,
                         t.value_cache, num_tokens=self.T_pad, stream=stream)

    def rope_cache_write(self, cos_sin, rotary_dim, is_neox=True, stream=None):
        """The fused alternative to ``cache_write``: rotate q (in place) and k by
        position, then write the rotated k and v to the cache."""
        t = self.t
        B.pa_rope_cache_write(self.desc, self.positions, cos_sin, rotary_dim, is_neox, t.q,
                              t.k_new, t.v_new, self.slot_mapping, t.key_cache, t.value_cache,
                              num_tokens=self.T_pad, stream=stream)

    def decode(self, stream=None):
        if self.num_decodes == 0:
            return
        t = self.t
        B.pa_decode(self.desc, 0, self.num_decodes, t.q, self.qsl, self.seq_lens, t.block_tables,
                    t.key_cache, t.value_cache, self.max_seq_len, self.workspace, self.out, stream)

    def prefill(self, stream=None):
        R = self.wl.num_reqs
        if R == self.num_decodes:
            return
        t = self.t
        B.pa_prefill_varlen(self.desc, self.num_decodes, R, t.q, self.qsl, self.seq_lens,
                            t.block_tables, t.key_cache, t.value_cache, self.max_prefill_len,
                            self.max_seq_len, self.out, stream)

    def attention(self, stream=None):
        self.decode(stream)
        self.prefill(stream)

    def run(self, stream=None):
        """Metadata, cache write, decode, prefill -- the whole hot path once."""
        self.metadata(stream)
        self.cache_write(stream)
        self.attention(stream)
