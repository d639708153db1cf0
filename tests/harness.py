"""Test-side helpers: oracle expectations for a synthetic workload.

Everything the oracle consumes here comes from the generator (the pool as
drawn, before the library writes into it) or from the oracle itself
(metadata, scatter); nothing is taken from the library's outputs.
"""

import numpy as np
import torch

from oracle import attention as OA
from oracle import cache as OC
from oracle import codecs as OD
from oracle import metadata as OM

TOL = {"f16": 5e-3, "bf16": 2e-2, "fp8": 6e-2}


def act_name(dtype):
    return {torch.float16: "f16", torch.bfloat16: "bf16"}[dtype]


def tol_of(wl):
    # int8 codes are integers of at most 8 bits, exact in both bf16 and fp16, so
    # an int8 cache adds no rounding beyond the activation dtype's
    return TOL["fp8"] if wl.cache_fp8 else TOL[act_name(wl.act_dtype)]


def oracle_cache_dtype(wl):
    return act_name(wl.act_dtype) if wl.cache_kind == "act" else wl.cache_kind


def bits16(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits8(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def cache_bits(t, one_byte):
    return bits8(t) if one_byte else bits16(t)


def oracle_metadata(wl, qsl_len=None):
    rows = [list(map(int, r)) for r in wl.block_tables]
    return OM.build_metadata(wl.num_computed.tolist(), wl.query_lens.tolist(), rows,
                             wl.block_size, max(wl.num_tokens_padded, wl.num_tokens), qsl_len)


def head_scales(tensors):
    """The K and V scales the library reads with: float32 arrays [Hkv] when the
    tensors carry per-head scales, else the tensor scales as float32."""
    def one(per_head, tensor):
        if per_head is not None:
            return per_head.cpu().numpy().astype(np.float32)
        return np.float32(tensor)
    return one(tensors.k_scales, tensors.k_scale), one(tensors.v_scales, tensors.v_scale)


class Snapshot:
    """Host copy of the generator's pool blocks that some requests reference."""

    def __init__(self, wl, tensors, requests):
        self.wl = wl
        ids = set()
        for r in requests:
            s = int(wl.seq_lens_host[r])
            nb = -(-s // wl.block_size)
            # entries outside the pool are absent blocks: nothing to copy
            ids.update(int(b) for b in wl.block_tables[r, :nb] if 0 <= b < wl.pool_blocks)
        self.ids = np.array(sorted(ids), dtype=np.int64)
        self.local = {int(b): i for i, b in enumerate(self.ids)}
        idx = torch.from_numpy(self.ids).to(tensors.key_cache.device)
        one = wl.cache_8bit
        self.kbits = cache_bits(tensors.key_cache.index_select(0, idx), one)
        self.vbits = cache_bits(tensors.value_cache.index_select(0, idx), one)


class OraclePrep:
    """The oracle's view of one step: its own metadata, its scatter of the
    step's new K/V into the generator's snapshot (taken before the library
    wrote to the pool), and the decoded queries.  Built once; rows for any set
    of requests come from ``rows``."""

    def __init__(self, wl, tensors, snapshot, qsl_len=None):
        qsl, seq_lens, positions, slots = oracle_metadata(wl, qsl_len)
        bs = wl.block_size
        act = act_name(wl.act_dtype)
        # remap the scatter to the snapshot's local block numbering
        local_slots = []
        for s in slots:
            if s < 0 or (s // bs) not in snapshot.local:
                local_slots.append(-1)
            else:
                local_slots.append(snapshot.local[s // bs] * bs + s % bs)
        T = max(wl.num_tokens_padded, wl.num_tokens)
        kb, vb = bits16(tensors.k_new[:T]), bits16(tensors.v_new[:T])
        self.cache_dt = oracle_cache_dtype(wl)
        k_sc, v_sc = head_scales(tensors)
        k_inv = np.float32(1.0) / k_sc
        v_inv = np.float32(1.0) / v_sc
        self.kc, self.vc = OC.scatter(snapshot.kbits, snapshot.vbits, kb, vb, local_slots, bs,
                                      act_dtype=act, cache_dtype=self.cache_dt, k_inv_scale=k_inv,
                                      v_inv_scale=v_inv, num_tokens=T)
        self.q = OD.decode(bits16(tensors.q), act)
        self.qsl, self.seq_lens = qsl, seq_lens
        self.wl, self.snapshot = wl, snapshot
        self.k_scale, self.v_scale = k_sc, v_sc

    def rows(self, requests, sliding_window=0, alibi_slopes=None):
        """Oracle rows {r: float64 [n_r, Hq, D]} for the given requests."""
        wl, snap, bs = self.wl, self.snapshot, self.wl.block_size
        requests = list(requests)
        wanted = set(requests)
        table = []
        for r in range(wl.num_reqs):
            nb = -(-self.seq_lens[r] // bs)
            if r in wanted:
                table.append([snap.local.get(int(b), -1) for b in wl.block_tables[r, :nb]])
            else:
                table.append([])
        return OA.paged_attention(self.q, self.kc, self.vc, table, self.qsl, self.seq_lens, bs,
                                  requests=requests, cache_dtype=self.cache_dt,
                                  k_scale=self.k_scale, v_scale=self.v_scale,
                                  sliding_window=sliding_window, alibi_slopes=alibi_slopes,
                                  num_blocks=len(snap.ids))


def oracle_outputs(wl, tensors, snapshot, requests, qsl_len=None, sliding_window=0,
                   alibi_slopes=None):
    """Oracle rows {r: float64 [n_r, Hq, D]} for the given requests.

    Metadata and the scatter of the step's new K/V are the oracle's own; the
    pool is the generator's snapshot taken before the library wrote to it.
    """
    prep = OraclePrep(wl, tensors, snapshot, qsl_len)
    return prep.rows(requests, sliding_window, alibi_slopes)


def gpu_rows(out, qsl, r):
    o = out[qsl[r]:qsl[r + 1]].float().cpu().numpy().astype(np.float64)
    return o


def compare(wl, out, expect, qsl):
    """Max-abs error over the given requests and the RMS of the expected rows."""
    worst, sq, cnt = 0.0, 0.0, 0
    for r, e in expect.items():
        g = gpu_rows(out, qsl, r)
        assert g.shape == e.shape, (g.shape, e.shape)
        assert np.all(np.isfinite(g)), f"request {r}: non-finite output"
        worst = max(worst, float(np.max(np.abs(g - e))) if e.size else 0.0)
        sq += float(np.sum(e * e))
        cnt += e.size
    rms = (sq / cnt) ** 0.5 if cnt else 0.0
    return worst, rms
