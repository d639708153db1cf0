"""GPU parity of the per-K/V-head scales of quantized (fp8, int8) caches.

The same tensors as the per-tensor tests, read and written with one scale per
K/V head (``synth.with_head_scales``: each head's scale is the tensor scale
times its own factor, so the pool's codes stand for other values and new rows
are encoded with other inverse scales).  Cache writes (plain and fused with
RoPE) must match the oracle's per-head encoding bit for bit; attention (decode
and prefill, every head layout, the mask variants and forced decode splits,
which exercise the workgroup merge and the reduce) must match the oracle's
per-head dequantisation within the per-tensor bars.
"""

import numpy as np
import pytest
import torch

from oracle import cache as OC
from oracle import rope as OR
from paged_kv_cache_hkv_amd import binding as B
from paged_kv_cache_hkv_amd import synth as S
from paged_kv_cache_hkv_amd.step import PagedAttentionStep

from harness import (Snapshot, act_name, bits16, cache_bits, compare, head_scales,
                     oracle_cache_dtype, oracle_metadata, oracle_outputs, tol_of)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


@pytest.mark.parametrize("act", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("kind", ["fp8", "int8"])
@pytest.mark.parametrize("d", [64, 128])
def test_cache_write_head_scales_bit_exact(act, kind, d):
    _need_gpu()
    wl = S.random_batch(61 + d, [3, 16, 200], [(0, 37), (16, 16)], hq=8, hkv=4, d=d, act=act,
                        fp8=kind == "fp8", int8=kind == "int8", pad=5)
    t = S.with_head_scales(S.make_tensors(wl, DEV, poison=True), seed=d + 7)
    before_k, before_v = cache_bits(t.key_cache, True), cache_bits(t.value_cache, True)
    print(f"[head-scales write] {kind} {act_name(act)} d={d}", flush=True)
    step = PagedAttentionStep(wl, t)
    step.metadata()
    step.cache_write()
    torch.cuda.synchronize()
    _, _, _, slots = oracle_metadata(wl)
    T = step.T_pad
    ks, vs = head_scales(t)
    want_k, want_v = OC.scatter(before_k, before_v, bits16(t.k_new[:T]), bits16(t.v_new[:T]),
                                slots, wl.block_size, act_dtype=act_name(act),
                                cache_dtype=oracle_cache_dtype(wl),
                                k_inv_scale=np.float32(1) / ks, v_inv_scale=np.float32(1) / vs,
                                num_tokens=T)
    assert np.array_equal(cache_bits(t.key_cache, True), want_k)
    assert np.array_equal(cache_bits(t.value_cache, True), want_v)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
@pytest.mark.parametrize("rotary_dim,neox", [(128, True), (64, False)])
def test_rope_cache_write_head_scales_bit_exact(kind, rotary_dim, neox):
    _need_gpu()
    wl = S.random_batch(71, [5, 40], [(0, 33), (20, 17)], hq=16, hkv=4, d=128,
                        act=torch.bfloat16, fp8=kind == "fp8", int8=kind == "int8", pad=3)
    t = S.with_head_scales(S.make_tensors(wl, DEV, poison=True), seed=rotary_dim)
    _, _, positions, slots = oracle_metadata(wl)
    Tp = t.q.shape[0]
    pos = np.array([0 if p is None else p for p in positions[:Tp]], np.int64)
    slots = np.array(slots[:Tp], np.int64)
    table = OR.cos_sin_table(int(pos.max()) + 1, rotary_dim, 10000.0)
    q0, k0, v0 = bits16(t.q), bits16(t.k_new), bits16(t.v_new)
    kc0, vc0 = cache_bits(t.key_cache, True), cache_bits(t.value_cache, True)
    cache_code = B.PA_FP8_E4M3 if kind == "fp8" else B.PA_INT8
    desc = B.make_desc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, B.PA_BF16,
                       cache_code, k_scale=t.k_scale, v_scale=t.v_scale, k_scales=t.k_scales,
                       v_scales=t.v_scales)
    print(f"[head-scales rope] {kind} rotary_dim={rotary_dim} neox={neox}", flush=True)
    B.pa_rope_cache_write(desc, torch.from_numpy(pos).to(DEV), torch.from_numpy(table).to(DEV),
                          rotary_dim, neox, t.q, t.k_new, t.v_new, torch.from_numpy(slots).to(DEV),
                          t.key_cache, t.value_cache, num_tokens=Tp)
    torch.cuda.synchronize()
    ks, vs = head_scales(t)
    _, want_k, want_v = OR.rope_cache_write(q0, k0, v0, pos, table, rotary_dim, neox, slots, kc0, vc0,
                                            wl.block_size, "bf16", oracle_cache_dtype(wl),
                                            np.float32(1) / ks, np.float32(1) / vs, Tp)
    assert np.array_equal(bits16(t.q), OR.apply_rope(q0, "bf16", pos, table, rotary_dim, neox))
    assert np.array_equal(cache_bits(t.key_cache, True), want_k)
    assert np.array_equal(cache_bits(t.value_cache, True), want_v)


def _attention(wl, t, workers=0, sliding_window=0, alibi=None):
    requests = list(range(wl.num_reqs))
    snap = Snapshot(wl, t, requests)
    a32 = None if alibi is None else np.asarray(alibi, dtype=np.float32)
    slopes = None if alibi is None else torch.from_numpy(a32).to(DEV)
    step = PagedAttentionStep(wl, t, decode_workers=workers, sliding_window=sliding_window,
                              alibi_slopes=slopes)
    step.run()
    torch.cuda.synchronize()
    qsl, _, _, _ = oracle_metadata(wl)
    expect = oracle_outputs(wl, t, snap, requests, sliding_window=sliding_window,
                            alibi_slopes=None if alibi is None else a32.astype(np.float64))
    err, rms = compare(wl, step.out, expect, qsl)
    tol = tol_of(wl)
    print(f"[head-scales {wl.name}] workers={workers} window={sliding_window} "
          f"alibi={alibi is not None} max_abs={err:.3e} rms={rms:.3e} tol={tol}", flush=True)
    assert err <= tol, (err, tol)


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (32, 1, 128), (8, 8, 64), (12, 4, 128),
                                      (32, 1, 64)])
@pytest.mark.parametrize("act,kind", [(torch.bfloat16, "fp8"), (torch.bfloat16, "int8"),
                                      (torch.float16, "int8")])
def test_attention_head_scales_parity(hq, hkv, d, act, kind):
    _need_gpu()
    seed = 300 + hq + hkv * 3 + d + (5 if kind == "int8" else 0) + (1 if act == torch.float16 else 0)
    decodes = [0, 15, 16, 33, 298, 1000]
    prefills = [(0, 1), (0, 17), (7, 40), (100, 129), (0, 298)]
    wl = S.random_batch(seed, decodes, prefills, hq=hq, hkv=hkv, d=d, act=act,
                        fp8=kind == "fp8", int8=kind == "int8", pad=3)
    t = S.with_head_scales(S.make_tensors(wl, DEV, poison=True), seed=seed)
    _attention(wl, t)


@pytest.mark.parametrize("k,v", [(True, False), (False, True)])
def test_attention_one_side_head_scales(k, v):
    _need_gpu()
    wl = S.random_batch(351, [20, 500], [(0, 70), (64, 64)], hq=16, hkv=4, d=128,
                        act=torch.bfloat16, int8=True)
    t = S.with_head_scales(S.make_tensors(wl, DEV, poison=True), seed=9, k=k, v=v)
    _attention(wl, t)


@pytest.mark.parametrize("workers", [1, 7, 64, 1000])
def test_decode_split_head_scales(workers):
    """Forced splits: heads cut between workers and workgroups are merged in
    the workgroup and by the reduce, each with its head's V scale."""
    _need_gpu()
    wl = S.random_batch(361, [700, 1500, 64, 3000], [], hq=32, hkv=8, d=128, act=torch.bfloat16,
                        fp8=True)
    t = S.with_head_scales(S.make_tensors(wl, DEV, poison=True), seed=workers)
    _attention(wl, t, workers=workers)


@pytest.mark.parametrize("kind", ["fp8", "int8"])
def test_masked_head_scales(kind):
    _need_gpu()
    wl = S.random_batch(371, [40, 900], [(0, 200), (300, 90)], hq=16, hkv=4, d=128,
                        act=torch.bfloat16, fp8=kind == "fp8", int8=kind == "int8")
    t = S.with_head_scales(S.make_tensors(wl, DEV, poison=True), seed=11)
    slopes = [2.0 ** (-8.0 * (h + 1) / 16) for h in range(16)]
    _attention(wl, t, sliding_window=100, alibi=slopes)
