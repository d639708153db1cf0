"""GPU parity of pa_copy_blocks against the oracle (oracle/blocks.py).

Byte-exact: every destination pool after the call must equal the oracle's
copy of the pools as drawn (taken to the host before the call).  Covers the
scheduler's three pair lists: a copy inside one device pool, a swap out to a
pinned host pool and a swap in from one, with the pair list on the device or
in pinned host memory; out-of-pool pairs; pageable memory rejected before
launch; and the large GQA pool with its touched blocks checked.
"""

import numpy as np
import pytest
import torch

from oracle import blocks as OB
from paged_kv_cache_hkv_amd import binding as B
from paged_kv_cache_hkv_amd import synth as S

from harness import cache_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _desc(wl, t):
    act = B.PA_F16 if wl.act_dtype == torch.float16 else B.PA_BF16
    cache = {"act": act, "fp8_e4m3": B.PA_FP8_E4M3, "int8": B.PA_INT8}[wl.cache_kind]
    return B.make_desc(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size, act,
                       cache, k_scale=t.k_scale, v_scale=t.v_scale)


def _pairs(rng, n_src, n_dst, n, same_pool=False):
    """n pairs with distinct destinations; inside one pool the destinations are
    not sources (the precondition of the copy)."""
    dst = rng.permutation(n_dst)[:n]
    if same_pool:
        src = rng.choice(np.setdiff1d(np.arange(n_src), dst), n)
    else:
        src = rng.integers(0, n_src, n)
    return np.stack([src, dst], 1).astype(np.int64)


def _host_pool(n, like, fill_seed):
    g = torch.Generator().manual_seed(fill_seed)
    shape = (n,) + tuple(like.shape[1:])
    bits = torch.randint(0, 256, shape + (like.element_size(),), generator=g, dtype=torch.uint8)
    p = torch.empty(shape, dtype=like.dtype, pin_memory=True)
    p.view(torch.uint8).view(shape + (like.element_size(),)).copy_(bits)
    return p


WORKLOADS = {
    "walkthrough_f16": lambda: S.CONFIGS["walkthrough"](),
    "gqa_bf16_fp8": lambda: S.random_batch(41, [2, 3], [(5, 300), (0, 70)], hq=8, hkv=2, d=128,
                                           act=torch.bfloat16, fp8=True),
    "mqa_f16_int8": lambda: S.random_batch(42, [2, 40], [(5, 300)], hq=8, hkv=1, d=64,
                                           act=torch.float16, int8=True),
}


@pytest.mark.parametrize("name", list(WORKLOADS))
@pytest.mark.parametrize("pairs_on_host", [False, True])
def test_copy_inside_one_pool(name, pairs_on_host):
    _need_gpu()
    wl = WORKLOADS[name]()
    t = S.make_tensors(wl, DEV, poison=False)
    fp8 = wl.cache_8bit
    k0, v0 = cache_bits(t.key_cache, fp8), cache_bits(t.value_cache, fp8)
    nb = k0.shape[0]
    rng = np.random.default_rng(7)
    pairs = _pairs(rng, nb, nb, min(300, nb // 4), same_pool=True)
    pt = torch.from_numpy(pairs)
    pt = pt.pin_memory() if pairs_on_host else pt.to(DEV)
    print(f"[blocks] copy {name} pairs={len(pairs)} host_pairs={pairs_on_host}", flush=True)
    B.pa_copy_blocks(_desc(wl, t), t.key_cache, t.value_cache, t.key_cache, t.value_cache, pt)
    torch.cuda.synchronize()
    wk, wv = OB.copy_blocks(k0, v0, k0, v0, pairs)
    assert np.array_equal(cache_bits(t.key_cache, fp8), wk)
    assert np.array_equal(cache_bits(t.value_cache, fp8), wv)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_swap_out_then_in(name):
    _need_gpu()
    wl = WORKLOADS[name]()
    t = S.make_tensors(wl, DEV, poison=False)
    fp8 = wl.cache_8bit
    desc = _desc(wl, t)
    k0, v0 = cache_bits(t.key_cache, fp8), cache_bits(t.value_cache, fp8)
    nb = k0.shape[0]
    rng = np.random.default_rng(8)
    host_k, host_v = _host_pool(96, t.key_cache, 1), _host_pool(96, t.value_cache, 2)
    hk0, hv0 = cache_bits(host_k, fp8), cache_bits(host_v, fp8)
    out_pairs = _pairs(rng, nb, 96, 64)
    print(f"[blocks] swap out {name} pairs={len(out_pairs)}", flush=True)
    B.pa_copy_blocks(desc, t.key_cache, t.value_cache, host_k, host_v,
                     torch.from_numpy(out_pairs).to(DEV))
    torch.cuda.synchronize()
    wk, wv = OB.copy_blocks(k0, v0, hk0, hv0, out_pairs)
    assert np.array_equal(cache_bits(host_k, fp8), wk)
    assert np.array_equal(cache_bits(host_v, fp8), wv)
    # swap back in, pair list in pinned host memory, onto other device blocks
    in_pairs = np.stack([out_pairs[:, 1], rng.permutation(nb)[:64]], 1).astype(np.int64)
    print(f"[blocks] swap in {name} pairs={len(in_pairs)}", flush=True)
    B.pa_copy_blocks(desc, host_k, host_v, t.key_cache, t.value_cache,
                     torch.from_numpy(in_pairs).pin_memory())
    torch.cuda.synchronize()
    gk, gv = OB.copy_blocks(wk, wv, k0, v0, in_pairs)
    assert np.array_equal(cache_bits(t.key_cache, fp8), gk)
    assert np.array_equal(cache_bits(t.value_cache, fp8), gv)
    # the blocks that went out and came back are the original ones
    got_k = cache_bits(t.key_cache, fp8)
    assert np.array_equal(got_k[in_pairs[:, 1]], k0[out_pairs[:, 0]])


def test_out_of_pool_pairs_are_skipped():
    _need_gpu()
    wl = WORKLOADS["walkthrough_f16"]()
    t = S.make_tensors(wl, DEV, poison=False)
    k0, v0 = cache_bits(t.key_cache, False), cache_bits(t.value_cache, False)
    nb = k0.shape[0]
    pairs = np.array([[-1, 3], [3, -1], [nb, 4], [5, nb], [1 << 40, 6], [10, 11]], np.int64)
    B.pa_copy_blocks(_desc(wl, t), t.key_cache, t.value_cache, t.key_cache, t.value_cache,
                     torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    wk, wv = OB.copy_blocks(k0, v0, k0, v0, pairs)
    assert np.array_equal(cache_bits(t.key_cache, False), wk)
    assert np.array_equal(cache_bits(t.value_cache, False), wv)


def test_pageable_memory_is_rejected():
    _need_gpu()
    wl = WORKLOADS["walkthrough_f16"]()
    t = S.make_tensors(wl, DEV, poison=False)
    pageable = torch.zeros((8,) + tuple(t.key_cache.shape[1:]), dtype=t.key_cache.dtype)
    assert not pageable.is_pinned()
    pairs = torch.tensor([[0, 1]], dtype=torch.int64, device=DEV)
    with pytest.raises(B.PaError) as e:
        B.pa_copy_blocks(_desc(wl, t), t.key_cache, t.value_cache, pageable, pageable, pairs)
    assert e.value.status == B.PA_ERR_INVALID_ARG
    with pytest.raises(B.PaError):
        B.pa_copy_blocks(_desc(wl, t), t.key_cache, t.value_cache, t.key_cache, t.value_cache,
                         pairs.cpu())                          # pageable pair list
    torch.cuda.synchronize()
    assert not pageable.any()


def test_large_gqa_pool_touched_blocks():
    """The GQA decode pool (bf16, 8 K/V heads, D 128: 32 KiB blocks): 4096 copies
    inside the pool; destinations hold the sources' pre-call bytes, a sample of
    other blocks is unchanged."""
    _need_gpu()
    wl = S.CONFIGS["decode_gqa"]()
    t = S.make_tensors(wl, DEV, poison=False)
    nb = t.key_cache.shape[0]
    rng = np.random.default_rng(9)
    used = np.unique(wl.block_tables[wl.block_tables >= 0])   # blocks holding drawn values
    src = rng.choice(used, 4096, replace=False)
    rest = rng.permutation(np.setdiff1d(np.arange(nb), src))
    dst, other = rest[:4096], rest[4096:4096 + 512]
    pairs = np.stack([src, dst], 1).astype(np.int64)
    idx = lambda a: torch.from_numpy(a).to(DEV)
    before_src_k = cache_bits(t.key_cache.index_select(0, idx(src)), False)
    before_src_v = cache_bits(t.value_cache.index_select(0, idx(src)), False)
    before_other = cache_bits(t.key_cache.index_select(0, idx(other)), False)
    print(f"[blocks] large gqa pool={nb} pairs=4096", flush=True)
    B.pa_copy_blocks(_desc(wl, t), t.key_cache, t.value_cache, t.key_cache, t.value_cache,
                     idx(pairs))
    torch.cuda.synchronize()
    assert np.array_equal(cache_bits(t.key_cache.index_select(0, idx(dst)), False), before_src_k)
    assert np.array_equal(cache_bits(t.value_cache.index_select(0, idx(dst)), False), before_src_v)
    assert np.array_equal(cache_bits(t.key_cache.index_select(0, idx(other)), False), before_other)
