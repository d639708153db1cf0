"""Pins of the oracle's scatter and attention.

* brute force: the paged result equals dense causal attention computed by
  torch's scaled_dot_product_attention (CPU, float64) on contiguous K/V with an
  explicit bottom-right boolean mask, under random block permutations;
* closed forms: one key returns its value exactly; equal keys return the mean
  of the attended values; a two-key case written out by hand;
* invariants: GQA equals MHA with each K/V head repeated over its G consecutive
  query heads (repeat_interleave); chunked prefill over several steps equals
  one prefill; a decode of token p equals row p of a prefill;
* scatter: equals NumPy fancy-index assignment; negative slots leave the pool
  untouched.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import cache as S
from oracle import metadata as M


def _paged_setup(rng, comp, ql, hq, hkv, d, bs, pool_blocks):
    seq = [c + n for c, n in zip(comp, ql)]
    perm = rng.permutation(pool_blocks)
    rows, k = [], 0
    for s in seq:
        nb = M.blocks_for_tokens(s, bs)
        rows.append(perm[k:k + nb].tolist())
        k += nb
    kc = rng.standard_normal((pool_blocks, bs, hkv, d))
    vc = rng.standard_normal((pool_blocks, bs, hkv, d))
    T = sum(ql)
    q = rng.standard_normal((T, hq, d))
    return seq, rows, kc, vc, q


def _sdpa_reference(q, k, v, c, scale):
    # q [n, Hq, D], k/v [s, Hkv, D] contiguous; explicit bottom-right mask
    n, hq, d = q.shape
    s, hkv, _ = k.shape
    g = hq // hkv
    kk = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)
    vv = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)
    qq = torch.from_numpy(q).permute(1, 0, 2)
    mask = torch.arange(s)[None, :] <= (c + torch.arange(n))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qq, kk, vv, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2), (4, 1)])
@pytest.mark.parametrize("bs", [16, 4])
def test_paged_equals_contiguous_sdpa(hq, hkv, bs):
    rng = np.random.default_rng(hq * 10 + hkv + bs)
    comp = [0, 5, 16, 33]
    ql = [7, 1, 17, 3]
    d = 8
    seq, rows, kc, vc, q = _paged_setup(rng, comp, ql, hq, hkv, d, bs, 64)
    qsl = [0] + list(np.cumsum(ql))
    res = A.paged_attention(q, kc, vc, rows, qsl, seq, bs)
    for r in range(len(ql)):
        k, v = A.gather_request_kv(kc, vc, rows[r], seq[r], bs)
        # contiguous copy built a second way: block by block in logical order
        k2 = np.concatenate([kc[b] for b in rows[r]], axis=0)[:seq[r]]
        assert np.array_equal(k, k2)
        ref = _sdpa_reference(q[qsl[r]:qsl[r + 1]], k2,
                              np.concatenate([vc[b] for b in rows[r]], axis=0)[:seq[r]],
                              comp[r], 1.0 / math.sqrt(d))
        np.testing.assert_allclose(res[r], ref, rtol=1e-12, atol=1e-12)


def test_block_permutation_invariance():
    rng = np.random.default_rng(3)
    comp, ql = [20, 0], [1, 37]
    hq, hkv, d, bs = 4, 2, 8, 16
    seq, rows, kc, vc, q = _paged_setup(rng, comp, ql, hq, hkv, d, bs, 32)
    qsl = [0] + list(np.cumsum(ql))
    base = A.paged_attention(q, kc, vc, rows, qsl, seq, bs)
    # move every used block to a new random physical id
    perm = rng.permutation(32)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    rows2 = [[int(perm[b]) for b in row] for row in rows]
    moved = A.paged_attention(q, kc2, vc2, rows2, qsl, seq, bs)
    for r in base:
        assert np.array_equal(base[r], moved[r])


def test_single_key_returns_value():
    rng = np.random.default_rng(0)
    kc = rng.standard_normal((4, 16, 1, 8))
    vc = rng.standard_normal((4, 16, 1, 8))
    q = rng.standard_normal((1, 3, 8)) * 50
    res = A.paged_attention(q, kc, vc, [[2]], [0, 1], [1], 16)
    for h in range(3):
        assert np.array_equal(res[0][0, h], vc[2, 0, 0])


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(1)
    kc = np.tile(rng.standard_normal((1, 1, 2, 8)), (8, 16, 1, 1))
    vc = rng.standard_normal((8, 16, 2, 8))
    q = rng.standard_normal((5, 4, 8))
    rows = [[3, 6, 1]]
    res = A.paged_attention(q, kc, vc, rows, [0, 5], [40], 16)[0]
    k, v = A.gather_request_kv(kc, vc, rows[0], 40, 16)
    for i in range(5):
        keys = 35 + i + 1
        for h in range(4):
            np.testing.assert_allclose(res[i, h], v[:keys, h // 2].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_two_key_closed_form():
    # D = 1, keys k0 = 1, k1 = -2, q = 3, scale 0.5 -> scores 1.5, -3
    kc = np.zeros((2, 16, 1, 1))
    vc = np.zeros((2, 16, 1, 1))
    kc[1, 0, 0, 0], kc[1, 1, 0, 0] = 1.0, -2.0
    vc[1, 0, 0, 0], vc[1, 1, 0, 0] = 10.0, -4.0
    q = np.array([[[3.0]]])
    res = A.paged_attention(q, kc, vc, [[1]], [0, 1], [2], 16, scale=0.5)[0]
    e0, e1 = math.exp(1.5), math.exp(-3.0)
    assert res[0, 0, 0] == pytest.approx((10 * e0 - 4 * e1) / (e0 + e1), rel=1e-15)
    # with the default scale 1/sqrt(1) = 1 -> scores 3, -6
    res = A.paged_attention(q, kc, vc, [[1]], [0, 1], [2], 16)[0]
    e0, e1 = math.exp(3.0), math.exp(-6.0)
    assert res[0, 0, 0] == pytest.approx((10 * e0 - 4 * e1) / (e0 + e1), rel=1e-15)


def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(5)
    comp, ql = [9, 0], [1, 12]
    hq, hkv, d, bs = 8, 2, 8, 16
    seq, rows, kc, vc, q = _paged_setup(rng, comp, ql, hq, hkv, d, bs, 16)
    qsl = [0] + list(np.cumsum(ql))
    gqa = A.paged_attention(q, kc, vc, rows, qsl, seq, bs)
    g = hq // hkv
    kc_rep = np.repeat(kc, g, axis=2)   # head h of the MHA cache = kv head h // g
    vc_rep = np.repeat(vc, g, axis=2)
    mha = A.paged_attention(q, kc_rep, vc_rep, rows, qsl, seq, bs)
    for r in gqa:
        assert np.array_equal(gqa[r], mha[r])


def test_chunked_prefill_and_decode_invariance():
    """Prefill 298 tokens in chunks, then decode one: rows equal a single 299-token prefill."""
    rng = np.random.default_rng(11)
    hq, hkv, d, bs = 2, 1, 8, 16
    L = 299
    nb = M.blocks_for_tokens(L, bs)
    row = rng.permutation(64)[:nb].tolist()
    kc = rng.standard_normal((64, bs, hkv, d))
    vc = rng.standard_normal((64, bs, hkv, d))
    q = rng.standard_normal((L, hq, d))
    full = A.paged_attention(q, kc, vc, [row], [0, L], [L], bs)[0]
    pieces = []
    start = 0
    for n in [100, 150, 48, 1]:        # three prefill chunks then one decode
        part = A.paged_attention(q[start:start + n], kc, vc, [row], [0, n], [start + n], bs)[0]
        pieces.append(part)
        start += n
    chunked = np.concatenate(pieces, axis=0)
    np.testing.assert_allclose(chunked, full, rtol=1e-13, atol=1e-14)


def test_scatter_matches_fancy_index_and_skips_negative():
    rng = np.random.default_rng(2)
    nb, bs, hkv, d = 8, 16, 2, 4
    kc = rng.integers(0, 65536, size=(nb, bs, hkv, d)).astype(np.uint16)
    vc = rng.integers(0, 65536, size=(nb, bs, hkv, d)).astype(np.uint16)
    T = 10
    k = rng.integers(0, 65536, size=(T, hkv, d)).astype(np.uint16)
    v = rng.integers(0, 65536, size=(T, hkv, d)).astype(np.uint16)
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[3] = -1
    slots[7] = -1
    kc2, vc2 = S.scatter(kc, vc, k, v, slots, bs)
    ref_k = kc.reshape(nb * bs, hkv, d).copy()
    ref_v = vc.reshape(nb * bs, hkv, d).copy()
    keep = slots >= 0
    ref_k[slots[keep]] = k[keep]
    ref_v[slots[keep]] = v[keep]
    assert np.array_equal(kc2.reshape(nb * bs, hkv, d), ref_k)
    assert np.array_equal(vc2.reshape(nb * bs, hkv, d), ref_v)
    # padding rows skipped: the pool differs from the original in exactly the kept slots
    changed = np.any(kc2.reshape(nb * bs, -1) != kc.reshape(nb * bs, -1), axis=1)
    assert set(np.nonzero(changed)[0]) <= set(slots[keep].tolist())


def test_scatter_fp8_encodes():
    from oracle import codecs as C
    rng = np.random.default_rng(4)
    nb, bs, hkv, d = 4, 16, 1, 8
    kc = np.zeros((nb, bs, hkv, d), np.uint8)
    vc = np.zeros((nb, bs, hkv, d), np.uint8)
    kx = rng.standard_normal((3, hkv, d)).astype(np.float32)
    bits = torch.from_numpy(kx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    slots = np.array([5, -1, 40])
    inv = np.float32(1.0) / np.float32(0.02)
    kc2, vc2 = S.scatter(kc, vc, bits, bits, slots, bs, act_dtype="bf16", cache_dtype="fp8_e4m3",
                         k_inv_scale=inv, v_inv_scale=inv)
    want = C.e4m3fn_encode(C.bf16_bits_to_f64(bits).astype(np.float32), inv)
    assert np.array_equal(kc2[0, 5], want[0])
    assert np.array_equal(kc2[2, 8], want[2])
    assert np.count_nonzero(kc2) == np.count_nonzero(want[0]) + np.count_nonzero(want[2])


def test_scatter_int8_encodes():
    # expected codes from torch's per-tensor quantization (independent of the
    # oracle's encoder), clipped to the symmetric range
    rng = np.random.default_rng(5)
    nb, bs, hkv, d = 4, 16, 1, 8
    kc = np.zeros((nb, bs, hkv, d), np.uint8)
    vc = np.full((nb, bs, hkv, d), 7, np.uint8)
    kx = (rng.standard_normal((3, hkv, d)) * 3).astype(np.float32)
    bits = torch.from_numpy(kx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    slots = np.array([5, -1, 40])
    scale = np.float32(0.02)
    inv = np.float32(1.0) / scale
    kc2, vc2 = S.scatter(kc, vc, bits, bits, slots, bs, act_dtype="bf16", cache_dtype="int8",
                         k_inv_scale=inv, v_inv_scale=inv)
    xb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    want = np.maximum(torch.quantize_per_tensor(xb, float(scale), 0, torch.qint8).int_repr().numpy(), -127)
    assert np.array_equal(kc2[0, 5].view(np.int8), want[0])
    assert np.array_equal(kc2[2, 8].view(np.int8), want[2])
    assert np.array_equal(vc2[2, 8].view(np.int8), want[2])
    # untouched slots keep their bytes (the padding token wrote nothing)
    assert np.count_nonzero(kc2) == np.count_nonzero(want[0]) + np.count_nonzero(want[2])
    assert np.sum(vc2 != 7) == np.sum(want[0] != 7) + np.sum(want[2] != 7)


def test_int8_cache_attention_equals_sdpa_on_dequantized():
    # an int8 cache with per-tensor scales attends like a float cache holding
    # code * scale: checked against torch SDPA on the dequantized contiguous K/V
    rng = np.random.default_rng(6)
    hq, hkv, d, bs, pool = 4, 2, 16, 4, 32
    comp, ql = [5, 0, 9], [1, 6, 3]
    seq, rows, _, _, q = _paged_setup(rng, comp, ql, hq, hkv, d, bs, pool)
    kcode = rng.integers(-127, 128, size=(pool, bs, hkv, d)).astype(np.int8)
    vcode = rng.integers(-127, 128, size=(pool, bs, hkv, d)).astype(np.int8)
    ks, vs = 0.013, 0.021
    qsl = [0] + list(np.cumsum(ql))
    scale = 1.0 / math.sqrt(d)
    got = A.paged_attention(q, kcode.view(np.uint8), vcode.view(np.uint8), rows, qsl, seq, bs,
                            cache_dtype="int8", k_scale=ks, v_scale=vs)
    for r in range(len(seq)):
        ids = rows[r]
        k = kcode[ids].reshape(-1, hkv, d)[:seq[r]].astype(np.float64) * ks
        v = vcode[ids].reshape(-1, hkv, d)[:seq[r]].astype(np.float64) * vs
        ref = _sdpa_reference(q[qsl[r]:qsl[r + 1]], k, v, comp[r], scale)
        assert np.allclose(got[r], ref, rtol=0, atol=1e-12), r


def test_absent_blocks_equal_sdpa_without_their_keys():
    """Table entries outside the pool hold no keys: the oracle equals SDPA over
    the dense K/V with those keys masked out (their cache contents, even NaN,
    never matter), and a row with no visible key is exactly zero."""
    rng = np.random.default_rng(91)
    hq, hkv, d, bs, nb_pool = 8, 2, 8, 4, 40
    comp = [9, 0, 3, 11]
    ql = [1, 6, 5, 1]
    seq, rows, kc, vc, q = _paged_setup(rng, comp, ql, hq, hkv, d, bs, nb_pool)
    rows = [list(r) for r in rows]
    rows[0][1] = -1               # decode: a middle block absent
    rows[1][0] = nb_pool + 3      # prefill: the first block outside the pool
    rows[2][1] = -7               # prefill with a cached prefix: the block of its last keys
    rows[3] = [-1] * len(rows[3])  # decode with every block absent
    # what sits in block 0 (read in place of absent ones) never matters: make
    # it NaN, after moving any present use of block 0 to an unused block
    used = {b for row in rows for b in row}
    spare = min(set(range(1, nb_pool)) - used)
    rows = [[spare if b == 0 else b for b in row] for row in rows]
    kc[spare], vc[spare] = kc[0], vc[0]
    kc[0] = np.nan
    vc[0] = np.nan
    qsl = [0] + list(np.cumsum(ql))
    res = A.paged_attention(q, kc, vc, rows, qsl, seq, bs, num_blocks=nb_pool)
    for r in range(len(ql)):
        s, c, n = seq[r], seq[r] - ql[r], ql[r]
        present = np.array([0 <= rows[r][j // bs] < nb_pool for j in range(s)])
        k = np.zeros((s, hkv, d))
        v = np.zeros((s, hkv, d))
        for j in range(s):
            if present[j]:
                k[j] = kc[rows[r][j // bs], j % bs]
                v[j] = vc[rows[r][j // bs], j % bs]
        g = hq // hkv
        kk = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)
        vv = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)
        qq = torch.from_numpy(q[qsl[r]:qsl[r + 1]]).permute(1, 0, 2)
        mask = (torch.arange(s)[None, :] <= (c + torch.arange(n))[:, None]) & \
            torch.from_numpy(present)[None, :]
        visible = mask.any(dim=1).numpy()
        got = res[r]
        assert np.all(np.isfinite(got))
        assert np.array_equal(got[~visible], np.zeros_like(got[~visible]))
        if visible.any():
            ref = torch.nn.functional.scaled_dot_product_attention(
                qq, kk, vv, attn_mask=mask, scale=1.0 / math.sqrt(d)).permute(1, 0, 2).numpy()
            np.testing.assert_allclose(got[visible], ref[visible], rtol=1e-12, atol=1e-12)
    assert not np.any(res[3])     # every block absent: zero output
    # a table of pool ids only: num_blocks changes nothing
    pool_rows = [list(range(1, 1 + len(r))) for r in rows]
    full = A.paged_attention(q, kc, vc, pool_rows, qsl, seq, bs, num_blocks=nb_pool)
    ref_full = A.paged_attention(q, kc, vc, pool_rows, qsl, seq, bs)
    for r in full:
        assert np.array_equal(full[r], ref_full[r])
