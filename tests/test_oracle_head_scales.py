"""Pins of the oracle's per-K/V-head scales of the quantized (fp8, int8) caches.

The per-head option applies the per-tensor reading head by head: a code of
K/V head h means ``code * scale[h]`` and is written with ``float32(1/scale[h])``.
The pins fix the head axis against things the per-tensor path already
satisfies: equal per-head scales are the per-tensor scale; each head's slice of
a per-head write or read equals a per-tensor write or read of that slice with
that head's scale; and in attention a V scale multiplies the output of the
query heads of its K/V head, while a K scale acts as that group's softmax scale
(both exact identities of the softmax).
"""

import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import cache as S
from oracle import codecs as C

FMT = ["fp8_e4m3", "int8"]


def _codes(rng, shape, fmt):
    """Random valid codes (no fp8 NaN, no int8 -128)."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    if fmt == "fp8_e4m3":
        return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)
    return np.where(c == 0x80, 0x81, c).astype(np.uint8)


def _bf16_bits(rng, shape, spread=1.0):
    x = (rng.standard_normal(shape) * spread).astype(np.float32)
    return C.f32_to_bf16_bits(x)


@pytest.mark.parametrize("fmt", FMT)
def test_scatter_equal_head_scales_is_tensor_scale(fmt):
    rng = np.random.default_rng(1)
    nb, bs, hkv, d, t = 6, 16, 4, 64, 40
    kc, vc = _codes(rng, (nb, bs, hkv, d), fmt), _codes(rng, (nb, bs, hkv, d), fmt)
    k, v = _bf16_bits(rng, (t, hkv, d), 3.0), _bf16_bits(rng, (t, hkv, d), 3.0)
    slots = rng.permutation(nb * bs)[:t]
    inv = np.float32(1.0) / np.float32(0.0213)
    a = S.scatter(kc, vc, k, v, slots, bs, "bf16", fmt, inv, inv)
    b = S.scatter(kc, vc, k, v, slots, bs, "bf16", fmt, np.full(hkv, inv, np.float32),
                  np.full(hkv, inv, np.float32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("fmt", FMT)
def test_scatter_head_slice_is_tensor_write_of_that_slice(fmt):
    rng = np.random.default_rng(2)
    nb, bs, hkv, d, t = 5, 16, 4, 32, 50
    kc, vc = _codes(rng, (nb, bs, hkv, d), fmt), _codes(rng, (nb, bs, hkv, d), fmt)
    k, v = _bf16_bits(rng, (t, hkv, d), 4.0), _bf16_bits(rng, (t, hkv, d), 4.0)
    slots = list(rng.permutation(nb * bs)[:t])
    slots[3] = -1
    ks = np.array([0.004, 0.03, 0.011, 0.2], np.float32)
    vs = np.array([0.05, 0.0071, 0.13, 0.002], np.float32)
    kinv, vinv = np.float32(1.0) / ks, np.float32(1.0) / vs
    kh, vh = S.scatter(kc, vc, k, v, slots, bs, "bf16", fmt, kinv, vinv)
    for h in range(hkv):
        ka, va = S.scatter(kc[:, :, h:h + 1], vc[:, :, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], slots,
                           bs, "bf16", fmt, kinv[h], vinv[h])
        assert np.array_equal(kh[:, :, h:h + 1], ka) and np.array_equal(vh[:, :, h:h + 1], va)
    # the heads' scales really differ in effect: a tensor write with head 0's
    # scale differs from the per-head write on some other head
    kt, _ = S.scatter(kc, vc, k, v, slots, bs, "bf16", fmt, kinv[0], vinv[0])
    assert not np.array_equal(kt, kh)


@pytest.mark.parametrize("fmt", FMT)
def test_decode_cache_head_slices(fmt):
    rng = np.random.default_rng(3)
    bits = _codes(rng, (3, 16, 4, 32), fmt)
    sc = np.array([0.5, 0.0625, 3.0, 0.01], np.float32)
    full = A.decode_cache(bits, fmt, sc)
    for h in range(4):
        assert np.array_equal(full[:, :, h], A.decode_cache(bits[:, :, h:h + 1], fmt, float(sc[h]))[:, :, 0])


def _pool(rng, fmt, nb, bs, hkv, d):
    return _codes(rng, (nb, bs, hkv, d), fmt), _codes(rng, (nb, bs, hkv, d), fmt)


@pytest.mark.parametrize("fmt", FMT)
def test_v_head_scale_multiplies_its_group_output(fmt):
    rng = np.random.default_rng(4)
    nb, bs, hq, hkv, d = 12, 16, 8, 2, 32
    G = hq // hkv
    kc, vc = _pool(rng, fmt, nb, bs, hkv, d)
    seq = [37, 70, 5]
    qlen = [1, 3, 2]
    qsl = np.concatenate([[0], np.cumsum(qlen)])
    q = rng.standard_normal((int(qsl[-1]), hq, d))
    perm = rng.permutation(nb)
    tables = [list(perm[:3]), list(perm[3:8]), list(perm[8:9])]
    ks = 0.037
    vs = np.array([0.02, 0.3], np.float32)
    got = A.paged_attention(q, kc, vc, tables, qsl, seq, bs, cache_dtype=fmt, k_scale=ks, v_scale=vs)
    one = A.paged_attention(q, kc, vc, tables, qsl, seq, bs, cache_dtype=fmt, k_scale=ks, v_scale=1.0)
    for r in got:
        for h in range(hq):
            assert np.allclose(got[r][:, h], float(vs[h // G]) * one[r][:, h], rtol=1e-12, atol=0)


@pytest.mark.parametrize("fmt", FMT)
def test_k_head_scale_acts_as_group_softmax_scale(fmt):
    rng = np.random.default_rng(5)
    nb, bs, hq, hkv, d = 10, 16, 6, 3, 32
    G = hq // hkv
    kc, vc = _pool(rng, fmt, nb, bs, hkv, d)
    seq = [50, 21]
    qlen = [2, 1]
    qsl = np.concatenate([[0], np.cumsum(qlen)])
    q = rng.standard_normal((int(qsl[-1]), hq, d))
    perm = rng.permutation(nb)
    tables = [list(perm[:4]), list(perm[4:6])]
    ks = np.array([0.01, 0.09, 0.04], np.float32)
    scale = 1.0 / math.sqrt(d)
    got = A.paged_attention(q, kc, vc, tables, qsl, seq, bs, cache_dtype=fmt, k_scale=ks, v_scale=0.5)
    for g in range(hkv):
        ref = A.paged_attention(q, kc, vc, tables, qsl, seq, bs, scale=scale * float(ks[g]),
                                cache_dtype=fmt, k_scale=1.0, v_scale=0.5)
        for r in got:
            for h in range(g * G, (g + 1) * G):
                assert np.allclose(got[r][:, h], ref[r][:, h], rtol=1e-10, atol=1e-12)
