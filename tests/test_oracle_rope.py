"""Pins of the oracle's rotary embedding + cache write (oracle/rope.py) and of
the float32 -> bfloat16 rounding (oracle/codecs.py).

The pages print no RoPE numbers, so the pins are closed forms and invariants:
position 0 and a quarter turn are exact, the float32 steps stay within one
output ulp of the exact rotation, rotations preserve pair norms and add angles,
the interleaved layout is the half-split layout under a fixed permutation,
partial rotation leaves the tail alone, and the fused write equals "rotate,
then scatter" with out-of-table tokens writing nothing.  The bf16 rounding is
checked against an independent library conversion (PyTorch's CPU cast),
including exact ties.
"""

import numpy as np
import pytest
import torch

from oracle import cache, codecs, rope

RNG = np.random.default_rng(1234)


def _bits(shape, dtype, scale=1.0):
    x = (RNG.standard_normal(shape) * scale).astype(np.float32)
    return codecs.f32_to_act_bits(x, dtype)


def test_table_closed_form():
    t = rope.cos_sin_table(3, 8, 10000.0)
    assert t.dtype == np.float32 and t.shape == (3, 8)
    assert np.array_equal(t[0], np.array([1, 1, 1, 1, 0, 0, 0, 0], np.float32))
    # position 1, pair j: angle 10000**(-2j/8)
    for j in range(4):
        a = 10000.0 ** (-j / 4.0)
        assert t[1, j] == np.float32(np.cos(a)) and t[1, 4 + j] == np.float32(np.sin(a))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("neox", [True, False])
def test_position_zero_is_identity(dtype, neox):
    table = rope.cos_sin_table(16, 64, 10000.0)
    x = _bits((5, 3, 64), dtype)
    y = rope.apply_rope(x, dtype, np.zeros(5, np.int64), table, 64, neox)
    assert np.array_equal(x, y)


@pytest.mark.parametrize("neox", [True, False])
def test_quarter_turn_exact(neox):
    # cos = 0, sin = 1 in every pair: (a, b) -> (-b, a) exactly
    D = 16
    table = np.zeros((2, D), np.float32)
    table[0, :D // 2] = 1.0
    table[1, D // 2:] = 1.0
    x = _bits((4, 2, D), "bf16")
    y = rope.apply_rope(x, "bf16", np.ones(4, np.int64), table, D, neox)
    i1, i2 = rope.pair_index(D, neox)
    xv = codecs.decode(x, "bf16")
    yv = codecs.decode(y, "bf16")
    assert np.array_equal(yv[..., i1], -xv[..., i2])
    assert np.array_equal(yv[..., i2], xv[..., i1])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_float32_steps_within_one_ulp_of_exact(dtype):
    table = rope.cos_sin_table(4096, 128, 500000.0)
    T, H, D = 64, 4, 128
    x = _bits((T, H, D), dtype, scale=3.0)
    pos = RNG.integers(0, 4096, T)
    y = codecs.decode(rope.apply_rope(x, dtype, pos, table, 128, True), dtype)
    cs = table[pos]
    exact = rope.rotate_f64(codecs.decode(x, dtype), cs[:, None, :64], cs[:, None, 64:], 128, True)
    # one ulp of the output format at the exact value (bf16: 8 bits, f16: 11 bits)
    mant = 8 if dtype == "bf16" else 11
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 2.0 ** -14))) - (mant - 1))
    assert np.all(np.abs(y - exact) <= ulp)


def test_rotation_preserves_pair_norm_and_adds_angles():
    table = rope.cos_sin_table(64, 32, 10000.0)
    x = RNG.standard_normal((8, 32))
    i1, i2 = rope.pair_index(32, True)

    def rot(v, p):
        return rope.rotate_f64(v, table[p, :16], table[p, 16:], 32, True)

    y = rot(x, 5)
    n0 = x[:, i1] ** 2 + x[:, i2] ** 2
    n1 = y[:, i1] ** 2 + y[:, i2] ** 2
    assert np.allclose(n0, n1, rtol=1e-6, atol=0)
    # rotating by 5 then 7 equals rotating by 12 (angles add; table rounding only)
    assert np.allclose(rot(rot(x, 5), 7), rot(x, 12), rtol=0, atol=1e-5)


def test_interleaved_is_half_split_under_permutation():
    D, rd = 64, 64
    table = rope.cos_sin_table(32, rd, 10000.0)
    x = _bits((6, 2, D), "bf16")
    pos = RNG.integers(0, 32, 6)
    # interleaved pair (2j, 2j+1) <-> half-split pair (j, j + rd/2)
    perm = np.empty(D, np.int64)
    perm[np.arange(rd // 2)] = 2 * np.arange(rd // 2)
    perm[rd // 2 + np.arange(rd // 2)] = 2 * np.arange(rd // 2) + 1
    y_inter = rope.apply_rope(x, "bf16", pos, table, rd, False)
    y_neox = rope.apply_rope(x[..., perm], "bf16", pos, table, rd, True)
    assert np.array_equal(y_inter[..., perm], y_neox)


@pytest.mark.parametrize("neox", [True, False])
def test_partial_rotation_leaves_tail(neox):
    table = rope.cos_sin_table(32, 32, 10000.0)
    x = _bits((5, 2, 128), "f16")
    pos = RNG.integers(1, 32, 5)
    y = rope.apply_rope(x, "f16", pos, table, 32, neox)
    assert np.array_equal(y[..., 32:], x[..., 32:])
    assert not np.array_equal(y[..., :32], x[..., :32])


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8_e4m3"])
def test_fused_write_is_rotate_then_scatter(cache_dtype):
    T, Hq, Hkv, D, bs, NB = 9, 4, 2, 64, 16, 6
    table = rope.cos_sin_table(100, D, 10000.0)
    q, k, v = _bits((T, Hq, D), "bf16"), _bits((T, Hkv, D), "bf16"), _bits((T, Hkv, D), "bf16")
    pos = np.array([0, 5, 99, 100, -1, 17, 3, 42, 7])          # 100 and -1 are outside the table
    slots = np.array([0, 17, 33, 40, 41, -1, 95, 2, 50])
    cdt = np.uint8 if cache_dtype == "fp8_e4m3" else np.uint16
    kc0 = RNG.integers(0, 255, (NB, bs, Hkv, D)).astype(cdt)
    vc0 = RNG.integers(0, 255, (NB, bs, Hkv, D)).astype(cdt)
    ks = 1.0 / np.float32(0.05) if cache_dtype == "fp8_e4m3" else 1.0
    q2, kc, vc = rope.rope_cache_write(q, k, v, pos, table, D, True, slots, kc0, vc0, bs,
                                       "bf16", cache_dtype, ks, ks)
    ok = (pos >= 0) & (pos < 100)
    # query rows: rotated where the position is in the table, untouched elsewhere
    assert np.array_equal(q2[~ok], q[~ok])
    assert np.array_equal(q2[ok], rope.apply_rope(q[ok], "bf16", pos[ok], table, D, True))
    k_rot = rope.apply_rope(k, "bf16", np.where(ok, pos, 0), table, D, True)
    ekc, evc = cache.scatter(kc0, vc0, k_rot, v, np.where(ok, slots, -1), bs, "bf16",
                             cache_dtype, ks, ks)
    assert np.array_equal(kc, ekc) and np.array_equal(vc, evc)
    # the out-of-table tokens (slots 40, 41) wrote nothing
    assert np.array_equal(kc[2, 8], kc0[2, 8]) and np.array_equal(kc[2, 9], kc0[2, 9])


def test_bf16_rounding_matches_library_cast():
    x = RNG.standard_normal(1 << 18).astype(np.float32) * np.float32(1e3)
    # exact ties: low 16 bits = 0x8000, both parities of the kept part
    ties = ((RNG.integers(0, 1 << 15, 4096, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.4028235e38, -3.4028235e38,
                        1e-45, -1e-45, 1.1754944e-38], np.float32)
    allx = np.concatenate([x, ties, special])
    ours = codecs.f32_to_bf16_bits(allx)
    ref = torch.from_numpy(allx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(allx)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0)
