"""Pins of the oracle's mask variants (sliding window, ALiBi).

* library: the paged result equals torch's scaled_dot_product_attention (CPU,
  float64) on contiguous K/V with an additive float mask that holds the ALiBi
  bias on allowed keys and -inf elsewhere;
* reductions: a window of 1 returns the query's own value; a window of W
  equals plain attention over only the W most recent keys (K/V sliced, no
  window); a window at least as long as the sequence, and zero slopes, change
  nothing;
* closed form: two equal keys under slope m weigh 1 and e^-m.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import metadata as M


def _setup(rng, comp, ql, hq, hkv, d, bs, pool_blocks):
    seq = [c + n for c, n in zip(comp, ql)]
    perm = rng.permutation(pool_blocks)
    rows, k = [], 0
    for s in seq:
        nb = M.blocks_for_tokens(s, bs)
        rows.append(perm[k:k + nb].tolist())
        k += nb
    kc = rng.standard_normal((pool_blocks, bs, hkv, d))
    vc = rng.standard_normal((pool_blocks, bs, hkv, d))
    q = rng.standard_normal((sum(ql), hq, d))
    qsl = np.concatenate([[0], np.cumsum(ql)])
    return seq, rows, kc, vc, q, qsl


def _sdpa(q, k, v, c, scale, window, slopes):
    n, hq, d = q.shape
    s, hkv, _ = k.shape
    g = hq // hkv
    kk = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)
    vv = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)
    qq = torch.from_numpy(q).permute(1, 0, 2)
    pos = c + torch.arange(n, dtype=torch.float64)[:, None]          # query positions
    key = torch.arange(s, dtype=torch.float64)[None, :]
    ok = key <= pos
    if window:
        ok &= key >= pos - (window - 1)
    bias = torch.zeros((hq, n, s), dtype=torch.float64)
    if slopes is not None:
        bias = torch.from_numpy(np.asarray(slopes, np.float64))[:, None, None] * (key - pos)[None]
    mask = torch.where(ok[None], bias, torch.tensor(-math.inf, dtype=torch.float64))
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


def alibi_slopes(h):
    """The geometric slopes 2^(-8 i / h), i = 1..h (a common choice; any slopes work)."""
    return np.array([2.0 ** (-8.0 * (i + 1) / h) for i in range(h)])


@pytest.mark.parametrize("window", [0, 1, 5, 16, 40])
@pytest.mark.parametrize("alibi", [False, True])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_paged_masks_equal_sdpa(window, alibi, hq, hkv):
    rng = np.random.default_rng(window * 7 + hq + 3 * alibi)
    comp, ql = [0, 9, 37, 50], [13, 1, 20, 1]
    d, bs = 16, 4
    seq, rows, kc, vc, q, qsl = _setup(rng, comp, ql, hq, hkv, d, bs, 96)
    slopes = alibi_slopes(hq) if alibi else None
    scale = 0.3
    got = A.paged_attention(q, kc, vc, rows, qsl, seq, bs, scale=scale, sliding_window=window,
                            alibi_slopes=slopes)
    for r in range(len(seq)):
        k, v = A.gather_request_kv(kc, vc, rows[r], seq[r], bs)
        want = _sdpa(q[qsl[r]:qsl[r + 1]], k, v, comp[r], scale, window, slopes)
        np.testing.assert_allclose(got[r], want, rtol=1e-10, atol=1e-12)


def test_window_one_returns_own_value():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((30, 2, 8))
    v = rng.standard_normal((30, 2, 8))
    q = rng.standard_normal((6, 4, 8))
    out = A.causal_attention(q, k, v, 24, 0.5, sliding_window=1, alibi_slopes=alibi_slopes(4))
    for i in range(6):
        for h in range(4):
            np.testing.assert_array_equal(out[i, h], v[24 + i, h // 2])


@pytest.mark.parametrize("window", [1, 3, 8, 17])
def test_window_equals_plain_attention_over_recent_keys(window):
    rng = np.random.default_rng(window)
    s, hq, hkv, d = 40, 4, 2, 8
    k = rng.standard_normal((s, hkv, d))
    v = rng.standard_normal((s, hkv, d))
    q = rng.standard_normal((1, hq, d))
    got = A.causal_attention(q, k, v, s - 1, 0.4, sliding_window=window)
    lo = s - window
    want = A.causal_attention(q, k[lo:], v[lo:], window - 1, 0.4)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-14)


def test_long_window_and_zero_slopes_change_nothing():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((20, 1, 8))
    v = rng.standard_normal((20, 1, 8))
    q = rng.standard_normal((5, 4, 8))
    plain = A.causal_attention(q, k, v, 15, 0.5)
    np.testing.assert_array_equal(A.causal_attention(q, k, v, 15, 0.5, sliding_window=20), plain)
    np.testing.assert_array_equal(A.causal_attention(q, k, v, 15, 0.5, sliding_window=1000), plain)
    np.testing.assert_allclose(A.causal_attention(q, k, v, 15, 0.5, alibi_slopes=np.zeros(4)), plain,
                               rtol=0, atol=0)


@pytest.mark.parametrize("m", [0.0, 0.25, 3.0])
def test_alibi_two_equal_keys_closed_form(m):
    rng = np.random.default_rng(3)
    key = rng.standard_normal(8)
    k = np.stack([key, key])[:, None, :]                 # positions 0 and 1, equal scores
    v = rng.standard_normal((2, 1, 8))
    q = rng.standard_normal((1, 1, 8))
    out = A.causal_attention(q, k, v, 1, 0.7, alibi_slopes=[m])
    w_old = math.exp(-m)                                 # key 0 is one position behind
    want = (w_old * v[0, 0] + v[1, 0]) / (w_old + 1.0)
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-14, atol=1e-15)
