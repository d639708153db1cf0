"""Pins of the oracle's block copy / swap (oracle/blocks.py).

Every block of a test pool holds a pattern computed from its own id, so what
a block must hold after a copy is written down from the pair list alone
(block d must show the pattern of block s) without running any copy.  The
deep dive's sequence A (table [12, 45, 89], tests/golden/deep_dive_blocks.json)
is the sharing example: a beam candidate forks from A, shares blocks 12 and
45, and gets a private copy of the partly filled block 89.
"""

import json
import os

import numpy as np
import pytest

from oracle import blocks as OB

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BS, H, D = 16, 2, 8


def pattern(block_id, salt, dtype=np.uint16):
    """[BS, H, D] bits that name their block: distinct for every (block, salt)."""
    i = np.arange(BS)[:, None, None]
    h = np.arange(H)[None, :, None]
    d = np.arange(D)[None, None, :]
    mod = 251 if dtype == np.uint8 else 65521
    return ((block_id * 131 + salt * 17 + i * 11 + h * 5 + d) % mod).astype(dtype)


def pool(num_blocks, salt, dtype=np.uint16):
    return np.stack([pattern(b, salt, dtype) for b in range(num_blocks)])


def expect(num_blocks, salt, moved, dtype=np.uint16, src_salt=None):
    """Pool whose block d shows the pattern of source block s for (s, d) in moved."""
    out = pool(num_blocks, salt, dtype)
    for s, d in moved:
        out[d] = pattern(s, salt if src_salt is None else src_salt, dtype)
    return out


def test_beam_fork_copies_the_shared_last_block():
    seq_a = json.load(open(os.path.join(GOLDEN, "deep_dive_blocks.json")))["seq_a"]
    table = seq_a["block_table"]                          # [12, 45, 89]
    k, v = pool(128, 1), pool(128, 2)
    fresh = 100                                           # a free block for the candidate
    nk, nv = OB.copy_blocks(k, v, k, v, [(table[-1], fresh)])
    assert np.array_equal(nk, expect(128, 1, [(89, 100)]))
    assert np.array_equal(nv, expect(128, 2, [(89, 100)]))
    # the candidate's table [12, 45, 100] now reads what A's [12, 45, 89] reads
    cand = table[:-1] + [fresh]
    assert np.array_equal(nk[cand], nk[table]) and np.array_equal(nv[cand], nv[table])
    # the inputs are not modified
    assert np.array_equal(k, pool(128, 1)) and np.array_equal(v, pool(128, 2))


def test_swap_out_and_back_in_restores_the_blocks():
    gpu_k, gpu_v = pool(64, 3), pool(64, 4)
    host_k, host_v = pool(32, 5), pool(32, 6)
    out_pairs = [(7, 0), (40, 31), (63, 9)]               # GPU block -> host block
    hk, hv = OB.copy_blocks(gpu_k, gpu_v, host_k, host_v, out_pairs)
    assert np.array_equal(hk, expect(32, 5, out_pairs, src_salt=3))
    assert np.array_equal(hv, expect(32, 6, out_pairs, src_salt=4))
    # swap back in to other GPU blocks of a pool whose contents were overwritten
    later_k, later_v = pool(64, 7), pool(64, 8)
    in_pairs = [(0, 1), (31, 2), (9, 3)]                  # host block -> GPU block
    gk, gv = OB.copy_blocks(hk, hv, later_k, later_v, in_pairs)
    for (g_old, h), (_, g_new) in zip(out_pairs, in_pairs):
        assert np.array_equal(gk[g_new], pattern(g_old, 3))
        assert np.array_equal(gv[g_new], pattern(g_old, 4))
    untouched = [b for b in range(64) if b not in (1, 2, 3)]
    assert np.array_equal(gk[untouched], pool(64, 7)[untouched])


def test_reads_see_the_pool_before_the_call():
    k, v = pool(8, 1), pool(8, 2)
    nk, _ = OB.copy_blocks(k, v, k, v, [(1, 2), (2, 3)])
    # block 3 receives block 2 as it was, not block 1's copy
    assert np.array_equal(nk, expect(8, 1, [(1, 2), (2, 3)]))


@pytest.mark.parametrize("pair", [(-1, 3), (3, -1), (8, 3), (3, 8), (1 << 40, 0)])
def test_out_of_pool_pairs_are_skipped(pair):
    k, v = pool(8, 1), pool(8, 2)
    nk, nv = OB.copy_blocks(k, v, k, v, [pair, (0, 5)])
    assert np.array_equal(nk, expect(8, 1, [(0, 5)]))
    assert np.array_equal(nv, expect(8, 2, [(0, 5)]))


def test_fp8_pools_move_as_bytes():
    k, v = pool(16, 1, np.uint8), pool(16, 2, np.uint8)
    hk, hv = pool(4, 3, np.uint8), pool(4, 4, np.uint8)
    nk, nv = OB.copy_blocks(k, v, hk, hv, [(15, 0), (2, 3)])
    assert nk.dtype == np.uint8
    assert np.array_equal(nk, expect(4, 3, [(15, 0), (2, 3)], np.uint8, src_salt=1))
    assert np.array_equal(nv, expect(4, 4, [(15, 0), (2, 3)], np.uint8, src_salt=2))


def test_random_pairs_against_a_flat_byte_loop():
    rng = np.random.default_rng(5)
    k = rng.integers(0, 1 << 16, (50, BS, H, D), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, (50, BS, H, D), dtype=np.uint16)
    dst_k = rng.integers(0, 1 << 16, (30, BS, H, D), dtype=np.uint16)
    dst_v = rng.integers(0, 1 << 16, (30, BS, H, D), dtype=np.uint16)
    pairs = list(zip(rng.integers(0, 50, 20), rng.permutation(30)[:20]))
    nk, nv = OB.copy_blocks(k, v, dst_k, dst_v, pairs)
    # brute force over the flat bytes of each block
    nbytes = BS * H * D * 2
    fk, fv = bytearray(dst_k.tobytes()), bytearray(dst_v.tobytes())
    sk, sv = k.tobytes(), v.tobytes()
    for s, d in pairs:
        for j in range(nbytes):
            fk[d * nbytes + j] = sk[s * nbytes + j]
            fv[d * nbytes + j] = sv[s * nbytes + j]
    assert nk.tobytes() == bytes(fk) and nv.tobytes() == bytes(fv)
