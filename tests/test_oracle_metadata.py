"""Pins of the oracle's metadata against values the pages print.

Fixtures: tests/golden/walkthrough_metadata.json ("Tour: One forward pass",
stops 1, 3, 4, 5, 10) and tests/golden/deep_dive_blocks.json ("vLLM 推理全流程深度解析",
BlockManager and prepare_input_tensors examples).
"""

import json
import os

import numpy as np
import pytest

from oracle import metadata as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_blocks_for_tokens_page_values():
    w = load("walkthrough_metadata.json")
    d = load("deep_dive_blocks.json")
    assert M.blocks_for_tokens(298, 16) == w["expect"]["r3_blocks"] == 19
    assert M.blocks_for_tokens(35, 16) == d["seq_a"]["num_blocks"] == 3
    # ceiling division: an exact multiple needs no spare block (reading of stop 1)
    assert M.blocks_for_tokens(32, 16) == 2
    assert M.blocks_for_tokens(1, 16) == 1
    assert M.blocks_for_tokens(0, 16) == 0


def _walkthrough_tables(rng):
    # The page prints no block ids; use a permutation of a 2048-block pool.
    perm = rng.permutation(2048)
    rows = [perm[0:34], perm[34:43], perm[43:62]]
    return [list(map(int, r)) for r in rows]


def test_walkthrough_metadata_matches_page():
    w = load("walkthrough_metadata.json")
    e = w["expect"]
    bs = w["block_size"]
    rng = np.random.default_rng(1)
    bt = _walkthrough_tables(rng)
    qsl, seq_lens, pos, slot = M.build_metadata(
        w["num_computed_tokens"], w["query_lens"], bt, bs,
        w["num_tokens_padded"], qsl_len=w["qsl_buffer_len"])
    assert qsl[:4] == e["query_start_loc"]
    assert all(v == e["query_start_loc_padding_value"] for v in qsl[4:])
    assert len(qsl) == w["qsl_buffer_len"]
    assert seq_lens == e["seq_lens"]
    assert pos[:4] == e["positions_head"]
    assert pos[299] == e["positions_last_real"]
    assert qsl[3] == e["num_actual_tokens"]
    for t in e["padding_rows"]:
        assert slot[t] == e["padding_slot"]
        assert pos[t] is None
    bi, off = e["block_index_offset"]["R1"]
    assert slot[0] == bt[0][bi] * bs + off
    bi, off = e["block_index_offset"]["R2"]
    assert slot[1] == bt[1][bi] * bs + off
    bi, off = e["block_index_offset"]["R3_last"]
    assert slot[299] == bt[2][bi] * bs + off
    # R3 spans block indexes 0..18, the last holding 10 tokens
    r3_blocks = sorted({slot[t] // bs for t in range(2, 300)})
    assert r3_blocks == sorted(bt[2][:19])
    last = [t for t in range(2, 300) if slot[t] // bs == bt[2][18]]
    assert len(last) == e["r3_tokens_in_last_block"]
    assert max(w["query_lens"]) == e["max_query_len"]
    assert max(seq_lens) == e["max_seq_len"]
    assert seq_lens == e["keys_read_per_request"]


def test_deep_dive_slot_example():
    d = load("deep_dive_blocks.json")
    a = d["seq_a"]
    bs = d["block_size"]
    qsl, seq_lens, pos, slot = M.build_metadata([0], [a["prompt_len"]], [a["block_table"]], bs, 35)
    assert slot[:2] == a["slots_first"]
    assert slot[16] == a["slot_16"]
    assert slot[34] == a["slot_last"]
    assert slot[:16] == [12 * 16 + i for i in range(16)]
    assert slot[16:32] == [45 * 16 + i for i in range(16)]
    assert slot[32:35] == [89 * 16 + i for i in range(3)]


def test_deep_dive_batch_shapes():
    d = load("deep_dive_blocks.json")
    b = d["batch"]
    qsl, seq_lens, pos, slot = M.build_metadata(
        b["num_computed_tokens"], b["query_lens"], b["block_tables"], d["block_size"], b["num_tokens"])
    assert qsl[-1] == b["num_tokens"] == 56
    assert seq_lens == b["seq_lens"]
    ctx = [s - n for s, n in zip(seq_lens, b["query_lens"])]
    assert ctx == b["context_lens"]
    assert pos == list(range(35)) + list(range(20)) + [5]
    # Seq C decodes position 5 in its first block (id 3): formula 3*16+5
    assert slot[55] == 3 * 16 + 5
    # Seq B's last token (position 19) is in its second block (id 22)
    assert slot[54] == 22 * 16 + 3
    x = d["input_ids_shape_two_prefill_three_decode"]
    assert sum(x["prefill_lens"]) + x["num_decodes"] == x["total"]


def test_slot_and_block_table_consistency_random():
    """slot[t] == bt[r][pos // bs] * bs + pos % bs and positions run c_r .. c_r+n_r-1."""
    rng = np.random.default_rng(7)
    for _ in range(20):
        bs = int(rng.choice([8, 16, 32]))
        R = int(rng.integers(1, 9))
        comp = rng.integers(0, 100, size=R).tolist()
        ql = rng.integers(0, 40, size=R).tolist()
        pool = 4096
        perm = rng.permutation(pool)
        rows, k = [], 0
        for c, n in zip(comp, ql):
            nb = M.blocks_for_tokens(c + n, bs)
            rows.append(perm[k:k + nb].tolist())
            k += nb
        T = sum(ql)
        Tpad = T + int(rng.integers(0, 5))
        qsl, sl, pos, slot = M.build_metadata(comp, ql, rows, bs, Tpad)
        seen = set()
        for r in range(R):
            for i in range(ql[r]):
                t = qsl[r] + i
                p = comp[r] + i
                assert pos[t] == p
                assert slot[t] == rows[r][p // bs] * bs + p % bs
                assert slot[t] not in seen
                seen.add(slot[t])
        for t in range(T, Tpad):
            assert slot[t] == -1
        assert qsl == [0] + list(np.cumsum(ql))


def test_empty_requests_produce_no_rows():
    qsl, sl, pos, slot = M.build_metadata([3, 0, 7], [0, 2, 0], [[5], [9], [1]], 16, 4)
    assert qsl == [0, 0, 2, 2]
    assert sl == [3, 2, 7]
    assert pos[:2] == [0, 1]
    assert slot == [9 * 16, 9 * 16 + 1, -1, -1]


@pytest.mark.parametrize("bs", [16])
def test_table_too_narrow_gives_pad_slot(bs):
    qsl, sl, pos, slot = M.build_metadata([16], [1], [[4]], bs, 1)
    assert pos == [16]
    assert slot == [-1]
