"""Per-step batch metadata of the oracle (test infrastructure only).

Follows "Tour: One forward pass":

* stop 1 -- a request of ``L`` tokens holds ``ceil(L / block_size)`` blocks
  (298 tokens -> 19 blocks at block size 16);
* stop 3 -- ``query_start_loc[0] = 0``, then the running sum of the scheduled
  token counts; entries past the last request are set to ``num_tokens`` so the
  buffer never decreases; ``seq_lens = num_computed_tokens + query_len``; the
  positions of a request's new tokens run from ``num_computed_tokens`` upward;
* stop 4 -- the slot of a token at position ``pos`` is
  ``block_table[pos // block_size] * block_size + pos % block_size``; the
  padding rows past the real tokens get ``PAD_SLOT_ID = -1``.

The batch row of request ``r`` is row ``r`` of ``block_tables`` (the table is
already in batch order, as stop 4's ``gather_block_tables`` leaves it).

Readings taken where the pages are silent or disagree:

* blocks per request: ceiling division (stop 1 of the tour); the deep-dive's
  BlockManager example writes ``len // block_size + 1``, which agrees for 35
  tokens but allocates one spare block when ``len`` is a multiple of the block
  size.
* positions of the padding rows are not written (stop 3: the kernels do not
  write the padding rows); only ``slot_mapping`` is padded, with -1.
* a token whose block-table entry would lie past the table's width gets -1.
"""

PAD_SLOT_ID = -1


def blocks_for_tokens(num_tokens, block_size):
    """Number of cache blocks holding ``num_tokens`` tokens: ceil(n / bs)."""
    return -(-int(num_tokens) // int(block_size))


def build_metadata(num_computed_tokens, query_lens, block_tables, block_size,
                   num_tokens_padded, qsl_len=None):
    """Return (query_start_loc, seq_lens, positions, slot_mapping) as int lists.

    ``num_computed_tokens`` / ``query_lens``: per request, in batch order.
    ``block_tables``: list of rows (lists of physical block ids), batch order.
    ``num_tokens_padded``: length of ``positions`` / ``slot_mapping``.
    ``qsl_len``: length of the query_start_loc buffer (default num_reqs + 1).

    ``positions[t]`` is ``None`` for padding rows (not written).
    """
    num_reqs = len(query_lens)
    if qsl_len is None:
        qsl_len = num_reqs + 1
    # query_start_loc: 0, running sum, then padded with num_tokens
    qsl = [0]
    for n in query_lens:
        qsl.append(qsl[-1] + int(n))
    num_tokens = qsl[-1]
    qsl = qsl + [num_tokens] * (qsl_len - len(qsl))

    seq_lens = [int(c) + int(n) for c, n in zip(num_computed_tokens, query_lens)]

    positions = [None] * num_tokens_padded
    slot_mapping = [PAD_SLOT_ID] * num_tokens_padded
    for r in range(num_reqs):
        row = block_tables[r]
        for i in range(int(query_lens[r])):
            t = qsl[r] + i
            if t >= num_tokens_padded:
                break
            pos = int(num_computed_tokens[r]) + i
            positions[t] = pos
            block_index = pos // block_size
            offset = pos % block_size
            if block_index < len(row):
                slot_mapping[t] = int(row[block_index]) * block_size + offset
            else:
                slot_mapping[t] = PAD_SLOT_ID
    return qsl, seq_lens, positions, slot_mapping
