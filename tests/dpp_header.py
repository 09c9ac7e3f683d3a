"""Parse the work list a plan uploads (record layout of csrc/dpp_internal.h)."""
from dataclasses import dataclass

import numpy as np

MAGIC = 0x44505031
HEADER_WORDS = 16


@dataclass
class ParsedPlan:
    requests: np.ndarray  # [B, 4]: q_start, qo_len, page_start, kv_len
    items: np.ndarray     # [N, 16]: request, row_start, split, tile_splits, kv_tile_begin, kv_tile_end,
                          # slot_base, pass, then the request's q_start, qo_len, page_start, kv_len, pad x4
    merges: np.ndarray    # [M, 4]: request, row_start, tile_splits, slot_base
    units: np.ndarray     # [U, 16]: persistent launches' unit records: the item's first 7 words,
                          # next, the request's 4 words, kv_head, block, pass, pad
    tables: dict          # pass -> block table of its wide launch when not persistent: entry b is
                          # the unit (kv_head * items + item) block b runs, -1 none


def parse(words: np.ndarray) -> ParsedPlan:
    w = np.asarray(words, dtype=np.int64)
    assert (int(w[0]) & 0xFFFFFFFF) == MAGIC
    nreq, nitems, nmerge, roff, ioff, moff = (int(x) for x in w[1:7])
    req = w[roff:roff + 4 * nreq].reshape(nreq, 4)
    items = w[ioff:ioff + 16 * nitems].reshape(nitems, 16)
    merges = w[moff:moff + 4 * nmerge].reshape(nmerge, 4)
    assert (w[8:12] == 0).all(), "zero chunk"
    uoff, nunits = int(w[12]), int(w[13])
    units = w[uoff:uoff + 16 * nunits].reshape(nunits, 16)
    toff, ntables = int(w[14]), int(w[15])
    tables = {}
    for _ in range(ntables):
        ps, blocks = int(w[toff]), int(w[toff + 1])
        tables[ps] = w[toff + 2:toff + 2 + blocks]
        toff += 2 + blocks
    assert toff == len(w) or ntables == 0, "block tables end the work list"
    return ParsedPlan(req, items, merges, units, tables)
