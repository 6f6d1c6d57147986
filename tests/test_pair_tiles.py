"""The tile numbering of the paired GEMM kernels (host check).

The paired kernels (bf16 and MXFP4, 64- or 128-row blocks) take tiles of up
to two consecutive blocks of one expert times 256 weight rows.  A pair table
lists each expert's pairs from the first block of its run (the last pair of
an odd block count holds one block); an expert's pairs form windows of two,
and a window's N tiles are numbered interleaved, (pair 0, n 0), (pair 1,
n 0), (pair 0, n 1), ..., so the two tiles that read the same weight rows
run side by side.  The kernels restate this in ``write_pair_table``
(align_block.h), ``pair_table_kernel`` and ``pair_tile`` (common.h); this
test restates it once more and checks, for routings of several shapes and
both block sizes, that the logical tiles [0, pairs x N tiles) cover every
(block, N tile) of the padded layout exactly once, with both blocks of a
tile belonging to one expert and every block index inside the block table.
The layout comes from the oracle's alignment.
"""

import numpy as np
import pytest

from oracle import align as oalign
from synth import make_topk_ids

TWO, WIN_FIRST, WIN_SECOND = 1 << 30, 1 << 29, 1 << 31
BLOCK_MASK = (1 << 29) - 1


def pair_table(start, bm):
    """Pair entries from the experts' first padded rows start[0..E]."""
    tab = []
    for e in range(len(start) - 1):
        nb = (start[e + 1] - start[e]) // bm
        m = (nb + 1) // 2
        for j in range(m):
            v = start[e] // bm + 2 * j
            v |= TWO if 2 * j + 1 < nb else 0
            v |= WIN_FIRST if (j % 2 == 0 and j + 1 < m) else 0
            v |= WIN_SECOND if j % 2 == 1 else 0
            tab.append(v)
    return tab


def pair_tile(tab, L, ntn):
    """(first block, two blocks, N tile) of logical tile L."""
    jj = L // ntn
    fw = tab[jj]
    w, sz = jj, 1
    if (fw & WIN_FIRST) and jj + 1 < len(tab):
        sz = 2
    elif (fw & WIN_SECOND) and jj > 0:
        w, sz = jj - 1, 2
    local = L - ntn * w
    pe = tab[w + local % sz]
    return pe & BLOCK_MASK, bool(pe & TWO), local // sz


CASES = [(T, k, E, kind) for T, k, E in ((8192, 6, 256), (4096, 8, 128), (700, 2, 8), (3000, 4, 16))
         for kind in ("uniform", "skewed")] + [(512, 8, 64, "hot")]


@pytest.mark.parametrize("T,k,E,kind", CASES)
@pytest.mark.parametrize("bm", [64, 128])
def test_pair_tiles_cover_every_block_once(T, k, E, kind, bm):
    ids = make_topk_ids(T, k, E, seed=T + k, kind=kind).numpy()
    _, block_expert, npp, _ = oalign.align(ids, E, bm)
    counts = np.bincount(ids.ravel(), minlength=E)
    start = np.concatenate([[0], np.cumsum(-(-counts // bm) * bm)])
    assert start[-1] == npp
    nblk = npp // bm
    tab = pair_table(start, bm)
    assert len(tab) <= nblk
    for ntn in (1, 3, 16):
        hits = np.zeros((nblk, ntn), dtype=np.int64)
        for L in range(len(tab) * ntn):
            blk, two, nt = pair_tile(tab, L, ntn)
            assert 0 <= blk and blk + two < nblk and 0 <= nt < ntn
            if two:
                assert block_expert[blk] == block_expert[blk + 1], "a pair spans two experts"
            hits[blk, nt] += 1
            if two:
                hits[blk + 1, nt] += 1
        assert np.all(hits == 1)
