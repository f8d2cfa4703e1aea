"""The reference the tile-list parity tests build from an index set
(gpu_harness.expected_tile_modes), pinned on small hand-worked cases.

Mask modes of a causal key tile (query block qb, key block kb <= qb), from the
definition of the allowed pairs of Alg. 1's attention step (CRISP summary page,
Methodology, Algorithm Overview): a VS head allows key j of row i when j's block
is a selected vertical block or the offset block (i - j) / B is a selected slash
block; a slash block s covers the keys c <= r of tile qb - s (lower part, mode 1)
and the keys c > r of tile qb - s - 1 (upper part, mode 2); a vertical block, or a
block in a PE head's row, covers the whole tile (mode 3); the diagonal tile keeps
only its causal (lower) part.  The expected matrices below were worked out by hand
from those rules."""
import numpy as np

from gpu_harness import expected_tile_modes

X = -1  # above the diagonal (no tile)


def _lower(rows):
    nb = len(rows)
    m = np.full((nb, nb), X, np.int32)
    for qb, row in enumerate(rows):
        m[qb, : qb + 1] = row
    return m


def _check(head, nb, rows):
    got = expected_tile_modes(head, nb).astype(np.int32)
    want = _lower(rows)
    tri = np.tril_indices(nb)
    assert np.array_equal(got[tri], want[tri]), (got, want)
    assert not got[np.triu_indices(nb, 1)].any()  # nothing above the diagonal


def test_vs_head_hand_worked():
    # vertical {0, 2}, slash {0, 1}: e.g. tile (2, 1) is the lower part of slash 1
    # (qb - kb = 1) and the upper part of slash 0 (qb - kb - 1 = 0): both, mode 3;
    # tile (3, 1) only the upper part of slash 1: mode 2
    _check(dict(route=1, vertical=np.array([0, 2]), slash=np.array([0, 1])), 4,
           [[1], [3, 1], [3, 3, 1], [3, 2, 3, 1]])


def test_vs_head_last_slash_block_and_no_vertical():
    # slash {0, 3} only: slash 3 reaches tile (3, 0) (lower part) and nothing else
    # (its upper part would be tile qb - 4 < 0)
    _check(dict(route=1, vertical=np.array([], np.int32), slash=np.array([0, 3])), 4,
           [[1], [2, 1], [0, 2, 1], [1, 0, 2, 1]])


def test_pe_head_hand_worked():
    # rows: qb 0 -> {0}, qb 1 -> {0, 1}, qb 2 -> {2}, qb 3 -> {1, 3}
    _check(dict(route=0, rowptr=np.array([0, 1, 3, 4, 6]), cols=np.array([0, 0, 1, 2, 1, 3])), 4,
           [[1], [3, 1], [0, 0, 1], [0, 3, 0, 1]])
