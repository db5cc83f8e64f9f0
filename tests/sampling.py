"""Seeded choice of query rows for parity checks at full size.

Every output row of the block (and of attention) depends only on its own
input row and on the keys/values of all tokens, so comparing a subset of rows
is exact for those rows.  The subset always covers the first tile, the tile
boundaries around the visual/text seam and the valid-text bound, the ragged
last tile, and seeded random visual rows.
"""

import numpy as np


def sample_rows(n_vis, n_txt, valid, n_random=96, seed=0, tile=128):
    N = n_vis + n_txt
    rows = set(range(min(N, 8)))
    rows.update(range(max(0, tile - 2), min(N, tile + 2)))
    for L in valid:
        for c in (n_vis, n_vis + int(L)):
            rows.update(range(max(0, c - 3), min(N, c + 3)))
    last_tile = (N - 1) // tile * tile
    rows.update(range(max(0, last_tile - 2), min(N, last_tile + 3)))
    rows.update(range(max(0, N - 6), N))
    rng = np.random.default_rng(0xD17 + seed)
    if n_vis > 0:
        rows.update(int(r) for r in rng.integers(0, n_vis, n_random))
    if n_txt > 0:
        rows.update(int(n_vis + r) for r in rng.integers(0, n_txt, 8))
    return np.array(sorted(rows), dtype=np.int64)
