"""Random block-table forests for plan tests (host only)."""

from __future__ import annotations

import numpy as np


def random_forest(rng, B, width, bs, alphabet):
    rows = []
    for i in range(B):
        if rows and rng.random() < 0.6:
            base = rows[int(rng.integers(0, len(rows)))]
            cut = int(rng.integers(0, width + 1))
            row = list(base[:cut]) + list(rng.integers(0, alphabet, size=width - cut))
        else:
            row = list(rng.integers(0, alphabet, size=width))
        rows.append(row)
    tables = np.array(rows, dtype=np.int32).reshape(B, width)
    lens = rng.integers(0, width * bs + 1, size=B).astype(np.int32)
    for i in range(B):
        nb = -(-int(lens[i]) // bs)
        tables[i, nb:] = rng.integers(-(2**31), 2**31, size=width - nb, dtype=np.int64).astype(np.int32)
    return tables, lens
