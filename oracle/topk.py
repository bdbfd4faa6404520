"""Indexer top-k selection from given scores (oracle; test infrastructure only).

Ratio-4 layers attend, for each token, the top-512 compressed rows that an
indexer selects ([P-DS4] "Architecture Deep Dive", Layer Compression; "GPU
Backend Architecture" lists the indexed mixed attention that consumes the list).
How the indexer scores rows is learned and not on the pages; what is defined
here is the selection step on given scores.

Readings taken where the pages are silent:

* order: float32 scores compare by the IEEE total order of their bit patterns
  (-0 < +0; a NaN with the sign bit clear ranks above +inf, one with it set
  below -inf), i.e. by ``order_key`` below;
* ties (equal keys) go to the lower index, so the selection is unique;
* the result lists the selected indices in ascending order (the attention reads
  the list as a set); a row with fewer than k scores lists all of them and pads
  with -1, the "unused entry" of the attention's index list.

The definition: for each row, the min(k, n) indices i that come first when the
indices are ordered by (order_key(s_i) descending, i ascending), then sorted.
"""

from __future__ import annotations

import numpy as np


def order_key(x: np.ndarray) -> np.ndarray:
    """Unsigned 32-bit keys whose integer order is the total order of the float32
    bit patterns: positive floats get the sign bit set, negative ones are
    complemented (so larger magnitudes of negatives rank lower)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    neg = (u >> np.uint32(31)).astype(bool)
    return np.where(neg, ~u, u | np.uint32(0x80000000)).astype(np.uint32)


def topk(scores: np.ndarray, k: int) -> np.ndarray:
    """int32 [rows, k]: per row the k largest scores' indices, ascending, -1 padded."""
    s = np.asarray(scores, dtype=np.float32)
    rows, n = s.shape
    out = np.full((rows, k), -1, dtype=np.int32)
    m = min(k, n)
    idx = np.arange(n, dtype=np.int64)
    for r in range(rows):
        key = order_key(s[r]).astype(np.int64)
        # lexsort sorts by the last key first: descending key, then ascending index
        order = np.lexsort((idx, -key))
        out[r, :m] = np.sort(order[:m])
    return out
