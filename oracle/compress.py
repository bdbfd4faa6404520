"""Compressor pooling: raw KV rows -> compressed KV rows (oracle; test infrastructure only).

Compressed layers keep, besides the raw sliding-window ring, rows pooled from the
raw rows: one compressed row per `ratio` raw rows (4 or 128), appended when a
ratio boundary is reached, with a rolling KV/score state holding the rows of the
group not yet complete ([P-DS4] "Architecture Deep Dive", Layer Compression and
KV Cache Design; "GPU Backend Architecture" lists compressor update and prefill
among the GPU operations).  The pages name the state (pending KV rows and their
scores) but give no formula.  Readings taken:

* a score accompanies every element of a raw row (the state holds KV and score
  rows of the same shape); the learned projection that produces the scores is
  not on the pages and the scores are inputs here;
* pooling: element d of the compressed row of group c is the softmax-weighted
  sum, over the group's `ratio` rows i, of kv[i][d] with weights
  exp(s[i][d]) / sum_j exp(s[j][d]) -- a softmax over the group, per element;
* streaming: rows arrive in order; the state holds the n_state < ratio rows of
  the current incomplete group; a call appends its new rows to that stream,
  emits one compressed row for every complete group, and keeps the trailing
  (n_state + n_new) mod ratio rows as the new state.

The definition is written out plainly in float64: per group, per element, a max,
the exponentials, their sum and the weighted sum.

Parity unpinned: the formula is this package's reading, not the pages'.  The
checks in tests/test_oracle_compress.py pin the code to the reading (brute force,
closed forms, invariants, planted mistakes); nothing on the pages pins the reading.
"""

from __future__ import annotations

import numpy as np


def pool_groups(kv: np.ndarray, score: np.ndarray, ratio: int) -> np.ndarray:
    """float64 [n // ratio, D]: one pooled row per complete group of `ratio` rows.

    kv, score: [n, D] (any float type; widened to float64).  Rows past the last
    complete group are ignored."""
    kv = np.asarray(kv, dtype=np.float64)
    s = np.asarray(score, dtype=np.float64)
    n, d = kv.shape
    groups = n // ratio
    out = np.zeros((groups, d), dtype=np.float64)
    for c in range(groups):
        g_kv = kv[c * ratio:(c + 1) * ratio]
        g_s = s[c * ratio:(c + 1) * ratio]
        m = g_s.max(axis=0)                      # per element
        w = np.exp(g_s - m)
        out[c] = (w * g_kv).sum(axis=0) / w.sum(axis=0)
    return out


def compress_step(state_kv: np.ndarray, state_score: np.ndarray, kv_new: np.ndarray,
                  score_new: np.ndarray, ratio: int):
    """One compressor call on one sequence.

    state_kv, state_score: [n_state, D] pending rows (n_state < ratio).
    kv_new, score_new: [n_new, D].
    Returns (pooled [n_out, D] float64, new_state_kv, new_state_score) where the
    new state rows are copies of the trailing (n_state + n_new) mod ratio rows of
    the stream (in the inputs' own types)."""
    if state_kv.shape[0] >= ratio:
        raise ValueError("the state holds fewer than `ratio` rows")
    kv = np.concatenate([state_kv, kv_new], axis=0)
    sc = np.concatenate([state_score, score_new], axis=0)
    n_out = kv.shape[0] // ratio
    pooled = pool_groups(kv, sc, ratio)
    rest = n_out * ratio
    return pooled, kv[rest:].copy(), sc[rest:].copy()
