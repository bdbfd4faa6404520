"""Plain float64 definition of the fused MQA attention step (oracle; test infrastructure only).

What is computed, and where the pages say so:

* Multi-query attention: every query head of a token attends with the one shared
  K/V head ([P-DS4] "Architecture Deep Dive", Fixed Model Shape: 64 heads, 1 KV
  head, head dim 512, 128-token sliding window).
* The keys a token may see come from two regions: the raw sliding-window rows and
  the pooled compressed rows; ratio-4 layers see only the indexer's top-512
  compressed rows, ratio-128 layers see all of them ([P-DS4] "Architecture Deep
  Dive", Layer Compression and KV Cache Design; "GPU Backend Architecture" lists
  raw, mixed and indexed mixed attention).  Both regions share one softmax.
* Q.K^T, softmax and the weighted sum of V form one fused operation ([P-Metal]
  "FlashAttention Kernel Architecture").  Masked pairs carry -inf, so a fully
  masked block contributes exactly nothing ([P-Metal] "Mask Handling and Block
  Skipping"): the blocked, skipping GPU method reaches the plain result below,
  up to rounding order.
* KV storage is padded to a multiple of 32 rows ([P-Metal] "KV-Cache Management
  on Metal Device Buffers"); the skip map holds one status byte per block
  ([P-Metal] "Mask Handling and Block Skipping").

Readings taken where the pages are silent:

* padded rows hold +0.0 and are never attended;
* status byte: 0 = every pair masked (skip), 1 = some pairs allowed, 2 = every
  pair allowed; a block is 32 KV rows by a tile of ``bq`` query tokens;
* window: key position p_k is visible to query position p_q iff
  0 <= p_q - p_k < window (the query's own row included); window 0 = no
  positional mask;
* index entries < 0 or >= n_rows are unused; entries act as a multiset;
* a query with no visible key outputs zeros.

The arithmetic is the definition itself: s_a = scale * sum_d q_d k_{a,d} over the
visible rows a, p_a = exp(s_a - max s) / sum exp(s - max s), o = sum_a p_a v_a,
all in float64 on the exact input values.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

ROWS_PER_BLOCK = 32  # [P-Metal] "KV-Cache Management on Metal Device Buffers"

SKIP, PARTIAL, FULL = 0, 1, 2


def ceil32(n: int) -> int:
    return -(-int(n) // ROWS_PER_BLOCK) * ROWS_PER_BLOCK


@dataclass
class Region:
    """One KV region: ``k``/``v`` are [B, >= n_rows, D]; ``valid`` is [B, >= n_rows] or None."""

    k: np.ndarray
    v: np.ndarray
    n_rows: int
    valid: Optional[np.ndarray] = None


@dataclass
class Problem:
    """Inputs of one attention call.

    ``q`` is [B, T, H, D]; ``scale`` is the float32 scale the caller passes (the
    oracle widens that exact value).  Region 0 holds the raw rows; row j sits at
    position ``k_pos0 + j`` and token t at ``q_pos0 + t``.  Region 1 (optional)
    holds compressed rows, either all visible under ``r1.valid`` or chosen per
    token by ``r1_index`` [B, T, k].
    """

    q: np.ndarray
    scale: float
    r0: Region
    window: int = 0
    q_pos0: int = 0
    k_pos0: int = 0
    r1: Optional[Region] = None
    r1_index: Optional[np.ndarray] = None

    @property
    def shape(self):
        b, t, h, d = self.q.shape
        return b, t, h, d


# --------------------------------------------------------------------------- visibility

def region0_allowed(p: Problem, b: int, t: int, rows: np.ndarray) -> np.ndarray:
    """Boolean visibility of region-0 rows ``rows`` for token ``t`` of sequence ``b``."""
    rows = np.asarray(rows, dtype=np.int64)
    ok = (rows >= 0) & (rows < p.r0.n_rows)
    if p.r0.valid is not None:
        vrow = np.zeros(rows.shape, dtype=bool)
        inside = rows < p.r0.n_rows
        vrow[inside] = np.asarray(p.r0.valid)[b, rows[inside]] != 0
        ok &= vrow
    if p.window > 0:
        delta = (p.q_pos0 + t) - (p.k_pos0 + rows)
        ok &= (delta >= 0) & (delta < p.window)
    return ok


def region1_rows(p: Problem, b: int, t: int) -> np.ndarray:
    """Visible region-1 rows of token ``t`` (a multiset when indexed)."""
    if p.r1 is None or p.r1.n_rows <= 0:
        return np.zeros(0, dtype=np.int64)
    n1 = p.r1.n_rows
    if p.r1_index is None:
        cand = np.arange(n1, dtype=np.int64)
    else:
        cand = np.asarray(p.r1_index[b, t], dtype=np.int64)
        cand = cand[(cand >= 0) & (cand < n1)]
    if p.r1.valid is not None:
        cand = cand[np.asarray(p.r1.valid)[b, cand] != 0]
    return cand


def visible_rows(p: Problem, b: int, t: int):
    """(region-0 rows, region-1 rows) visible to token t of sequence b."""
    r0 = np.arange(p.r0.n_rows, dtype=np.int64)
    r0 = r0[region0_allowed(p, b, t, r0)]
    return r0, region1_rows(p, b, t)


# --------------------------------------------------------------------------- attention

class _Widened:
    """float64 views of the inputs, made once per problem."""

    def __init__(self, p: Problem):
        self.q = np.asarray(p.q, dtype=np.float64)
        self.k0 = np.asarray(p.r0.k, dtype=np.float64)
        self.v0 = np.asarray(p.r0.v, dtype=np.float64)
        if p.r1 is not None:
            self.k1 = np.asarray(p.r1.k, dtype=np.float64)
            self.v1 = np.asarray(p.r1.v, dtype=np.float64)
        self.scale = float(np.float32(p.scale))


def _token(p: Problem, w: _Widened, b: int, t: int, want_probs: bool):
    rows0, rows1 = visible_rows(p, b, t)
    _, _, h, d = p.shape
    keys = [w.k0[b, rows0]]
    vals = [w.v0[b, rows0]]
    if len(rows1):
        keys.append(w.k1[b, rows1])
        vals.append(w.v1[b, rows1])
    kmat = np.concatenate(keys, axis=0)  # [A, D]
    vmat = np.concatenate(vals, axis=0)
    if kmat.shape[0] == 0:
        out = np.zeros((h, d), dtype=np.float64)
        return (out, np.zeros((h, 0)), rows0, rows1) if want_probs else out
    s = w.scale * (w.q[b, t] @ kmat.T)            # [H, A] scores
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    probs = e / e.sum(axis=1, keepdims=True)       # softmax over the visible keys
    out = probs @ vmat                              # [H, D]
    return (out, probs, rows0, rows1) if want_probs else out


def attention(p: Problem, tokens=None) -> np.ndarray:
    """O = softmax(scale * Q K^T + mask) V in float64.

    With ``tokens=None`` returns [B, T, H, D]; otherwise ``tokens`` is a list of
    (b, t) pairs and the result is [len(tokens), H, D].
    """
    w = _Widened(p)
    bsz, tn, h, d = p.shape
    if tokens is None:
        out = np.zeros((bsz, tn, h, d), dtype=np.float64)
        for b in range(bsz):
            for t in range(tn):
                out[b, t] = _token(p, w, b, t, False)
        return out
    return np.stack([_token(p, w, b, t, False) for (b, t) in tokens]) if tokens else \
        np.zeros((0, h, d))


def attention_probs(p: Problem, b: int, t: int):
    """(O, P, rows0, rows1) for one token: P is [H, A] over the visible keys in
    the order rows0 then rows1 (for the invariant checks on tiny inputs)."""
    return _token(p, _Widened(p), b, t, True)


# --------------------------------------------------------------------------- padded layout

def pad_layout(k: np.ndarray, v: np.ndarray, valid: Optional[np.ndarray], n_rows: int):
    """The 32-row padded layout of one region, bit for bit.

    Rows [0, n_rows) are copied unchanged; rows [n_rows, ceil32(n_rows)) are
    +0.0 in K and V (every bit zero) and invalid (0) in the validity bytes.
    Rows are copied as raw bits, so the element dtype is kept.
    """
    bsz, _, d = k.shape
    npad = ceil32(n_rows)
    kp = np.zeros((bsz, npad, d), dtype=k.dtype)
    vp = np.zeros((bsz, npad, d), dtype=v.dtype)
    kp[:, :n_rows] = k[:, :n_rows]
    vp[:, :n_rows] = v[:, :n_rows]
    validp = np.zeros((bsz, npad), dtype=np.uint8)
    if valid is None:
        validp[:, :n_rows] = 1
    else:
        validp[:, :n_rows] = np.asarray(valid)[:, :n_rows].astype(np.uint8)
    return kp, vp, validp


# --------------------------------------------------------------------------- block map

def dense_blocks(p: Problem):
    """(blocks of region 0, blocks of region 1 covered by the map).

    Region 1 is in the map only when it is not indexed (indexed rows are
    gathered per token, so there is no shared block to skip)."""
    nb0 = ceil32(p.r0.n_rows) // ROWS_PER_BLOCK
    nb1 = 0
    if p.r1 is not None and p.r1_index is None:
        nb1 = ceil32(p.r1.n_rows) // ROWS_PER_BLOCK
    return nb0, nb1


def allowed_matrix(p: Problem, b: int) -> np.ndarray:
    """Boolean [T, 32*(nb0+nb1)]: token t may see padded row column c."""
    _, tn, _, _ = p.shape
    nb0, nb1 = dense_blocks(p)
    cols0 = np.arange(nb0 * ROWS_PER_BLOCK, dtype=np.int64)
    a0 = np.stack([region0_allowed(p, b, t, cols0) for t in range(tn)]) if tn else \
        np.zeros((0, cols0.size), dtype=bool)
    if nb1 == 0:
        return a0
    cols1 = np.arange(nb1 * ROWS_PER_BLOCK, dtype=np.int64)
    vis1 = cols1 < p.r1.n_rows
    if p.r1.valid is not None:
        inside = cols1[vis1]
        v1 = np.zeros(cols1.shape, dtype=bool)
        v1[inside] = np.asarray(p.r1.valid)[b, inside] != 0
        vis1 &= v1
    a1 = np.broadcast_to(vis1, (tn, cols1.size))
    return np.concatenate([a0, a1], axis=1)


def blockmap(p: Problem, bq: int) -> np.ndarray:
    """Status byte per (sequence, query tile of ``bq`` tokens, 32-row KV block).

    The literal count of allowed (token, row) pairs in the tile x block:
    0 pairs -> SKIP (0), all pairs -> FULL (2), otherwise PARTIAL (1).
    """
    bsz, tn, _, _ = p.shape
    nb0, nb1 = dense_blocks(p)
    nb = nb0 + nb1
    ntiles = -(-tn // bq)
    out = np.zeros((bsz, ntiles, nb), dtype=np.uint8)
    for b in range(bsz):
        a = allowed_matrix(p, b)
        for qt in range(ntiles):
            rows = a[qt * bq: min(tn, (qt + 1) * bq)]
            for jb in range(nb):
                blk = rows[:, jb * ROWS_PER_BLOCK:(jb + 1) * ROWS_PER_BLOCK]
                count = int(blk.sum())
                if count == 0:
                    out[b, qt, jb] = SKIP
                elif count == blk.size:
                    out[b, qt, jb] = FULL
                else:
                    out[b, qt, jb] = PARTIAL
    return out


# --------------------------------------------------------------------------- adapter

def from_workload(w, logical_ring: bool = True) -> Problem:
    """Build a ``Problem`` from a seeded workload object (duck-typed: any object
    with ``q``, ``scale``, ``r0``, ``r1``, ``r1_index``, ``window``, ``q_pos0``,
    ``k_pos0``).  Ring regions are given to the oracle in logical order when
    ``logical_ring`` is set, so that the GPU (physical order) and the oracle see
    the same keys in a different order."""

    def region(r):
        if r is None:
            return None
        if logical_ring:
            k, v, valid = r.logical()
        else:
            k, v, valid = r.k, r.v, r.valid
        return Region(k.numpy(), v.numpy(), int(r.n_rows),
                      None if valid is None else valid.numpy())

    idx = None if w.r1_index is None else w.r1_index.numpy()
    return Problem(q=w.q.numpy(), scale=float(w.scale), r0=region(w.r0), window=int(w.window),
                   q_pos0=int(w.q_pos0), k_pos0=int(w.k_pos0), r1=region(w.r1), r1_index=idx)
