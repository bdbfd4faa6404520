"""Pure-Python brute force of the same attention step (test infrastructure only).

A second, independent formulation used to pin ``oracle.reference`` on tiny
inputs: no NumPy arithmetic, an explicit additive mask of 0.0 / -inf over the
full key list of each token (all region-0 rows, then every region-1 candidate),
scores by nested loops, softmax with ``math.exp``.  It follows the same pages:
fused Q.K^T / softmax / PV with -inf on masked pairs ([P-Metal] "FlashAttention
Kernel Architecture", "Mask Handling and Block Skipping"); raw window rows plus
compressed rows, all of them or an index-selected subset ([P-DS4] "Architecture
Deep Dive": Layer Compression, KV Cache Design, GPU Backend Architecture).
"""

from __future__ import annotations

import math
import struct

NEG_INF = float("-inf")


def _f(x):
    return float(x)


def _as_float32(x):
    """The scale travels as a 32-bit float; round it the way a C float would."""
    return struct.unpack("<f", struct.pack("<f", float(x)))[0]


def _keys_for_token(p, b, t):
    """List of (key vector, value vector, additive mask) over every candidate key."""
    keys = []
    n0 = p.r0.n_rows
    k0 = p.r0.k[b].tolist()
    v0 = p.r0.v[b].tolist()
    valid0 = None if p.r0.valid is None else p.r0.valid[b].tolist()
    qpos = p.q_pos0 + t
    for j in range(n0):
        bias = 0.0
        if valid0 is not None and not valid0[j]:
            bias = NEG_INF
        if p.window > 0:
            kpos = p.k_pos0 + j
            if kpos > qpos or qpos - kpos > p.window - 1:
                bias = NEG_INF
        keys.append((k0[j], v0[j], bias))
    if p.r1 is not None and p.r1.n_rows > 0:
        n1 = p.r1.n_rows
        k1 = p.r1.k[b].tolist()
        v1 = p.r1.v[b].tolist()
        valid1 = None if p.r1.valid is None else p.r1.valid[b].tolist()
        if p.r1_index is None:
            cands = list(range(n1))
        else:
            cands = [int(c) for c in p.r1_index[b][t].tolist()]
        for c in cands:
            if c < 0 or c >= n1:
                continue  # unused index entry
            bias = 0.0
            if valid1 is not None and not valid1[c]:
                bias = NEG_INF
            keys.append((k1[c], v1[c], bias))
    return keys


def attention_token(p, b, t):
    """[H][D] nested lists: output of token t of sequence b."""
    scale = _as_float32(p.scale)
    qb = p.q[b][t].tolist()
    keys = _keys_for_token(p, b, t)
    out = []
    for qh in qb:
        scores = []
        for kvec, _, bias in keys:
            acc = 0.0
            for qd, kd in zip(qh, kvec):
                acc += _f(qd) * _f(kd)
            scores.append(scale * acc + bias)
        finite = [s for s in scores if s != NEG_INF]
        dim = len(qh)
        if not finite:
            out.append([0.0] * dim)
            continue
        mx = max(finite)
        weights = [math.exp(s - mx) if s != NEG_INF else 0.0 for s in scores]
        total = math.fsum(weights)
        row = []
        for d in range(dim):
            row.append(math.fsum(wt * _f(kv[1][d]) for wt, kv in zip(weights, keys)) / total)
        out.append(row)
    return out


def attention(p):
    """[B][T][H][D] nested lists."""
    bsz, tn = p.q.shape[0], p.q.shape[1]
    return [[attention_token(p, b, t) for t in range(tn)] for b in range(bsz)]


def blockmap(p, bq):
    """Status bytes by materialising every (token, padded row) pair of the dense
    regions and counting, with the brute-force mask above."""
    bsz, tn = p.q.shape[0], p.q.shape[1]
    n0 = p.r0.n_rows
    nb0 = (n0 + 31) // 32
    cols = [("r0", j) for j in range(nb0 * 32)]
    if p.r1 is not None and p.r1_index is None:
        nb1 = (p.r1.n_rows + 31) // 32
        cols += [("r1", c) for c in range(nb1 * 32)]
    nb = len(cols) // 32
    ntiles = (tn + bq - 1) // bq
    res = []
    for b in range(bsz):
        valid0 = None if p.r0.valid is None else p.r0.valid[b].tolist()
        valid1 = None
        if p.r1 is not None and p.r1.valid is not None:
            valid1 = p.r1.valid[b].tolist()
        seq = []
        for qt in range(ntiles):
            toks = list(range(qt * bq, min(tn, (qt + 1) * bq)))
            row = []
            for jb in range(nb):
                count = 0
                for t in toks:
                    for which, j in cols[jb * 32:(jb + 1) * 32]:
                        if which == "r0":
                            ok = j < n0 and (valid0 is None or valid0[j])
                            if ok and p.window > 0:
                                kpos, qpos = p.k_pos0 + j, p.q_pos0 + t
                                ok = kpos <= qpos and qpos - kpos <= p.window - 1
                        else:
                            ok = j < p.r1.n_rows and (valid1 is None or valid1[j])
                        count += 1 if ok else 0
                total = len(toks) * 32
                row.append(0 if count == 0 else (2 if count == total else 1))
            seq.append(row)
        res.append(seq)
    return res
