"""Seeded synthetic inputs for the attention step (no attention arithmetic here).

This module only draws random numbers and arranges them; it is shared by the
tests, the benchmark and the oracle-side checks, and it holds none of the
method's arithmetic.  Every tensor is made on the CPU from a
``torch.Generator`` seeded per workload, in a fixed draw order: Q, K0, V0, K1,
V1 (float32 ``randn``, then rounded to float16 unless the workload is float32),
then the integers (ring offsets, compressed-row counts, index lists).

Shapes follow the pages: 64 query heads sharing one KV head of dimension 512
with a 128-token sliding window ([P-DS4] "Architecture Deep Dive", Fixed Model
Shape), raw rows kept in a 128-row ring and compressed rows pooled every 4 or
128 tokens, with the top-512 indexer on ratio-4 layers ([P-DS4] "Architecture
Deep Dive", Layer Compression and KV Cache Design), and prefill in 2048-token
chunks ([P-DS4] "Architecture Deep Dive", Whole-Model Graph Execution).

[P-DS4] = the page "DwarfStar 4 (DS4) -- DeepSeek V4 Flash Inference Engine".
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

N_HEAD = 64          # query heads sharing the one KV head
HEAD_DIM = 512
WINDOW = 128         # raw sliding-window rows
TOPK = 512           # indexer top-k on ratio-4 layers
PREFILL_CHUNK = 2048


def scale_for(head_dim: int) -> float:
    """The float32 value of 1/sqrt(head_dim), returned as a Python float."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


@dataclass
class RegionInputs:
    """One KV region as the GPU sees it.

    ``k``/``v`` are [B, N, D] with N >= ``n_rows`` (physical row order);
    ``valid`` is uint8 [B, N] or None.  For a ring, ``ring_offset[b]`` is the
    physical slot of logical row 0: logical row j lives at (offset + j) mod N.
    """

    k: torch.Tensor
    v: torch.Tensor
    n_rows: int
    valid: Optional[torch.Tensor] = None
    ring_offset: Optional[torch.Tensor] = None
    k_scale: Optional[torch.Tensor] = None   # FP8 rows: k/v are uint8 E4M3 codes and these
    v_scale: Optional[torch.Tensor] = None   # are float32 [B, N] row scales

    def _ring_index(self):
        n = self.k.shape[1]
        j = torch.arange(n)
        return (self.ring_offset.view(-1, 1) + j.view(1, -1)) % n       # [B, N]

    def logical(self):
        """(k, v, valid) in logical ring order (identity when not a ring)."""
        if self.ring_offset is None:
            return self.k, self.v, self.valid
        idx = self._ring_index()
        gather = idx.unsqueeze(-1).expand(-1, -1, self.k.shape[2])
        k = torch.gather(self.k, 1, gather)
        v = torch.gather(self.v, 1, gather)
        valid = None if self.valid is None else torch.gather(self.valid, 1, idx)
        return k, v, valid

    def logical_scales(self):
        """(k_scale, v_scale) in logical ring order (FP8 rows)."""
        if self.ring_offset is None or self.k_scale is None:
            return self.k_scale, self.v_scale
        idx = self._ring_index()
        return torch.gather(self.k_scale, 1, idx), torch.gather(self.v_scale, 1, idx)


@dataclass
class Workload:
    name: str
    seed: int
    q: torch.Tensor                      # [B, T, H, D]
    scale: float
    r0: RegionInputs
    window: int = 0
    q_pos0: int = 0
    k_pos0: int = 0
    r1: Optional[RegionInputs] = None
    r1_index: Optional[torch.Tensor] = None   # int32 [B, T, k]
    notes: dict = field(default_factory=dict)

    @property
    def dims(self):
        b, t, h, d = self.q.shape
        return b, t, h, d

    @property
    def dtype(self) -> str:
        return {torch.float16: "f16", torch.float32: "f32"}[self.q.dtype]


def _normal(g, shape, dtype, std=1.0):
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def _ring_physical(logical: torch.Tensor, offset: torch.Tensor) -> torch.Tensor:
    """Place logical row j of sequence b at physical slot (offset[b] + j) mod N."""
    bsz, n, d = logical.shape
    phys = torch.empty_like(logical)
    j = torch.arange(n)
    for b in range(bsz):
        phys[b, (int(offset[b]) + j) % n] = logical[b]
    return phys


def tiny_mqa(seed: int = 101) -> Workload:
    """1 token, 4 query heads, head dim 64, 27 valid KV rows (padded to 32), float32."""
    g = torch.Generator().manual_seed(seed)
    q = _normal(g, (1, 1, 4, 64), torch.float32)
    k = _normal(g, (1, 27, 64), torch.float32)
    v = _normal(g, (1, 27, 64), torch.float32)
    return Workload("tiny_mqa_h4_d64_n27", seed, q, 0.125, RegionInputs(k, v, 27))


def decode_raw_swa(seed: int = 102, batch: int = 64) -> Workload:
    """Decode on a raw sliding-window layer: 1 token x 64 heads x d512 per sequence,
    a full 128-row ring per sequence with its write pointer at a seeded slot."""
    g = torch.Generator().manual_seed(seed)
    q = _normal(g, (batch, 1, N_HEAD, HEAD_DIM), torch.float16, std=0.5)
    k = _normal(g, (batch, WINDOW, HEAD_DIM), torch.float16)
    v = _normal(g, (batch, WINDOW, HEAD_DIM), torch.float16)
    off = torch.randint(0, WINDOW, (batch,), generator=g)
    r0 = RegionInputs(_ring_physical(k, off), _ring_physical(v, off), WINDOW, ring_offset=off)
    return Workload(f"decode_raw_swa_b{batch}_n128", seed, q, scale_for(HEAD_DIM), r0)


def decode_ratio128(seed: int = 103, batch: int = 1, context: int = 32768) -> Workload:
    """Decode on a ratio-128 layer at a 32K context: 128 raw ring rows plus
    context/128 = 256 compressed slots, the last compressed block partly valid."""
    g = torch.Generator().manual_seed(seed)
    n1 = context // 128
    q = _normal(g, (batch, 1, N_HEAD, HEAD_DIM), torch.float16)
    k0 = _normal(g, (batch, WINDOW, HEAD_DIM), torch.float16)
    v0 = _normal(g, (batch, WINDOW, HEAD_DIM), torch.float16)
    k1 = _normal(g, (batch, n1, HEAD_DIM), torch.float16)
    v1 = _normal(g, (batch, n1, HEAD_DIM), torch.float16)
    off = torch.randint(0, WINDOW, (batch,), generator=g)
    short = torch.randint(1, 32, (batch,), generator=g)        # r ~ U{1..31}
    n_comp = n1 - short
    valid1 = (torch.arange(n1).view(1, -1) < n_comp.view(-1, 1)).to(torch.uint8)
    r0 = RegionInputs(_ring_physical(k0, off), _ring_physical(v0, off), WINDOW, ring_offset=off)
    r1 = RegionInputs(k1, v1, n1, valid=valid1)
    return Workload(f"decode_ratio128_b{batch}_n128+{n1}", seed, q, scale_for(HEAD_DIM), r0,
                    r1=r1, notes={"n_comp": n_comp.tolist()})


def decode_ratio4(seed: int = 106, batch: int = 64, context: int = 8192,
                  topk: int = TOPK) -> Workload:
    """Decode on a ratio-4 indexed layer: per sequence a full 128-row raw ring plus
    context/4 compressed rows pooling positions [0, context), of which the token
    attends a sorted, unique, uniform top-``topk`` index list."""
    g = torch.Generator().manual_seed(seed)
    n1 = context // 4
    q = _normal(g, (batch, 1, N_HEAD, HEAD_DIM), torch.float16)
    k0 = _normal(g, (batch, WINDOW, HEAD_DIM), torch.float16)
    v0 = _normal(g, (batch, WINDOW, HEAD_DIM), torch.float16)
    k1 = _normal(g, (batch, n1, HEAD_DIM), torch.float16)
    v1 = _normal(g, (batch, n1, HEAD_DIM), torch.float16)
    off = torch.randint(0, WINDOW, (batch,), generator=g)
    keys = torch.rand(batch, n1, generator=g)
    idx = keys.argsort(dim=1)[:, :topk].sort(dim=1).values.to(torch.int32)
    r0 = RegionInputs(_ring_physical(k0, off), _ring_physical(v0, off), WINDOW, ring_offset=off)
    return Workload(f"decode_ratio4_b{batch}_n128+{topk}of{n1}", seed, q, scale_for(HEAD_DIM), r0,
                    r1=RegionInputs(k1, v1, n1), r1_index=idx.view(batch, 1, topk))


def prefill_raw_swa(seed: int = 104, tokens: int = PREFILL_CHUNK) -> Workload:
    """Prefill chunk on a raw layer: causal + 128-token sliding window over the chunk."""
    g = torch.Generator().manual_seed(seed)
    q = _normal(g, (1, tokens, N_HEAD, HEAD_DIM), torch.float16)
    k = _normal(g, (1, tokens, HEAD_DIM), torch.float16)
    v = _normal(g, (1, tokens, HEAD_DIM), torch.float16)
    return Workload(f"prefill_raw_swa_t{tokens}", seed, q, scale_for(HEAD_DIM),
                    RegionInputs(k, v, tokens), window=WINDOW, q_pos0=0, k_pos0=0)


def prefill_ratio4(seed: int = 105, tokens: int = PREFILL_CHUNK, start: int = 30720,
                   topk: int = TOPK) -> Workload:
    """Prefill chunk on a ratio-4 indexed layer starting at position ``start``.

    Raw region: the 127 rows before the chunk plus the chunk's own rows.
    Compressed region: start/4 rows pooling positions [0, start), all causally
    visible to every query of the chunk; each query draws a sorted, unique,
    uniform top-``topk`` index list.
    """
    g = torch.Generator().manual_seed(seed)
    n0 = (WINDOW - 1) + tokens
    n1 = start // 4
    q = _normal(g, (1, tokens, N_HEAD, HEAD_DIM), torch.float16)
    k0 = _normal(g, (1, n0, HEAD_DIM), torch.float16)
    v0 = _normal(g, (1, n0, HEAD_DIM), torch.float16)
    k1 = _normal(g, (1, n1, HEAD_DIM), torch.float16)
    v1 = _normal(g, (1, n1, HEAD_DIM), torch.float16)
    keys = torch.rand(tokens, n1, generator=g)
    idx = keys.argsort(dim=1)[:, :topk].sort(dim=1).values.to(torch.int32)
    return Workload(f"prefill_ratio4_t{tokens}_at{start}", seed, q, scale_for(HEAD_DIM),
                    RegionInputs(k0, v0, n0), window=WINDOW, q_pos0=start,
                    k_pos0=start - (WINDOW - 1), r1=RegionInputs(k1, v1, n1),
                    r1_index=idx.view(1, tokens, topk))


def _fp8_rows(g, shape):
    """E4M3 codes (uint8, sign and magnitude code drawn uniformly over the finite
    codes up to 224, subnormals included) and float32 row scales near 2^-7."""
    mag = torch.randint(0, 0x77, shape, generator=g, dtype=torch.int32)
    sign = torch.randint(0, 2, shape, generator=g, dtype=torch.int32) * 0x80
    codes = (mag + sign).to(torch.uint8)
    scales = torch.exp2(torch.rand(shape[:-1], generator=g) - 7.5).to(torch.float32)
    return codes, scales


def fp8_variant(w: Workload, seed: int) -> Workload:
    """The same workload (Q, structure, validity, rings, index lists) with its K/V
    rows drawn as FP8 codes and per-row scales from generator ``seed`` (in the
    order K0, V0, K1, V1)."""
    g = torch.Generator().manual_seed(seed)

    def conv(r):
        if r is None:
            return None
        kc, ks = _fp8_rows(g, tuple(r.k.shape))
        vc, vs = _fp8_rows(g, tuple(r.v.shape))
        return RegionInputs(kc, vc, r.n_rows, r.valid, r.ring_offset, ks, vs)

    r0, r1 = conv(w.r0), conv(w.r1)
    return Workload(w.name + "_fp8", seed, w.q, w.scale, r0, window=w.window, q_pos0=w.q_pos0,
                    k_pos0=w.k_pos0, r1=r1, r1_index=w.r1_index, notes=dict(w.notes, kv="fp8_e4m3"))


def named(name: str) -> Workload:
    """The five reference workloads, the batched ratio-128 decode variant and the
    ratio-4 indexed decode."""
    table = {
        "tiny": tiny_mqa,
        "decode_swa": decode_raw_swa,
        "decode_r128": decode_ratio128,
        "decode_r128_b64": lambda: decode_ratio128(batch=64),
        "decode_r4": decode_ratio4,
        "prefill_swa": prefill_raw_swa,
        "prefill_r4": prefill_ratio4,
        # FP8 rows (E4M3 codes, per-row scales) on the same structures
        "decode_swa_fp8": lambda: fp8_variant(decode_raw_swa(), 107),
        "decode_r4_fp8": lambda: fp8_variant(decode_ratio4(), 108),
        "decode_r128_fp8": lambda: fp8_variant(decode_ratio128(batch=64), 109),
        "prefill_r4_fp8": lambda: fp8_variant(prefill_ratio4(), 110),
    }
    return table[name]()


def random_problem(seed: int, batch: int, tokens: int, heads: int, head_dim: int,
                   dtype: torch.dtype = torch.float16, n0: int = 64,
                   valid0_frac: Optional[float] = None, window: int = 0,
                   q_pos0: int = 0, k_pos0: int = 0, n1: int = 0,
                   r1_mode: str = "none", valid1_frac: Optional[float] = None,
                   r1_k: int = 0, idx_invalid_frac: float = 0.0,
                   q_std: float = 1.0) -> Workload:
    """A general seeded problem for parity tests (ragged sizes, every mask kind).

    ``r1_mode``: "none" (no region 1), "all" (every row visible under the
    optional validity mask) or "index" (``r1_k`` entries per token, sorted,
    unique, with ``idx_invalid_frac`` of them replaced by -1).
    """
    g = torch.Generator().manual_seed(seed)
    q = _normal(g, (batch, tokens, heads, head_dim), dtype, std=q_std)
    k0 = _normal(g, (batch, n0, head_dim), dtype)
    v0 = _normal(g, (batch, n0, head_dim), dtype)
    valid0 = None
    r1 = None
    idx = None
    if r1_mode != "none":
        k1 = _normal(g, (batch, n1, head_dim), dtype)
        v1 = _normal(g, (batch, n1, head_dim), dtype)
    if valid0_frac is not None:
        valid0 = (torch.rand(batch, n0, generator=g) < valid0_frac).to(torch.uint8)
    if r1_mode != "none":
        valid1 = None
        if valid1_frac is not None:
            valid1 = (torch.rand(batch, n1, generator=g) < valid1_frac).to(torch.uint8)
        r1 = RegionInputs(k1, v1, n1, valid=valid1)
        if r1_mode == "index":
            keys = torch.rand(batch * tokens, max(n1, 1), generator=g)
            take = min(r1_k, n1)
            sel = keys.argsort(dim=1)[:, :take].sort(dim=1).values.to(torch.int32)
            full = torch.full((batch * tokens, r1_k), -1, dtype=torch.int32)
            full[:, :take] = sel
            if idx_invalid_frac > 0:
                drop = torch.rand(batch * tokens, r1_k, generator=g) < idx_invalid_frac
                full[drop] = -1
            idx = full.view(batch, tokens, r1_k)
    return Workload(f"random_s{seed}", seed, q, scale_for(head_dim),
                    RegionInputs(k0, v0, n0, valid=valid0), window=window, q_pos0=q_pos0,
                    k_pos0=k_pos0, r1=r1, r1_index=idx)


def indexer_scores(seed: int, rows: int, n: int, kind: str = "normal") -> torch.Tensor:
    """float32 [rows, n] scores for the top-k selection step (the indexer that
    produces them is learned and not on the pages, so the values are drawn).

    ``normal``: standard normal.  ``coarse``: multiples of 1/4 in [-2, 2], so that
    most selections end inside a run of equal scores.  ``special``: normal with
    about one entry in eight replaced by +0, -0, +inf, -inf or a NaN of either sign.
    """
    g = torch.Generator().manual_seed(seed)
    if kind == "normal":
        return torch.randn(rows, n, generator=g)
    if kind == "coarse":
        return torch.randint(-8, 9, (rows, n), generator=g).float() * 0.25
    if kind == "special":
        s = torch.randn(rows, n, generator=g)
        pick = torch.randint(0, 8, (rows, n), generator=g) == 0
        which = torch.randint(0, 6, (rows, n), generator=g)
        bits = torch.tensor([0x00000000, 0x80000000 - (1 << 32), 0x7F800000, 0xFF800000 - (1 << 32),
                             0x7FC00001, 0xFFC00001 - (1 << 32)], dtype=torch.int32)
        special = bits[which].view(torch.float32)
        return torch.where(pick, special, s)
    raise ValueError(f"unknown score kind {kind!r}")


@dataclass
class CompressInputs:
    """One compressor call's inputs: the rolling state (ratio rows, the first
    n_state pending) and the new raw rows, with a score per element."""
    ratio: int
    n_state: int
    state_kv: torch.Tensor      # float16 [B, ratio, D]
    state_score: torch.Tensor   # float32 [B, ratio, D]
    kv_new: torch.Tensor        # float16 [B, n_new, D]
    score_new: torch.Tensor     # float32 [B, n_new, D]


def compress_inputs(seed: int, batch: int, ratio: int, n_state: int, n_new: int,
                    head_dim: int = HEAD_DIM, score_std: float = 1.0) -> CompressInputs:
    """Seeded compressor inputs (the learned score projection is not on the pages,
    so scores are drawn).  Draw order: state rows, state scores, new rows, new
    scores; rows N(0, 1) rounded to float16, scores N(0, score_std) float32.  State
    rows past n_state are drawn too (the step must neither read nor keep them)."""
    g = torch.Generator().manual_seed(seed)
    st_kv = _normal(g, (batch, ratio, head_dim), torch.float16)
    st_sc = _normal(g, (batch, ratio, head_dim), torch.float32, score_std)
    kv = _normal(g, (batch, n_new, head_dim), torch.float16)
    sc = _normal(g, (batch, n_new, head_dim), torch.float32, score_std)
    return CompressInputs(ratio, n_state, st_kv, st_sc, kv, sc)
