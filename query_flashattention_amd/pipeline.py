"""The three stages of the attention step on device-resident inputs.

``to_device`` places a seeded workload in GPU memory the way an engine holds its
KV cache: each region in a buffer with capacity for whole 32-row blocks, the
tail rows not yet initialised ([P-Metal] "KV-Cache Management on Metal Device
Buffers").  ``step`` then runs pad (in place) -> block map -> fused attention,
all in libds4attn's kernels on torch's current stream ([P-Metal]
"FlashAttention Kernel Architecture": pad, blk and impl kernels).

[P-Metal] = the page "How DeepSeek V4 Flash Model Inference Works on Apple
Silicon with Metal Backend".
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import ds4attn as da


def _ceil32(n: int) -> int:
    return -(-n // 32) * 32


@dataclass
class DeviceRegion:
    k: torch.Tensor              # [B, ceil32(n), D] storage, rows >= n uninitialised until padded
    v: torch.Tensor
    n_rows: int
    valid: Optional[torch.Tensor]      # [B, ceil32(n)] uint8 storage: the caller's bytes in
                                       # [0, n), the tail uninitialised until padded; or None
    k_scale: Optional[torch.Tensor] = None   # FP8 rows: float32 [B, n] row scales
    v_scale: Optional[torch.Tensor] = None

    def region(self) -> da.Region:
        return da.region(self.k, self.v, self.n_rows, self.valid, self.k_scale, self.v_scale)

    def pad_in_place(self, stream=None):
        """Stage 1 in place: zero the tail rows and tail validity bytes (nothing is
        launched when the region already fills whole blocks)."""
        b, _, d = self.k.shape
        da.ds4attn_pad(self.region(), b, d, da._dtype_code(self.k.dtype), self.k, self.v, self.valid,
                       stream)


@dataclass
class DeviceProblem:
    q: torch.Tensor
    o: torch.Tensor
    r0: DeviceRegion
    r1: Optional[DeviceRegion]
    idx: Optional[torch.Tensor]
    scale: float
    window: int
    q_pos0: int
    k_pos0: int
    flags: int = 0

    def args(self) -> da.Args:
        fmt = da.KV_FP8_E4M3 if self.r0.k.dtype == torch.uint8 else da.KV_PLAIN
        return da.args(self.q, self.o, self.r0.region(), None if self.r1 is None else self.r1.region(),
                       self.idx, self.scale, self.window, self.q_pos0, self.k_pos0, self.flags, fmt)


def _region_to_device(r, device) -> Optional[DeviceRegion]:
    if r is None:
        return None
    b, n, d = r.k.shape
    cap = _ceil32(r.n_rows)
    k = torch.empty((b, cap, d), dtype=r.k.dtype, device=device)
    v = torch.empty((b, cap, d), dtype=r.v.dtype, device=device)
    k[:, :r.n_rows].copy_(r.k[:, :r.n_rows])
    v[:, :r.n_rows].copy_(r.v[:, :r.n_rows])
    valid = None
    if r.valid is not None:
        valid = torch.empty((b, cap), dtype=torch.uint8, device=device)
        valid[:, :r.n_rows].copy_(r.valid[:, :r.n_rows])
    ks = vs = None
    if getattr(r, "k_scale", None) is not None:
        ks = r.k_scale[:, :r.n_rows].contiguous().to(device)
        vs = r.v_scale[:, :r.n_rows].contiguous().to(device)
    return DeviceRegion(k, v, r.n_rows, valid, ks, vs)


def to_device(w, device="cuda") -> DeviceProblem:
    """Copy a seeded workload to the GPU (physical ring order, unpadded tails)."""
    q = w.q.to(device)
    o = torch.empty(q.shape, dtype=torch.float32, device=device)
    idx = None if w.r1_index is None else w.r1_index.contiguous().to(device)
    return DeviceProblem(q, o, _region_to_device(w.r0, device), _region_to_device(w.r1, device), idx,
                         w.scale, w.window, w.q_pos0, w.k_pos0)


def step(dp: DeviceProblem, entry: str = "decode", bq: int = 1, blk: Optional[torch.Tensor] = None,
         stream=None, splits: Optional[int] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One pass of the hot path: pad (in place) -> block map -> fused attention.

    ``blk`` may be a preallocated map buffer of the right size; the output is
    ``dp.o`` (float32 [B, T, H, D]).  ``splits``: None = the library's own plan for
    the call (``ds4attn_workspace_bytes``; its workspace is allocated here when
    ``workspace`` is omitted), 1 = unsplit, > 1 = decode with each token's blocks
    divided over that many workgroups (``ds4attn_decode_split``)."""
    dp.r0.pad_in_place(stream)
    if dp.r1 is not None:
        dp.r1.pad_in_place(stream)
    a = dp.args()
    if blk is None:
        blk = da.blockmap(a, bq, dp.q.device, stream)
    else:
        da.ds4attn_blockmap(a, bq, blk if blk.numel() else None, stream)
    mp = blk if blk.numel() else None
    if entry == "decode" and splits is not None and splits > 1:
        if workspace is None:
            nbytes = da.ds4attn_decode_workspace_bytes(a, splits)
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dp.q.device)
        da.ds4attn_decode_split(a, dp.q, mp, bq, dp.o, splits, workspace, stream)
        return dp.o
    prefill = entry != "decode"
    if splits is None and workspace is None:
        nbytes = da.ds4attn_workspace_bytes(a, prefill)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dp.q.device)
    if splits == 1:
        workspace = None
    fn = da.ds4attn_prefill if prefill else da.ds4attn_decode
    fn(a, dp.q, mp, bq, dp.o, workspace, stream)
    return dp.o
