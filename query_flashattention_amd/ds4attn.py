"""Python binding of libds4attn (ctypes): argument marshalling only.

The functions keep the C names (``ds4attn_pad``, ``ds4attn_blockmap``,
``ds4attn_decode``, ``ds4attn_prefill``, ...).  Tensors are PyTorch tensors on
the GPU: the binding reads their data pointers, byte strides and torch's
current HIP stream and passes them through; every step of the computation runs
in the library's HIP kernels.  There is no fallback: if the library is not
built, or a call returns an error, a ``RuntimeError`` is raised.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libds4attn.so")

OK, E_INVAL, E_UNSUPPORTED, E_WORKSPACE, E_HIP = 0, 1, 2, 3, 4
F16, F32, E4M3 = 0, 1, 2
KV_PLAIN, KV_FP8_E4M3 = 0, 1
BLK_SKIP, BLK_PARTIAL, BLK_FULL = 0, 1, 2
FLAG_GENERIC = 1
FLAG_DECODE_DIMS = 2
FLAG_DECODE_KEYS = 4
FLAG_DECODE_WIDE = 8

_c_void_p = ctypes.c_void_p
_i32, _i64 = ctypes.c_int32, ctypes.c_int64


class Region(ctypes.Structure):
    _fields_ = [("k", _c_void_p), ("v", _c_void_p), ("valid", _c_void_p),
                ("k_scale", _c_void_p), ("v_scale", _c_void_p),
                ("stride_b", _i64), ("stride_row", _i64), ("valid_stride_b", _i64),
                ("scale_stride_b", _i64), ("n_rows", _i32), ("reserved", _i32)]


class Args(ctypes.Structure):
    _fields_ = [("batch", _i32), ("n_tok", _i32), ("n_head", _i32), ("head_dim", _i32),
                ("dtype", _i32), ("flags", _i32),
                ("q_stride_b", _i64), ("q_stride_t", _i64), ("q_stride_h", _i64),
                ("o_stride_b", _i64), ("o_stride_t", _i64), ("o_stride_h", _i64),
                ("scale", ctypes.c_float), ("window", _i32),
                ("q_pos0", _i64), ("k_pos0", _i64),
                ("r0", Region), ("r1", Region),
                ("r1_index", _c_void_p), ("r1_k", _i32), ("kv_format", _i32)]


EXPORTS = ("ds4attn_pad", "ds4attn_blockmap", "ds4attn_blockmap_dims", "ds4attn_decode",
           "ds4attn_prefill", "ds4attn_workspace_bytes", "ds4attn_decode_noalloc", "ds4attn_prefill_bq",
           "ds4attn_topk",
           "ds4attn_quantize_fp8", "ds4attn_decode_split", "ds4attn_decode_workspace_bytes",
           "ds4attn_compress", "ds4attn_status_string")

_lib = None


def lib() -> ctypes.CDLL:
    """Load libds4attn.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python __graft_entry__.py build)")
        h = ctypes.CDLL(LIB_PATH)
        h.ds4attn_pad.argtypes = [ctypes.POINTER(Region), _i32, _i32, _i32, _c_void_p, _c_void_p,
                                  _i64, _i64, _c_void_p, _i64, _c_void_p]
        h.ds4attn_blockmap.argtypes = [ctypes.POINTER(Args), _i32, _c_void_p, _c_void_p]
        h.ds4attn_blockmap_dims.argtypes = [ctypes.POINTER(Args), _i32, ctypes.POINTER(_i64),
                                            ctypes.POINTER(_i32)]
        for name in ("ds4attn_decode", "ds4attn_prefill"):
            getattr(h, name).argtypes = [ctypes.POINTER(Args), _c_void_p, _c_void_p, _i32,
                                         _c_void_p, _c_void_p, _i64, _c_void_p]
        h.ds4attn_workspace_bytes.argtypes = [ctypes.POINTER(Args), _i32, ctypes.POINTER(_i64)]
        h.ds4attn_decode_noalloc.argtypes = [ctypes.POINTER(Args), _c_void_p, _c_void_p, _i32, _c_void_p,
                                             _c_void_p]
        h.ds4attn_topk.argtypes = [_c_void_p, _i64, _i32, _i64, _i32, _c_void_p, _i64, _c_void_p]
        h.ds4attn_decode_split.argtypes = [ctypes.POINTER(Args), _c_void_p, _c_void_p, _i32, _c_void_p,
                                           _i32, _c_void_p, _i64, _c_void_p]
        h.ds4attn_decode_workspace_bytes.argtypes = [ctypes.POINTER(Args), _i32, ctypes.POINTER(_i64)]
        h.ds4attn_quantize_fp8.argtypes = [_c_void_p, _i32, _i32, _i32, _i32, _i64, _i64, _c_void_p,
                                           _i64, _i64, _c_void_p, _i64, _c_void_p]
        h.ds4attn_compress.argtypes = [_i32, _i32, _i32, _i32, _i32, _c_void_p, _i64, _c_void_p, _i64,
                                       _c_void_p, _i64, _c_void_p, _i64, _c_void_p, _i64, _c_void_p]
        for name in EXPORTS[:-1]:
            getattr(h, name).restype = _i32
        h.ds4attn_status_string.argtypes = [_i32]
        h.ds4attn_status_string.restype = ctypes.c_char_p
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().ds4attn_status_string(status).decode()


def _check(status: int, what: str):
    if status != OK:
        raise RuntimeError(f"{what} failed: {status_string(status)} ({status})")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float16:
        return F16
    if dt == torch.float32:
        return F32
    if dt == torch.uint8:      # E4M3 codes
        return E4M3
    raise ValueError(f"unsupported element type {dt}")


# --------------------------------------------------------------------------- marshalling

def region(k: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None, n_rows: int = 0,
           valid: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
           v_scale: Optional[torch.Tensor] = None) -> Region:
    """A ``Region`` over [B, N, D] K/V tensors (rows contiguous) and optional uint8 [B, N]
    validity; for FP8 rows, K/V are uint8 codes and k_scale/v_scale float32 [B, >= N]."""
    r = Region()
    if k_scale is not None:
        if v_scale is None or v_scale.stride(0) != k_scale.stride(0) or k_scale.dtype != torch.float32:
            raise ValueError("FP8 regions take float32 K and V scales with one batch stride")
        r.k_scale, r.v_scale = k_scale.data_ptr(), v_scale.data_ptr()
        r.scale_stride_b = k_scale.stride(0) * 4
    r.n_rows = int(n_rows)
    if k is not None:
        es = k.element_size()
        r.k, r.v = k.data_ptr(), v.data_ptr()
        r.stride_b, r.stride_row = k.stride(0) * es, k.stride(1) * es
        if v.stride() != k.stride():
            raise ValueError("K and V of one region must share strides")
    if valid is not None:
        r.valid = valid.data_ptr()
        r.valid_stride_b = valid.stride(0)
    return r


def args(q: torch.Tensor, o: Optional[torch.Tensor], r0: Region, r1: Optional[Region] = None,
         r1_index: Optional[torch.Tensor] = None, scale: float = None, window: int = 0,
         q_pos0: int = 0, k_pos0: int = 0, flags: int = 0, kv_format: int = KV_PLAIN) -> Args:
    """``Args`` for q [B, T, H, D] and float32 o [B, T, H, D] (o may be None for a map)."""
    a = Args()
    a.kv_format = kv_format
    b, t, h, d = q.shape
    a.batch, a.n_tok, a.n_head, a.head_dim = b, t, h, d
    a.dtype = _dtype_code(q.dtype)
    a.flags = flags
    es = q.element_size()
    a.q_stride_b, a.q_stride_t, a.q_stride_h = (s * es for s in q.stride()[:3])
    if o is not None:
        a.o_stride_b, a.o_stride_t, a.o_stride_h = (s * 4 for s in o.stride()[:3])
    a.scale = float(scale) if scale is not None else 1.0 / d ** 0.5
    a.window, a.q_pos0, a.k_pos0 = int(window), int(q_pos0), int(k_pos0)
    a.r0 = r0
    a.r1 = r1 if r1 is not None else Region()
    if r1_index is not None:
        a.r1_index = r1_index.data_ptr()
        a.r1_k = r1_index.shape[-1]
    return a


# --------------------------------------------------------------------------- entry points

def ds4attn_pad(reg: Region, batch: int, head_dim: int, dtype: int, k_pad: torch.Tensor,
                v_pad: torch.Tensor, valid_pad: Optional[torch.Tensor] = None, stream=None) -> None:
    es = k_pad.element_size()
    _check(lib().ds4attn_pad(ctypes.byref(reg), batch, head_dim, dtype, k_pad.data_ptr(),
                             v_pad.data_ptr(), k_pad.stride(0) * es, k_pad.stride(1) * es,
                             _ptr(valid_pad), 0 if valid_pad is None else valid_pad.stride(0),
                             _stream(stream)), "ds4attn_pad")


def ds4attn_blockmap_dims(a: Args, bq: int):
    nt, nb = _i64(), _i32()
    _check(lib().ds4attn_blockmap_dims(ctypes.byref(a), bq, ctypes.byref(nt), ctypes.byref(nb)),
           "ds4attn_blockmap_dims")
    return int(nt.value), int(nb.value)


def ds4attn_blockmap(a: Args, bq: int, blk: Optional[torch.Tensor], stream=None) -> None:
    _check(lib().ds4attn_blockmap(ctypes.byref(a), bq, _ptr(blk), _stream(stream)), "ds4attn_blockmap")


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def ds4attn_decode(a: Args, q: torch.Tensor, blk: Optional[torch.Tensor], bq: int, o: torch.Tensor,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Decode; ``workspace`` (a device tensor of ``ds4attn_workspace_bytes(a, 0)``
    bytes) lets the library split small batches over more workgroups; None runs
    unsplit."""
    _check(lib().ds4attn_decode(ctypes.byref(a), q.data_ptr(), _ptr(blk), bq, o.data_ptr(),
                                _ptr(workspace), _nbytes(workspace), _stream(stream)), "ds4attn_decode")


def ds4attn_prefill(a: Args, q: torch.Tensor, blk: Optional[torch.Tensor], bq: int, o: torch.Tensor,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    _check(lib().ds4attn_prefill(ctypes.byref(a), q.data_ptr(), _ptr(blk), bq, o.data_ptr(),
                                 _ptr(workspace), _nbytes(workspace), _stream(stream)), "ds4attn_prefill")


def ds4attn_decode_noalloc(a: Args, q: torch.Tensor, blk: Optional[torch.Tensor], bq: int, o: torch.Tensor,
                           stream=None) -> None:
    """Decode with the split's scratch in the library's static per-device array
    (no allocation anywhere); calls that overlap in time on one device race."""
    _check(lib().ds4attn_decode_noalloc(ctypes.byref(a), q.data_ptr(), _ptr(blk), bq, o.data_ptr(),
                                        _stream(stream)), "ds4attn_decode_noalloc")


def ds4attn_workspace_bytes(a: Args, is_prefill: bool) -> int:
    n = _i64()
    _check(lib().ds4attn_workspace_bytes(ctypes.byref(a), int(bool(is_prefill)), ctypes.byref(n)),
           "ds4attn_workspace_bytes")
    return int(n.value)


def ds4attn_decode_workspace_bytes(a: Args, splits: int) -> int:
    n = _i64()
    _check(lib().ds4attn_decode_workspace_bytes(ctypes.byref(a), splits, ctypes.byref(n)),
           "ds4attn_decode_workspace_bytes")
    return int(n.value)


def ds4attn_decode_split(a: Args, q: torch.Tensor, blk: Optional[torch.Tensor], bq: int, o: torch.Tensor,
                         splits: int, workspace: Optional[torch.Tensor], stream=None) -> None:
    _check(lib().ds4attn_decode_split(ctypes.byref(a), q.data_ptr(), _ptr(blk), bq, o.data_ptr(), splits,
                                      _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "ds4attn_decode_split")


def ds4attn_topk(scores: torch.Tensor, k: int, idx: torch.Tensor, stream=None) -> None:
    """Top-k index selection: scores float32 [rows, n] (rows contiguous), idx int32 [rows, k]."""
    if scores.dtype != torch.float32 or idx.dtype != torch.int32:
        raise TypeError("ds4attn_topk takes float32 scores and an int32 output")
    rows, n = scores.shape
    if (n > 1 and scores.stride(1) != 1) or (k > 1 and idx.stride(1) != 1) or idx.shape != (rows, k):
        raise ValueError("ds4attn_topk needs rows with unit element stride and idx of shape [rows, k]")
    _check(lib().ds4attn_topk(scores.data_ptr() if n else None, rows, n, scores.stride(0) * 4, k,
                              idx.data_ptr(), idx.stride(0) * 4, _stream(stream)), "ds4attn_topk")


def topk(scores: torch.Tensor, k: int, stream=None) -> torch.Tensor:
    """Allocate the output and run ``ds4attn_topk``."""
    idx = torch.empty((scores.shape[0], k), dtype=torch.int32, device=scores.device)
    ds4attn_topk(scores, k, idx, stream)
    return idx


def ds4attn_quantize_fp8(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, n_rows: int = None,
                         stream=None) -> None:
    """FP8 quantize step: x [B, N, D] float16/float32 rows -> uint8 codes [B, N, D] and
    float32 scales [B, N] (rows contiguous along D)."""
    b, n, d = x.shape
    n = n if n_rows is None else int(n_rows)
    if codes.dtype != torch.uint8 or scales.dtype != torch.float32:
        raise TypeError("ds4attn_quantize_fp8 writes uint8 codes and float32 scales")
    if x.stride(2) != 1 or codes.stride(2) != 1 or (n > 1 and scales.stride(1) != 1):
        raise ValueError("rows must be contiguous along the head dimension")
    es = x.element_size()
    _check(lib().ds4attn_quantize_fp8(x.data_ptr(), _dtype_code(x.dtype), b, n, d, x.stride(0) * es,
                                      x.stride(1) * es, codes.data_ptr(), codes.stride(0),
                                      codes.stride(1), scales.data_ptr(), scales.stride(0) * 4,
                                      _stream(stream)), "ds4attn_quantize_fp8")


def quantize_fp8(x: torch.Tensor, stream=None):
    """Allocate (codes, scales) and run ``ds4attn_quantize_fp8``."""
    b, n, d = x.shape
    codes = torch.empty((b, n, d), dtype=torch.uint8, device=x.device)
    scales = torch.empty((b, n), dtype=torch.float32, device=x.device)
    ds4attn_quantize_fp8(x, codes, scales, stream=stream)
    return codes, scales


def ds4attn_compress(state_kv: torch.Tensor, state_score: torch.Tensor, n_state: int, kv_new: torch.Tensor,
                     score_new: torch.Tensor, ratio: int, comp: Optional[torch.Tensor], stream=None) -> int:
    """Compressor step: state_kv [B, ratio, D] float16 and state_score [B, ratio, D]
    float32 (rows [0, n_state) pending, updated in place), new rows kv_new [B, n, D]
    float16 and score_new [B, n, D] float32 -> comp [B, >= n_out, D] float16 (rows
    0 .. n_out - 1 written).  Returns n_out = (n_state + n) // ratio; the new state
    count is (n_state + n) % ratio."""
    b, n, d = kv_new.shape
    if state_kv.dtype != torch.float16 or kv_new.dtype != torch.float16 or \
            state_score.dtype != torch.float32 or score_new.dtype != torch.float32:
        raise TypeError("ds4attn_compress takes float16 rows and float32 scores")
    if comp is not None and comp.dtype != torch.float16:
        raise TypeError("ds4attn_compress writes float16 rows")
    for t in (state_kv, state_score, kv_new, score_new) + ((comp,) if comp is not None else ()):
        if t.dim() != 3 or t.shape[0] != b or t.shape[2] != d or t.stride(2) != 1 or \
                (t.shape[1] > 1 and t.stride(1) != d):
            raise ValueError("ds4attn_compress needs [B, rows, D] tensors with packed rows")
    if state_kv.shape[1] < ratio or state_score.shape[1] < ratio:
        raise ValueError("the state buffers hold ratio rows")
    n_out = (n_state + n) // ratio
    if n_out and (comp is None or comp.shape[1] < n_out):
        raise ValueError("comp holds fewer than n_out rows")
    _check(lib().ds4attn_compress(b, d, ratio, n_state, n, state_kv.data_ptr(), state_kv.stride(0) * 2,
                                  state_score.data_ptr(), state_score.stride(0) * 4, kv_new.data_ptr(),
                                  kv_new.stride(0) * 2, score_new.data_ptr(), score_new.stride(0) * 4,
                                  _ptr(comp), comp.stride(0) * 2 if comp is not None else 0,
                                  _stream(stream)), "ds4attn_compress")
    return n_out


def ds4attn_prefill_bq() -> int:
    return int(lib().ds4attn_prefill_bq())


# --------------------------------------------------------------------------- the three stages on GPU tensors

def pad_region(k: torch.Tensor, v: torch.Tensor, n_rows: int, valid: Optional[torch.Tensor] = None,
               stream=None):
    """Stage 1: new padded K/V [B, ceil32(n), D] and validity [B, ceil32(n)] on k's device."""
    b, _, d = k.shape
    npad = -(-n_rows // 32) * 32
    kp = torch.empty((b, npad, d), dtype=k.dtype, device=k.device)
    vp = torch.empty((b, npad, d), dtype=v.dtype, device=v.device)
    vap = torch.empty((b, npad), dtype=torch.uint8, device=k.device)
    ds4attn_pad(region(k, v, n_rows, valid), b, d, _dtype_code(k.dtype), kp, vp, vap, stream)
    return kp, vp, vap


def blockmap(a: Args, bq: int, device, stream=None) -> torch.Tensor:
    """Stage 2: the uint8 skip map [B, ceil(T/bq), nb]."""
    nt, nb = ds4attn_blockmap_dims(a, bq)
    blk = torch.empty((a.batch, nt, nb), dtype=torch.uint8, device=device)
    ds4attn_blockmap(a, bq, blk if blk.numel() else None, stream)
    return blk
