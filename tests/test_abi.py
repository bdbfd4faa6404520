"""Host-side checks of the C ABI (no GPU needed; no kernel is launched).

* the built library loads and exports every function include/ds4attn.h declares;
* the ctypes structures have the C layout (checked against gcc's offsetof/sizeof);
* argument checks return their status codes before anything would be enqueued.
"""

import ctypes
import os
import re
import subprocess
import sys

import pytest

from query_flashattention_amd import ds4attn as da

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ds4attn.h")
FAKE = 0x7F0000000000  # an aligned address that is never dereferenced on the host


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|const char \*)\s*(ds4attn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 7
    lib = da.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ds4attn.h but not exported"
    assert set(names) == set(da.EXPORTS)


def test_struct_layout_matches_c_header(tmp_path):
    fields = {
        "ds4attn_region": [f[0] for f in da.Region._fields_],
        "ds4attn_args": [f[0] for f in da.Args._fields_],
    }
    lines = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void){"]
    for st, names in fields.items():
        lines.append(f'printf("{st} size %zu\\n", sizeof({st}));')
        for n in names:
            lines.append(f'printf("{st} {n} %zu\\n", offsetof({st}, {n}));')
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-o", str(exe), str(src)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    c = {}
    for line in out:
        if line:
            st, key, val = line.split()
            c[(st, key)] = int(val)
    for st, cls in (("ds4attn_region", da.Region), ("ds4attn_args", da.Args)):
        assert c[(st, "size")] == ctypes.sizeof(cls)
        for n in fields[st]:
            assert c[(st, n)] == getattr(cls, n).offset, (st, n)


def _good_args(head_dim=512, dtype=da.F16, heads=64):
    a = da.Args()
    es = 2 if dtype == da.F16 else 4
    a.batch, a.n_tok, a.n_head, a.head_dim, a.dtype = 1, 1, heads, head_dim, dtype
    a.q_stride_h = head_dim * es
    a.q_stride_t = heads * head_dim * es
    a.q_stride_b = a.q_stride_t
    a.o_stride_h = head_dim * 4
    a.o_stride_t = heads * head_dim * 4
    a.o_stride_b = a.o_stride_t
    a.scale = 0.044194173
    a.r0.k = a.r0.v = FAKE
    a.r0.n_rows = 128
    a.r0.stride_row = head_dim * es
    a.r0.stride_b = 128 * head_dim * es
    return a


def _decode(a, q=FAKE, o=FAKE, blk=None, bq=1, ws=None, ws_bytes=0):
    return da.lib().ds4attn_decode(ctypes.byref(a), q, blk, bq, o, ws, ws_bytes, None)


@pytest.mark.parametrize("mutate,expect", [
    (lambda a: setattr(a, "head_dim", 96), da.E_UNSUPPORTED),
    (lambda a: setattr(a, "head_dim", 0), da.E_INVAL),
    (lambda a: setattr(a, "dtype", 7), da.E_INVAL),
    (lambda a: setattr(a, "n_head", 0), da.E_INVAL),
    (lambda a: setattr(a, "n_tok", -1), da.E_INVAL),
    (lambda a: setattr(a, "window", -3), da.E_INVAL),
    (lambda a: setattr(a, "scale", float("nan")), da.E_INVAL),
    (lambda a: setattr(a, "q_stride_h", 1000), da.E_INVAL),          # not a multiple of 16
    (lambda a: setattr(a, "q_stride_h", 512), da.E_INVAL),           # rows overlap
    (lambda a: setattr(a.r0, "stride_row", 8), da.E_INVAL),
    (lambda a: setattr(a.r0, "k", FAKE + 8), da.E_INVAL),            # misaligned
    (lambda a: setattr(a.r0, "v", None), da.E_INVAL),
    (lambda a: setattr(a.r0, "n_rows", -1), da.E_INVAL),
    (lambda a: (setattr(a, "r1_index", FAKE), setattr(a, "r1_k", 4097)), da.E_INVAL),
    (lambda a: (setattr(a, "r1_index", FAKE), setattr(a, "r1_k", 0)), da.E_INVAL),
])
def test_decode_rejects_bad_arguments(mutate, expect):
    a = _good_args()
    mutate(a)
    assert _decode(a) == expect


def test_null_pointers_and_tile_size():
    lib = da.lib()
    assert lib.ds4attn_decode(None, FAKE, None, 1, FAKE, None, 0, None) == da.E_INVAL
    a = _good_args()
    assert _decode(a, q=None) == da.E_INVAL
    assert _decode(a, o=FAKE + 4) == da.E_INVAL
    assert _decode(a, blk=FAKE, bq=0) == da.E_INVAL
    assert lib.ds4attn_blockmap(ctypes.byref(a), 0, FAKE, None) == da.E_INVAL
    assert lib.ds4attn_blockmap(None, 1, FAKE, None) == da.E_INVAL
    assert lib.ds4attn_blockmap(ctypes.byref(a), 1, None, None) == da.E_INVAL


def test_empty_problems_succeed_without_launch():
    a = _good_args()
    a.batch = 0
    assert _decode(a, q=None, o=None) == da.OK
    a = _good_args()
    a.n_tok = 0
    assert da.lib().ds4attn_prefill(ctypes.byref(a), None, None, 16, None, None, 0, None) == da.OK
    assert da.lib().ds4attn_blockmap(ctypes.byref(a), 16, None, None) == da.OK


def test_blockmap_dims():
    a = _good_args()
    a.n_tok = 2048
    a.r0.n_rows = 2175
    assert da.ds4attn_blockmap_dims(a, 16) == (128, 68)
    a.r1.n_rows = 256
    assert da.ds4attn_blockmap_dims(a, 1) == (2048, 68 + 8)
    a.r1_index = FAKE
    a.r1_k = 512
    assert da.ds4attn_blockmap_dims(a, 1) == (2048, 68)   # indexed rows are not mapped


def test_pad_rejects_bad_arguments():
    lib = da.lib()
    r = da.Region()
    r.k = r.v = FAKE
    r.n_rows, r.stride_row, r.stride_b = 27, 256, 27 * 256
    out = FAKE + (1 << 30)
    assert lib.ds4attn_pad(ctypes.byref(r), 1, 64, da.F32, out, out + (1 << 20), 32 * 256 + 16, 8,
                           None, 0, None) == da.E_INVAL          # output row stride too small
    assert lib.ds4attn_pad(ctypes.byref(r), 1, 64, 5, out, out + (1 << 20), 0, 256, None, 0,
                           None) == da.E_INVAL                   # dtype
    # outputs overlapping the inputs without being the same buffer
    assert lib.ds4attn_pad(ctypes.byref(r), 1, 64, da.F32, FAKE + 256, out, 32 * 256, 256, None, 0,
                           None) == da.E_INVAL
    # K and V outputs sharing a buffer while the inputs differ
    r.v = FAKE + (1 << 24)
    assert lib.ds4attn_pad(ctypes.byref(r), 1, 64, da.F32, out, out, 32 * 256, 256, None, 0,
                           None) == da.E_INVAL
    # a V output overlapping the K input (K and V inputs distinct), and the mirror case
    r.v = FAKE + (1 << 24)
    assert lib.ds4attn_pad(ctypes.byref(r), 1, 64, da.F32, out, FAKE + 512, 32 * 256, 256, None, 0,
                           None) == da.E_INVAL
    assert lib.ds4attn_pad(ctypes.byref(r), 1, 64, da.F32, r.v + 512, out, 32 * 256, 256, None, 0,
                           None) == da.E_INVAL
    r.v = FAKE
    r0 = da.Region()
    assert lib.ds4attn_pad(ctypes.byref(r0), 1, 64, da.F32, None, None, 0, 0, None, 0, None) == da.OK
    # validity output overlapping the validity input without being it
    r.v = r.k
    r.valid, r.valid_stride_b = FAKE + (1 << 28), 64
    assert lib.ds4attn_pad(ctypes.byref(r), 2, 64, da.F32, out, out, 32 * 256 * 2, 256,
                           r.valid + 1, 64, None) == da.E_INVAL


def test_pad_with_nothing_to_write_launches_nothing():
    """A region that already fills whole blocks, padded in place (K, V and validity
    outputs are their inputs): no kernel is needed, so this succeeds without a GPU."""
    lib = da.lib()
    r = da.Region()
    r.k, r.v = FAKE, FAKE + (1 << 24)
    r.n_rows, r.stride_row, r.stride_b = 64, 256, 64 * 256
    r.valid, r.valid_stride_b = FAKE + (1 << 28), 64
    assert lib.ds4attn_pad(ctypes.byref(r), 3, 64, da.F32, r.k, r.v, r.stride_b, r.stride_row,
                           r.valid, r.valid_stride_b, None) == da.OK
    assert lib.ds4attn_pad(ctypes.byref(r), 3, 64, da.F32, r.k, r.v, r.stride_b, r.stride_row,
                           None, 0, None) == da.OK


def test_topk_rejects_bad_arguments():
    lib = da.lib()
    out = FAKE + (1 << 30)
    # k outside 1..2048, negative sizes
    assert lib.ds4attn_topk(FAKE, 4, 100, 400, 0, out, 4, None) == da.E_INVAL
    assert lib.ds4attn_topk(FAKE, 4, 100, 400, 2049, out, 2049 * 4, None) == da.E_INVAL
    assert lib.ds4attn_topk(FAKE, -1, 100, 400, 8, out, 32, None) == da.E_INVAL
    assert lib.ds4attn_topk(FAKE, 4, -1, 400, 8, out, 32, None) == da.E_INVAL
    # misaligned pointers or strides, strides shorter than a row
    assert lib.ds4attn_topk(FAKE + 2, 4, 100, 400, 8, out, 32, None) == da.E_INVAL
    assert lib.ds4attn_topk(FAKE, 4, 100, 400, 8, out + 1, 32, None) == da.E_INVAL
    assert lib.ds4attn_topk(FAKE, 4, 100, 402, 8, out, 32, None) == da.E_INVAL
    assert lib.ds4attn_topk(FAKE, 4, 100, 396, 8, out, 32, None) == da.E_INVAL
    assert lib.ds4attn_topk(FAKE, 4, 100, 400, 8, out, 28, None) == da.E_INVAL
    # null buffers; output overlapping the scores
    assert lib.ds4attn_topk(None, 4, 100, 400, 8, out, 32, None) == da.E_INVAL
    assert lib.ds4attn_topk(FAKE, 4, 100, 400, 8, None, 32, None) == da.E_INVAL
    assert lib.ds4attn_topk(FAKE, 4, 100, 400, 8, FAKE + 1200, 32, None) == da.E_INVAL
    # more rows than one launch takes
    assert lib.ds4attn_topk(FAKE, (1 << 24) + 1, 100, 400, 8, out, 32, None) == da.E_UNSUPPORTED
    assert lib.ds4attn_topk(FAKE, 1, 1 << 30, 0, 8, out, 32, None) == da.E_UNSUPPORTED
    # no rows: nothing to launch
    assert lib.ds4attn_topk(FAKE, 0, 100, 400, 8, out, 32, None) == da.OK


def _fp8_args(**kw):
    a = _good_args(**kw)
    a.kv_format = da.KV_FP8_E4M3
    a.r0.stride_row = 512
    a.r0.stride_b = 128 * 512
    a.r0.k_scale = a.r0.v_scale = FAKE + (1 << 24)
    a.r0.scale_stride_b = 4 * 128
    return a


@pytest.mark.parametrize("mutate,expect", [
    (lambda a: setattr(a, "kv_format", 5), da.E_INVAL),
    (lambda a: setattr(a.r0, "k_scale", None), da.E_INVAL),
    (lambda a: setattr(a.r0, "v_scale", FAKE + 2), da.E_INVAL),          # misaligned
    (lambda a: setattr(a.r0, "scale_stride_b", 6), da.E_INVAL),
    (lambda a: (setattr(a, "batch", 2), setattr(a.r0, "scale_stride_b", 4 * 127)), da.E_INVAL),
    (lambda a: setattr(a.r0, "stride_row", 496), da.E_INVAL),            # shorter than a row
    (lambda a: setattr(a, "n_head", 8), da.E_UNSUPPORTED),               # no matrix-core kernel
    (lambda a: setattr(a, "flags", da.FLAG_GENERIC), da.E_UNSUPPORTED),
])
def test_fp8_attention_rejects_bad_arguments(mutate, expect):
    a = _fp8_args()
    mutate(a)
    assert _decode(a) == expect


def test_fp8_attention_needs_float16_queries():
    assert _decode(_fp8_args(dtype=da.F32)) == da.E_UNSUPPORTED


def test_fp8_attention_with_empty_regions_needs_no_scales():
    a = _fp8_args()
    a.batch = 0
    a.r0.k_scale = None
    assert _decode(a, q=None, o=None) == da.OK


def test_quantize_rejects_bad_arguments():
    lib = da.lib()
    x, c, s = FAKE, FAKE + (1 << 26), FAKE + (1 << 27)

    def q(**kw):
        p = dict(x=x, dtype=da.F16, batch=2, n=10, d=512, xsb=10 * 1024, xsr=1024, c=c, csb=10 * 512,
                 csr=512, s=s, ssb=40)
        p.update(kw)
        return lib.ds4attn_quantize_fp8(p["x"], p["dtype"], p["batch"], p["n"], p["d"], p["xsb"],
                                        p["xsr"], p["c"], p["csb"], p["csr"], p["s"], p["ssb"], None)

    assert q(dtype=da.E4M3) == da.E_INVAL
    assert q(d=96) == da.E_UNSUPPORTED
    assert q(d=-1) == da.E_INVAL
    assert q(batch=-1) == da.E_INVAL
    assert q(x=FAKE + 8) == da.E_INVAL
    assert q(s=s + 2) == da.E_INVAL
    assert q(xsr=1000) == da.E_INVAL
    assert q(xsr=512) == da.E_INVAL                  # rows overlap
    assert q(csr=496) == da.E_INVAL
    assert q(ssb=36) == da.E_INVAL                   # fewer scales than rows
    assert q(c=x + 4096) == da.E_INVAL               # codes overlap the input
    assert q(s=c + 64) == da.E_INVAL                 # scales overlap the codes
    assert q(x=None) == da.E_INVAL
    assert q(n=0) == da.OK                           # nothing to do, nothing launched
    assert q(batch=0, x=None, c=None, s=None) == da.OK


def test_compress_rejects_bad_arguments():
    lib = da.lib()
    d = 512
    st_kv, st_sc, kv, sc, comp = (FAKE, FAKE + (1 << 26), FAKE + (2 << 26), FAKE + (3 << 26), FAKE + (4 << 26))

    def c(**kw):
        p = dict(batch=2, d=d, ratio=4, n_state=3, n_new=10, st_kv=st_kv, st_kv_sb=4 * 2 * d, st_sc=st_sc,
                 st_sc_sb=4 * 4 * d, kv=kv, kv_sb=10 * 2 * d, sc=sc, sc_sb=10 * 4 * d, comp=comp,
                 comp_sb=3 * 2 * d)
        p.update(kw)
        return lib.ds4attn_compress(p["batch"], p["d"], p["ratio"], p["n_state"], p["n_new"], p["st_kv"],
                                    p["st_kv_sb"], p["st_sc"], p["st_sc_sb"], p["kv"], p["kv_sb"], p["sc"],
                                    p["sc_sb"], p["comp"], p["comp_sb"], None)

    assert c(ratio=0) == da.E_INVAL
    assert c(n_state=4) == da.E_INVAL                # the state holds fewer than ratio rows
    assert c(n_state=-1) == da.E_INVAL
    assert c(n_new=-1) == da.E_INVAL
    assert c(d=96) == da.E_UNSUPPORTED
    assert c(ratio=2048, n_state=0) == da.E_UNSUPPORTED
    assert c(st_kv=st_kv + 8) == da.E_INVAL          # alignment
    assert c(kv_sb=10 * 2 * d - 16) == da.E_INVAL    # sequences' new rows overlap
    assert c(st_sc_sb=3 * 4 * d) == da.E_INVAL       # a state shorter than ratio rows
    assert c(comp_sb=2 * 2 * d) == da.E_INVAL        # fewer than n_out = 3 compressed rows
    assert c(comp=None) == da.E_INVAL                # n_out > 0 needs an output
    assert c(comp=kv + 64) == da.E_INVAL             # output overlaps an input
    assert c(st_kv=kv + 1024) == da.E_INVAL          # state overlaps the new rows
    assert c(st_sc=st_kv + 16) == da.E_INVAL         # the two state buffers overlap
    assert c(n_new=0) == da.OK                       # nothing to do, nothing launched
    assert c(batch=0) == da.OK


def test_pad_accepts_fp8_rows():
    """E4M3 rows are 1-byte elements: a 512-dim row is 512 bytes; a region that
    fills whole blocks in place launches nothing."""
    lib = da.lib()
    r = da.Region()
    r.k, r.v = FAKE, FAKE + (1 << 24)
    r.n_rows, r.stride_row, r.stride_b = 64, 512, 64 * 512
    assert lib.ds4attn_pad(ctypes.byref(r), 2, 512, da.E4M3, r.k, r.v, r.stride_b, r.stride_row,
                           None, 0, None) == da.OK
    assert lib.ds4attn_pad(ctypes.byref(r), 2, 512, 3, r.k, r.v, r.stride_b, r.stride_row,
                           None, 0, None) == da.E_INVAL


def test_split_decode_rejects_bad_arguments():
    lib = da.lib()
    a = _good_args()
    need = da.ds4attn_decode_workspace_bytes(a, 4)
    assert need == 1 * 1 * 4 * 4 * (16 * 512 * 4 + 128)
    assert da.ds4attn_decode_workspace_bytes(a, 1) == 0
    ws = FAKE + (1 << 32)

    def split(aa, splits, w=ws, nbytes=need, q=FAKE, o=FAKE):
        return lib.ds4attn_decode_split(ctypes.byref(aa), q, None, 1, o, splits, w, nbytes, None)

    assert split(a, 0) == da.E_INVAL
    assert split(a, 65) == da.E_INVAL
    assert split(a, 4, w=None) == da.E_INVAL
    assert split(a, 4, nbytes=need - 1) == da.E_WORKSPACE
    assert split(a, 4, w=ws + 8) == da.E_INVAL                   # misaligned
    assert split(a, 4, w=FAKE) == da.E_INVAL                     # overlaps o
    g = _good_args(heads=8)                                      # no matrix-core kernel
    assert split(g, 4) == da.E_UNSUPPORTED
    b = _good_args()
    b.flags = da.FLAG_GENERIC
    assert split(b, 4) == da.E_UNSUPPORTED
    e = _good_args()
    e.batch = 0
    assert split(e, 4, w=None, nbytes=0, q=None, o=None) == da.OK   # nothing to do
    n = ctypes.c_int64()
    assert lib.ds4attn_decode_workspace_bytes(ctypes.byref(_good_args(heads=8)), 2, ctypes.byref(n)) == \
        da.E_UNSUPPORTED
    assert lib.ds4attn_decode_workspace_bytes(ctypes.byref(a), 0, ctypes.byref(n)) == da.E_INVAL


def test_status_strings_and_tile():
    assert da.status_string(da.OK) == "ok"
    assert "invalid" in da.status_string(da.E_INVAL)
    assert da.ds4attn_prefill_bq() >= 1


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """The Python side has no fallback path: a missing library is an error."""
    code = ("import query_flashattention_amd.ds4attn as d; d.LIB_PATH='/nonexistent/libds4attn.so';"
            "\ntry:\n d.lib()\nexcept RuntimeError as e:\n print('raised', e)")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert "raised" in out.stdout


def _prefill(a, q=FAKE, o=FAKE, blk=None, bq=1):
    return da.lib().ds4attn_prefill(ctypes.byref(a), q, blk, bq, o, None, 0, None)


@pytest.mark.parametrize("flags,fp8,entry,expect", [
    (da.FLAG_DECODE_DIMS | da.FLAG_DECODE_KEYS, False, "decode", da.E_INVAL),
    (da.FLAG_DECODE_KEYS | da.FLAG_GENERIC, False, "decode", da.E_UNSUPPORTED),
    (da.FLAG_DECODE_DIMS | da.FLAG_GENERIC, False, "decode", da.E_UNSUPPORTED),
    (da.FLAG_DECODE_DIMS, False, "prefill", da.E_UNSUPPORTED),           # 64-head prefill kernel
])
def test_decode_split_flags_rejected(flags, fp8, entry, expect):
    a = _fp8_args() if fp8 else _good_args()
    a.flags = flags
    assert (_decode(a) if entry == "decode" else _prefill(a)) == expect


def test_decode_split_flags_need_the_matrix_core_kernel():
    a = _good_args(head_dim=128)
    a.flags = da.FLAG_DECODE_KEYS
    assert _decode(a) == da.E_UNSUPPORTED


@pytest.mark.parametrize("flags,expect", [
    (da.FLAG_DECODE_WIDE | da.FLAG_DECODE_DIMS, da.E_INVAL),
    (da.FLAG_DECODE_WIDE | da.FLAG_DECODE_KEYS, da.E_INVAL),
    (da.FLAG_DECODE_WIDE | da.FLAG_GENERIC, da.E_UNSUPPORTED),
])
def test_wide_decode_flag_rejected(flags, expect):
    a = _good_args()
    a.flags = flags
    assert _decode(a) == expect


def test_wide_decode_needs_32_heads_and_no_index_list():
    a = _good_args(heads=48)
    a.flags = da.FLAG_DECODE_WIDE
    assert _decode(a) == da.E_UNSUPPORTED
    a = _good_args()
    a.flags = da.FLAG_DECODE_WIDE
    a.r1.k = a.r1.v = FAKE + (1 << 30)
    a.r1.n_rows = 256
    a.r1.stride_row = 1024
    a.r1.stride_b = 256 * 1024
    a.r1_index = FAKE
    a.r1_k = 64
    assert _decode(a) == da.E_UNSUPPORTED


def test_wide_decode_is_never_split():
    """A chosen wide split plans no parts (no workspace), and the split entry point
    refuses it before anything is enqueued."""
    lib = da.lib()
    a = _good_args()
    a.flags = da.FLAG_DECODE_WIDE
    assert da.ds4attn_workspace_bytes(a, False) == 0
    ws = FAKE + (1 << 32)
    need = 1 * 1 * 4 * 2 * (16 * 512 * 4 + 128)
    assert lib.ds4attn_decode_split(ctypes.byref(a), FAKE, None, 1, FAKE, 2, ws, need, None) == da.E_UNSUPPORTED


def _ratio128_args(batch=1):
    """One decode token of a ratio-128 layer at 32K: 128 raw rows + 256 compressed slots."""
    a = _good_args()
    a.batch = batch
    a.r1.k = a.r1.v = FAKE + (1 << 30)
    a.r1.n_rows = 256
    a.r1.stride_row = 1024
    a.r1.stride_b = 256 * 1024
    return a


def test_workspace_plan():
    """The library splits a decode batch that leaves most CUs idle: one sequence of
    the ratio-128 layer (4 groups of 16 heads, 12 key blocks) in 6 parts of two
    blocks; a 64-sequence batch, prefill, short lists and the vector-ALU kernel
    run unsplit."""
    rec = 16 * 512 * 4 + 128
    assert da.ds4attn_workspace_bytes(_ratio128_args(), False) == 4 * 6 * rec
    assert da.ds4attn_workspace_bytes(_ratio128_args(64), False) == 0
    assert da.ds4attn_workspace_bytes(_ratio128_args(), True) == 0
    assert da.ds4attn_workspace_bytes(_good_args(), False) == 0               # 4 blocks: too short to split
    assert da.ds4attn_workspace_bytes(_good_args(heads=8), False) == 0        # vector-ALU kernel
    g = _ratio128_args()
    g.flags = da.FLAG_GENERIC
    assert da.ds4attn_workspace_bytes(g, False) == 0
    w = _ratio128_args()
    w.window = 128
    w.r0.n_rows = 4096                      # 128-row window: at most 6 blocks reachable + 8
    assert da.ds4attn_workspace_bytes(w, False) == 4 * 7 * rec
    long = _ratio128_args()
    long.r0.n_rows = 4096                   # no window: 128 + 8 blocks, at most 8 parts
    assert da.ds4attn_workspace_bytes(long, False) == 4 * 8 * rec
    r4 = _ratio128_args()
    r4.r1.n_rows = 32 * 20 - 128            # 20 blocks: 8 parts would hold 3 blocks at most, as 7 do
    r4.r1.stride_b = r4.r1.n_rows * 1024
    assert da.ds4attn_workspace_bytes(r4, False) == 4 * 7 * rec
    e = _ratio128_args()
    e.batch = 0
    assert da.ds4attn_workspace_bytes(e, False) == 0
    lib = da.lib()
    n = ctypes.c_int64()
    assert lib.ds4attn_workspace_bytes(None, 0, ctypes.byref(n)) == da.E_INVAL
    assert lib.ds4attn_workspace_bytes(ctypes.byref(_ratio128_args()), 0, None) == da.E_INVAL
    bad = _ratio128_args()
    bad.head_dim = 96
    assert lib.ds4attn_workspace_bytes(ctypes.byref(bad), 0, ctypes.byref(n)) == da.E_UNSUPPORTED


def test_decode_workspace_checked_before_launch():
    a = _ratio128_args()
    need = da.ds4attn_workspace_bytes(a, False)
    ws = FAKE + (1 << 32)
    assert _decode(a, ws=ws, ws_bytes=need - 16) == da.E_WORKSPACE
    assert _decode(a, ws=ws + 8, ws_bytes=need) == da.E_INVAL      # misaligned
    assert _decode(a, ws=FAKE, ws_bytes=need) == da.E_INVAL        # overlaps o
    assert _decode(a, ws=ws, ws_bytes=-1) == da.E_INVAL


def test_tile_larger_than_the_chunk():
    """bq is clamped to the chunk: any bq >= n_tok is one tile (no 32-bit overflow)."""
    a = _good_args()
    a.n_tok = 2048
    assert da.ds4attn_blockmap_dims(a, 2 ** 31 - 1) == (1, 4)
    a.batch = 0
    assert _decode(a, q=None, o=None, blk=FAKE, bq=2 ** 31 - 1) == da.OK


def test_noalloc_decode_checks_before_launch():
    """The no-allocation decode entry point validates like ds4attn_decode before any
    HIP call; an empty problem succeeds without touching a device."""
    lib = da.lib()
    assert lib.ds4attn_decode_noalloc(None, FAKE, None, 1, FAKE, None) == da.E_INVAL
    a = _ratio128_args()
    a.head_dim = 96
    assert lib.ds4attn_decode_noalloc(ctypes.byref(a), FAKE, None, 1, FAKE, None) == da.E_UNSUPPORTED
    a = _ratio128_args()
    a.batch = 0
    assert lib.ds4attn_decode_noalloc(ctypes.byref(a), None, None, 1, None, None) == da.OK
