"""GPU parity cases built to expose single-row mistakes that the attention
tolerance alone (max-abs 1e-2, mean-abs 1e-3) could let through.

* Poisoned hidden rows: every K/V row that no token of its sequence may see
  (outside every window, hidden by validity, never named by an index list,
  region-1 row 0 that unused index entries read, the padding tail when the pad
  stage has not run) holds NaN, in float16 and in FP8 rows.  One leaked row makes
  the output non-finite.
* One-hot values: V rows are unit vectors, a distinct column per row a token
  sees, so O[h, c] is that row's softmax weight; a dropped row leaves an exact
  zero where the oracle has its weight (per-element bound in parity_util).
* Wrong speculative starts: the kernels fetch their first list entries from the
  window arithmetic before the block map arrives.  A window whose reach ends in
  one raw block followed by a dense region 1, and leading raw blocks that are all
  invalid, make those guesses wrong in every kernel (HEADS prefill, DIMS, wide DIMS
  and KEYS decode, split parts, FP8 rows), while the guessed rows hold NaN.
* A query tile longer than the chunk (bq = 2^31 - 1) is one tile.

Every case runs through the C ABI and is compared with the float64 oracle.
"""

import dataclasses
import zlib

import numpy as np
import pytest
import torch

from oracle import fp8 as ofp8
from oracle import reference as ref
from query_flashattention_amd import ds4attn as da
from query_flashattention_amd import pipeline, workloads as wl
from tests.parity_util import check_onehot, compare, free_row0, onehot_values, poison_hidden, poison_tail

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    da.lib()  # fail loudly if the HIP library is missing


MODES = {
    # mode: (entry, flags, splits)
    "prefill": ("prefill", 0, 1),
    "dims": ("decode", da.FLAG_DECODE_DIMS, 1),
    "keys": ("decode", da.FLAG_DECODE_KEYS, 1),
    "split3": ("decode", 0, 3),
    "plan": ("decode", 0, None),
    # DIMS over 32 heads per workgroup: no index lists
    "wide": ("decode", da.FLAG_DECODE_WIDE, 1),
}
KERNEL_MODES = ["prefill", "dims", "keys", "split3", "wide"]


def _indexed(kw):
    return kw.get("r1_mode") == "index"


def _run(w, mode, use_map=True, pad=True, bq=None):
    entry, flags, splits = MODES[mode]
    if bq is None:
        bq = da.ds4attn_prefill_bq() if entry == "prefill" else 1
    dp = pipeline.to_device(w, DEV)
    dp.flags = flags
    if pad:
        dp.r0.pad_in_place()
        if dp.r1 is not None:
            dp.r1.pad_in_place()
    else:
        poison_tail(dp)
    a = dp.args()
    blk = da.blockmap(a, bq, DEV) if use_map else None
    if blk is not None and blk.numel() == 0:
        blk = None
    if splits is not None and splits > 1:
        ws = torch.empty(da.ds4attn_decode_workspace_bytes(a, splits), dtype=torch.uint8, device=DEV)
        da.ds4attn_decode_split(a, dp.q, blk, bq, dp.o, splits, ws)
    else:
        fn = da.ds4attn_prefill if entry == "prefill" else da.ds4attn_decode
        ws = None
        if splits is None:
            n = da.ds4attn_workspace_bytes(a, entry == "prefill")
            ws = torch.empty(n, dtype=torch.uint8, device=DEV) if n else None
        fn(a, dp.q, blk, bq, dp.o, ws)
    torch.cuda.synchronize()
    return dp.o.cpu().double().numpy()


def _oracle_fp8_problem(w) -> ref.Problem:
    """The oracle's view of FP8 rows: dequantized in float64 (physical order)."""

    def region(r):
        if r is None:
            return None
        return ref.Region(ofp8.dequantize_rows(r.k.numpy(), r.k_scale.numpy()),
                          ofp8.dequantize_rows(r.v.numpy(), r.v_scale.numpy()), int(r.n_rows),
                          None if r.valid is None else r.valid.numpy())

    idx = None if w.r1_index is None else w.r1_index.numpy()
    return ref.Problem(q=w.q.numpy(), scale=float(w.scale), r0=region(w.r0), window=int(w.window),
                       q_pos0=int(w.q_pos0), k_pos0=int(w.k_pos0), r1=region(w.r1), r1_index=idx)


def _oracle(w):
    if w.r0.k.dtype == torch.uint8:
        return ref.attention(_oracle_fp8_problem(w))
    return ref.attention(ref.from_workload(w, logical_ring=False))


# --------------------------------------------------------------------------- poisoned hidden rows

POISON_CASES = [
    ("window", dict(batch=1, tokens=7, heads=64, head_dim=512, n0=300, window=100, q_pos0=260, k_pos0=0)),
    ("valid", dict(batch=2, tokens=3, heads=64, head_dim=512, n0=290, valid0_frac=0.5)),
    ("index_unused", dict(batch=1, tokens=3, heads=64, head_dim=512, n0=70, window=32, q_pos0=60, k_pos0=0,
                          n1=900, r1_mode="index", r1_k=300, idx_invalid_frac=0.1)),
    ("two_regions_valid", dict(batch=2, tokens=2, heads=64, head_dim=512, n0=128, n1=450, r1_mode="all",
                               valid1_frac=0.8)),
    ("index_valid", dict(batch=2, tokens=1, heads=64, head_dim=512, n0=33, n1=640, r1_mode="index",
                         r1_k=500, valid1_frac=0.6)),
    ("long_valid", dict(batch=1, tokens=1, heads=64, head_dim=512, n0=4500, valid0_frac=0.9)),
]


POISON_PARAMS = [(label, kw, mode) for label, kw in POISON_CASES for mode in KERNEL_MODES
                 if not (mode == "wide" and _indexed(kw))]


@pytest.mark.parametrize("label,kw,mode", POISON_PARAMS, ids=[f"{c[0]}-{c[2]}" for c in POISON_PARAMS])
def test_poisoned_hidden_rows(label, kw, mode):
    w = free_row0(wl.random_problem(zlib.crc32(label.encode()) % 1000 + 31, **kw))
    w, n = poison_hidden(w)
    assert n > 0
    want = _oracle(w)
    compare(_run(w, mode), want, f"{label}/{mode} ({n} NaN rows)")
    compare(_run(w, mode, use_map=False), want, f"{label}/{mode} no map")


@pytest.mark.parametrize("mode", KERNEL_MODES)
@pytest.mark.parametrize("fp8", [False, True], ids=["f16", "fp8"])
def test_unpadded_tail_stays_hidden(mode, fp8):
    """The rows between the live count and the block end hold NaN (the pad stage
    has not run): they are masked like any hidden row."""
    w = wl.random_problem(55, batch=2, tokens=3, heads=64, head_dim=512, n0=77, n1=45, r1_mode="all",
                          valid1_frac=0.9)
    if fp8:
        w = wl.fp8_variant(w, 56)
    want = _oracle(w)
    compare(_run(w, mode, pad=False), want, f"unpadded tail/{mode}/{'fp8' if fp8 else 'f16'}")


@pytest.mark.parametrize("mode", ["dims", "keys", "plan"])
def test_poisoned_decode_workloads(mode):
    """Full-size decode batches with their hidden rows poisoned: the ratio-128
    layer's invalid compressed slots, and the ratio-4 layer's compressed rows
    outside each sequence's top-512 (1536 of 2048 per sequence)."""
    for name in ("decode_r128_b64", "decode_r4"):
        w, n = poison_hidden(wl.named(name))
        assert n > 0
        compare(_run(w, mode), _oracle(w), f"{name}/{mode} ({n} NaN rows)")


def test_poisoned_decode_workloads_wide():
    """The same for the wide DIMS split on the batches without index lists."""
    for name in ("decode_r128_b64", "decode_swa"):
        w, n = poison_hidden(wl.named(name))
        compare(_run(w, "wide"), _oracle(w), f"{name}/wide ({n} NaN rows)")


# --------------------------------------------------------------------------- one-hot values

def _decode_r4_onehot(topk=384):
    """The ratio-4 decode batch with a top-384 list (128 ring rows + 384 entries
    fill the 512 columns): ring row j -> column j, listed compressed row -> 128 +
    its rank in the sequence's list; the rest are poisoned."""
    w = wl.decode_ratio4(seed=116, topk=topk)
    rank = {}
    for b in range(w.q.shape[0]):
        for k, c in enumerate(w.r1_index[b, 0].tolist()):
            rank[(b, c)] = 128 + k
    w = onehot_values(w, lambda b, j: j, lambda b, c: rank.get((b, c), -1))
    return poison_hidden(w)[0]


@pytest.mark.parametrize("mode", ["dims", "keys", "plan", "split3", "wide"])
def test_onehot_decode_workloads(mode):
    w = wl.named("decode_r128_b64")
    w = poison_hidden(onehot_values(w, lambda b, j: j, lambda b, c: 128 + c))[0]
    out, want = _run(w, mode), _oracle(w)
    compare(out, want, f"decode_r128_b64 one-hot/{mode}")
    check_onehot(out, want, f"decode_r128_b64 one-hot/{mode}")
    if mode == "wide":
        return   # (the ratio-4 batch has index lists)
    w = _decode_r4_onehot()
    out, want = _run(w, mode), _oracle(w)
    compare(out, want, f"decode_r4 top-384 one-hot/{mode}")
    check_onehot(out, want, f"decode_r4 top-384 one-hot/{mode}")


def test_onehot_prefill_chunks():
    """The 2048-token window chunk (row j -> column j mod 128: a 128-row window
    never repeats a column) and a 2048-token indexed chunk at position 30720
    (2175 raw rows, column j mod 128; 384 compressed rows, top-256 lists, column
    128 + c), through the prefill kernel in the benchmark's launch."""
    w = onehot_values(wl.named("prefill_swa"), lambda b, j: j % 128, None)
    out, want = _run(w, "prefill"), _oracle(w)
    compare(out, want, "prefill_swa one-hot")
    check_onehot(out, want, "prefill_swa one-hot")
    w = wl.random_problem(117, batch=1, tokens=2048, heads=64, head_dim=512, n0=2175, window=128,
                          q_pos0=30720, k_pos0=30593, n1=384, r1_mode="index", r1_k=256)
    w = onehot_values(w, lambda b, j: j % 128, lambda b, c: 128 + c)
    out, want = _run(w, "prefill"), _oracle(w)
    compare(out, want, "indexed chunk one-hot")
    check_onehot(out, want, "indexed chunk one-hot")


# --------------------------------------------------------------------------- wrong speculative starts

def _window_then_dense(tokens, heads, batch=2):
    """Raw rows 0..199 with a 16-row window that ends in raw block 3 for every
    token, then 100 dense compressed rows: the lists are [3, 7, 8, 9, 10] while
    the window arithmetic guesses 3, 4, 5, ... (block 4 onward is skipped)."""
    return wl.random_problem(121, batch=batch, tokens=tokens, heads=heads, head_dim=512, n0=200, window=16,
                             q_pos0=111, k_pos0=0, n1=100, r1_mode="all")


def _leading_invalid(tokens, heads, r1=False):
    """Raw rows 0..299 of which rows 0..63 (blocks 0 and 1) are invalid: the lists
    start at block 2 while the first entries are guessed as blocks 0 and 1."""
    kw = dict(n1=80, r1_mode="index", r1_k=64) if r1 else {}
    w = wl.random_problem(122, batch=2, tokens=tokens, heads=heads, head_dim=512, n0=300, valid0_frac=0.7,
                          **kw)
    w.r0.valid[:, :64] = 0
    return w


def _first_block_invalid(tokens, heads, batch=2):
    """The window case with raw block 3 invalid: no raw row is visible, so a tile's
    list starts in region 1 while HEADS prefill guesses block 3."""
    w = _window_then_dense(tokens, heads, batch)
    valid = torch.ones(w.r0.k.shape[:2], dtype=torch.uint8)
    valid[:, 96:128] = 0
    return dataclasses.replace(w, r0=dataclasses.replace(w.r0, valid=valid))


SPEC_CASES = [
    ("window_then_dense", _window_then_dense),
    ("leading_invalid", _leading_invalid),
    ("leading_invalid_indexed", lambda t, h: _leading_invalid(t, h, r1=True)),
    ("first_block_invalid", _first_block_invalid),
]


SPEC_PARAMS = [(label, make, mode) for label, make in SPEC_CASES for mode in KERNEL_MODES
               if not (mode == "wide" and label.endswith("indexed"))]


@pytest.mark.parametrize("fp8", [False, True], ids=["f16", "fp8"])
@pytest.mark.parametrize("label,make,mode", SPEC_PARAMS, ids=[f"{c[0]}-{c[2]}" for c in SPEC_PARAMS])
def test_wrong_speculative_start(label, make, mode, fp8):
    tokens = 16 if mode == "prefill" else 1
    w = make(tokens, 64)
    if fp8:
        w = wl.fp8_variant(w, 123)
    w, n = poison_hidden(w)
    assert n > 0
    want = _oracle(w)
    compare(_run(w, mode), want, f"{label}/{mode}/{'fp8' if fp8 else 'f16'} ({n} NaN rows)")


@pytest.mark.parametrize("fp8", [False, True], ids=["f16", "fp8"])
@pytest.mark.parametrize("label,make", [("window_then_dense", _window_then_dense),
                                        ("first_block_invalid", _first_block_invalid)])
def test_speculative_start_full_grid(label, make, fp8):
    """64 sequences x 4 head groups: 256 DIMS workgroups, as many as the chip has
    CUs.  With lists this short (5 and 4 entries) the float16 producers stage the
    second entry's V rows late and masked; the second case also stages the first
    entry again (its guess is wrong)."""
    w = make(1, 64, batch=64)
    if fp8:
        w = wl.fp8_variant(w, 126)
    w, n = poison_hidden(w)
    assert n > 0
    compare(_run(w, "dims"), _oracle(w), f"{label}/full grid/{'fp8' if fp8 else 'f16'} ({n} NaN rows)")


def test_split_parts_with_wrong_guesses():
    """Split parts guess their first entries from an even share of the dense
    blocks; with leading invalid blocks every part's share moves."""
    w, _ = poison_hidden(_leading_invalid(1, 64))
    want = _oracle(w)
    for splits in (2, 4, 7):
        dp = pipeline.to_device(w, DEV)
        out = pipeline.step(dp, "decode", 1, splits=splits).cpu().double().numpy()
        torch.cuda.synchronize()
        compare(out, want, f"leading_invalid split {splits}")


# --------------------------------------------------------------------------- tile size

def test_tile_longer_than_the_chunk():
    """bq = 2^31 - 1: the map has one tile, and attention with the same bq agrees
    with the oracle (the host clamps the tile to the chunk)."""
    w = wl.random_problem(124, batch=2, tokens=40, heads=64, head_dim=512, n0=100, window=24, q_pos0=60,
                          k_pos0=0)
    big = 2 ** 31 - 1
    want = _oracle(w)
    compare(_run(w, "prefill", bq=big), want, "prefill bq = 2^31 - 1")
    compare(_run(w, "dims", bq=big), want, "decode bq = 2^31 - 1")


# --------------------------------------------------------------------------- large score jumps

@pytest.mark.parametrize("mode", KERNEL_MODES)
def test_score_jump_after_the_first_block(mode):
    """Keys of a later block scaled by 16: the scores there exceed the first block's
    maximum by far more than 2^8 in the base-2 softmax, so every kernel must move
    its reference max and rescale the output after weights exist.  Compared with
    the oracle."""
    w = wl.random_problem(125, batch=1, tokens=19, heads=64, head_dim=512, n0=160, q_std=2.0, window=96,
                          q_pos0=140, k_pos0=0)
    k = w.r0.k.clone()
    k[:, 96:128] = (k[:, 96:128].float() * 16).half()
    w = dataclasses.replace(w, r0=dataclasses.replace(w.r0, k=k))
    want = _oracle(w)
    compare(_run(w, mode), want, f"score jump/{mode}")
