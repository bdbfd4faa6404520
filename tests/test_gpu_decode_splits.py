"""GPU parity of the ways the matrix-core decode kernel divides a workgroup's
work over its four waves, each forced with its flag: DIMS (the waves share every
key block and split the head dimension; also WIDE, the same over 32 heads per
workgroup) and KEYS (the waves take different 16-row halves of the key blocks and
merge their partial results).  Both against the
float64 oracle within the attention tolerance (max-abs 1e-2, mean-abs 1e-3), on
the decode workloads at full size and on general cases (windows, validity masks,
two regions, index lists with unused entries, empty regions, tokens that see no
row, lists that do not fill a round of the four waves), with and without a block
map, plain and split over several workgroups.
"""

import zlib

import numpy as np
import pytest
import torch

from oracle import reference as ref
from query_flashattention_amd import ds4attn as da
from query_flashattention_amd import pipeline, workloads as wl
from tests.parity_util import compare as _compare, oracle_full

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3
DEV = "cuda:0"
SPLITS = {"dims": da.FLAG_DECODE_DIMS, "keys": da.FLAG_DECODE_KEYS}
# DIMS over 32 heads per workgroup: head counts that are multiples of 32, no index lists
WIDE = da.FLAG_DECODE_WIDE


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    da.lib()  # fail loudly if the HIP library is missing


def _run(w, flags, use_map=True, splits=1):
    dp = pipeline.to_device(w, DEV)
    dp.flags = flags
    if use_map:
        out = pipeline.step(dp, "decode", 1, splits=splits)
    else:
        dp.r0.pad_in_place()
        if dp.r1 is not None:
            dp.r1.pad_in_place()
        a = dp.args()
        if splits > 1:
            ws = torch.empty(da.ds4attn_decode_workspace_bytes(a, splits), dtype=torch.uint8, device=DEV)
            da.ds4attn_decode_split(a, dp.q, None, 1, dp.o, splits, ws)
        else:
            da.ds4attn_decode(a, dp.q, None, 1, dp.o)   # no workspace: unsplit
        out = dp.o
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


@pytest.mark.parametrize("split", list(SPLITS))
@pytest.mark.parametrize("name", ["decode_swa", "decode_r128", "decode_r128_b64"])
def test_workload_full(name, split):
    w = wl.named(name)
    _compare(_run(w, SPLITS[split]), ref.attention(ref.from_workload(w)), f"{name}/{split}")


@pytest.mark.parametrize("split", list(SPLITS))
def test_ratio4_full(split):
    w = wl.named("decode_r4")
    _compare(_run(w, SPLITS[split]), oracle_full("decode_r4"), f"decode_r4/{split}")


CASES = [
    ("ragged", dict(batch=3, tokens=2, heads=16, head_dim=512, n0=77)),
    ("one_row", dict(batch=1, tokens=1, heads=16, head_dim=512, n0=1)),
    ("window", dict(batch=1, tokens=7, heads=32, head_dim=512, n0=300, window=100, q_pos0=260, k_pos0=0)),
    ("valid", dict(batch=2, tokens=3, heads=48, head_dim=512, n0=290, valid0_frac=0.5)),
    ("two_regions", dict(batch=2, tokens=2, heads=64, head_dim=512, n0=128, n1=450, r1_mode="all",
                         valid1_frac=0.8)),
    ("index", dict(batch=1, tokens=3, heads=64, head_dim=512, n0=70, window=32, q_pos0=60, k_pos0=0,
                   n1=900, r1_mode="index", r1_k=300, idx_invalid_frac=0.1)),
    ("index_valid", dict(batch=2, tokens=1, heads=64, head_dim=512, n0=33, n1=640, r1_mode="index",
                         r1_k=500, valid1_frac=0.6)),
    ("big_scores", dict(batch=1, tokens=3, heads=64, head_dim=512, n0=400, q_std=4.0)),
    ("empty_r0", dict(batch=1, tokens=2, heads=16, head_dim=512, n0=0, n1=330, r1_mode="all")),
    ("masked_tokens", dict(batch=1, tokens=5, heads=16, head_dim=512, n0=40, window=4, q_pos0=0, k_pos0=3)),
    ("index_all_unused", dict(batch=1, tokens=2, heads=16, head_dim=512, n0=10, n1=20, r1_mode="index",
                              r1_k=32, idx_invalid_frac=1.0)),
    # a window that reaches one or two blocks of a ten-block region: a block guessed
    # past the end of the list is in flight while the list is consumed
    ("short_window", dict(batch=2, tokens=3, heads=32, head_dim=512, n0=320, window=20, q_pos0=300,
                          k_pos0=0)),
    # long lists: more than one chunk of 64 list entries (the visibility masks are
    # rebuilt as the waves go) and more than one chunk of 512 index entries
    ("long_dense", dict(batch=1, tokens=1, heads=16, head_dim=512, n0=4500, valid0_frac=0.9)),
    ("long_index", dict(batch=1, tokens=2, heads=16, head_dim=512, n0=128, n1=3000, r1_mode="index",
                        r1_k=1500, idx_invalid_frac=0.05)),
]


@pytest.mark.parametrize("split", list(SPLITS))
@pytest.mark.parametrize("label,kw", CASES, ids=[c[0] for c in CASES])
def test_random(label, kw, split):
    w = wl.random_problem(zlib.crc32(label.encode()) % 1000, **kw)
    want = ref.attention(ref.from_workload(w))
    out = _run(w, SPLITS[split])
    _compare(out, want, f"{label}/{split}")
    _compare(_run(w, SPLITS[split], use_map=False), want, f"{label}/{split} no map")
    if label == "masked_tokens":
        assert (out[0, :3] == 0).all()   # tokens 0..2 see no row: exact zeros


@pytest.mark.parametrize("split", list(SPLITS))
@pytest.mark.parametrize("label,kw,splits", [
    ("valid", dict(batch=2, tokens=3, heads=16, head_dim=512, n0=450, valid0_frac=0.5), 4),
    ("index", dict(batch=1, tokens=2, heads=64, head_dim=512, n0=70, window=32, q_pos0=60, k_pos0=0,
                   n1=900, r1_mode="index", r1_k=300, idx_invalid_frac=0.1), 3),
    ("masked_tokens", dict(batch=1, tokens=5, heads=16, head_dim=512, n0=40, window=4, q_pos0=0,
                           k_pos0=3), 2),
    ("short_window", dict(batch=2, tokens=3, heads=32, head_dim=512, n0=320, window=70, q_pos0=290,
                          k_pos0=0), 3),
], ids=["valid", "index", "masked_tokens", "short_window"])
def test_split_over_workgroups(label, kw, splits, split):
    w = wl.random_problem(zlib.crc32(label.encode()) % 1000 + 7, **kw)
    want = ref.attention(ref.from_workload(w))
    _compare(_run(w, SPLITS[split], splits=splits), want, f"{label}/{split} x{splits}")
    _compare(_run(w, SPLITS[split], use_map=False, splits=splits), want, f"{label}/{split} x{splits} no map")


@pytest.mark.parametrize("name", ["decode_swa", "decode_r128", "decode_r128_b64"])
def test_wide_workload_full(name):
    w = wl.named(name)
    _compare(_run(w, WIDE), ref.attention(ref.from_workload(w)), f"{name}/wide")


WIDE_CASES = [(label, kw) for label, kw in CASES if kw["heads"] % 32 == 0 and kw.get("r1_mode") != "index"] + [
    ("wide_one_row", dict(batch=2, tokens=1, heads=64, head_dim=512, n0=1)),
    ("wide_masked_tokens", dict(batch=1, tokens=5, heads=32, head_dim=512, n0=40, window=4, q_pos0=0, k_pos0=3)),
    ("wide_long_dense", dict(batch=1, tokens=1, heads=32, head_dim=512, n0=4500, valid0_frac=0.9)),
    ("wide_ragged", dict(batch=3, tokens=2, heads=96, head_dim=512, n0=77)),
]


@pytest.mark.parametrize("label,kw", WIDE_CASES, ids=[c[0] for c in WIDE_CASES])
def test_wide_random(label, kw):
    w = wl.random_problem(zlib.crc32(label.encode()) % 1000 + 3, **kw)
    want = ref.attention(ref.from_workload(w))
    out = _run(w, WIDE)
    _compare(out, want, f"{label}/wide")
    _compare(_run(w, WIDE, use_map=False), want, f"{label}/wide no map")
    if label == "wide_masked_tokens":
        assert (out[0, :3] == 0).all()   # tokens 0..2 see no row: exact zeros


def test_both_splits_agree_on_ratio128_single_sequence():
    w = wl.named("decode_r128")
    a = _run(w, da.FLAG_DECODE_DIMS)
    b = _run(w, da.FLAG_DECODE_KEYS)
    _compare(a, b, "dims vs keys")
