"""ds4attn_decode_noalloc (the decode entry point for callers that cannot
allocate) against ds4attn_decode with a caller workspace, through the C ABI.

Two split calls in a row share the device's static scratch array: the ratio-128
layer at 32K for one sequence (the plan splits it over 4 parts per group of 16
heads: 16 records), then a smaller one (16 heads, 96 compressed rows: 2 parts, 2
records), whose records must not mix with the first call's.  A 64-sequence batch
(no split) takes the unsplit path, and the single sequence on FP8 rows splits
too.  Each output equals ds4attn_decode's bit for
bit (same kernels, same split) and is within the attention tolerance of the
float64 oracle.
"""

import numpy as np
import pytest
import torch

from oracle import reference as ref
from query_flashattention_amd import ds4attn as da
from query_flashattention_amd import pipeline, workloads as wl
from tests.parity_util import compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _small_split_case():
    return wl.random_problem(131, batch=1, tokens=1, heads=16, head_dim=512, n0=128, n1=96,
                             r1_mode="all", valid1_frac=0.9)


def _both(w):
    """(noalloc output, decode-with-workspace output, split count the plan picked)."""
    dp = pipeline.to_device(w, DEV)
    dp.r0.pad_in_place()
    if dp.r1 is not None:
        dp.r1.pad_in_place()
    a = dp.args()
    blk = da.blockmap(a, 1, DEV)
    blk = blk if blk.numel() else None
    nbytes = da.ds4attn_workspace_bytes(a, False)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV) if nbytes else None
    da.ds4attn_decode(a, dp.q, blk, 1, dp.o, ws)
    want = dp.o.clone()
    dp.o.fill_(float("nan"))
    da.ds4attn_decode_noalloc(a, dp.q, blk, 1, dp.o)
    torch.cuda.synchronize()
    records = nbytes // (16 * 512 * 4 + 128)
    return dp.o.cpu(), want.cpu(), records


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    da.lib()


def test_noalloc_matches_decode_two_calls_in_a_row():
    big = wl.named("decode_r128")
    got, want, rec = _both(big)
    assert rec == 24                        # 4 groups of 16 heads x 6 parts
    assert torch.equal(got, want)
    compare(got.double().numpy(), ref.attention(ref.from_workload(big)), "noalloc decode_r128")
    small = _small_split_case()
    got, want, rec = _both(small)
    assert rec == 3                         # 1 group x 3 parts: a smaller input in the same array
    assert torch.equal(got, want)
    compare(got.double().numpy(), ref.attention(ref.from_workload(small)), "noalloc small split")


def test_noalloc_unsplit_batch():
    w = wl.named("decode_swa")
    got, want, rec = _both(w)
    assert rec == 0
    assert torch.equal(got, want)
    compare(got.double().numpy(), ref.attention(ref.from_workload(w)), "noalloc decode_swa")


def test_noalloc_fp8_rows_split():
    """FP8 rows through the split: each part folds its V scales into the weights
    under a factor of its own and leaves its record in true units, in the static
    array as in a caller's workspace."""
    from tests.test_gpu_fp8 import _oracle_problem
    w = wl.fp8_variant(wl.named("decode_r128"), 5)
    got, want, rec = _both(w)
    assert rec > 0                          # the plan splits the single sequence
    assert torch.equal(got, want)
    compare(got.double().numpy(), ref.attention(_oracle_problem(w)), "noalloc decode_r128 fp8")

