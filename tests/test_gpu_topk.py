"""GPU parity of the top-k index selection (``ds4attn_topk``) against the oracle
(``oracle.topk``): the index lists must be identical, element by element.

Sizes: the ratio-4 prefill chunk (2048 tokens scoring 7680 compressed rows) and
the ratio-4 decode batch (64 tokens scoring 2048 rows), both with k = 512, plus
edge cases -- empty rows, rows shorter than k, k = 1, k = n, the largest k,
rows longer than the kernel keeps in LDS, runs of equal scores, signed zeros,
infinities and NaNs, and a row stride wider than the row.  The last test feeds
the selection into the indexed attention and compares that with the oracle's
attention over the oracle's selection.
"""

import dataclasses

import numpy as np
import pytest
import torch

from oracle import reference as ref
from oracle import topk as otk
from query_flashattention_amd import ds4attn as da
from query_flashattention_amd import pipeline, workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; none is visible")
    da.lib()  # fail loudly if the HIP library is missing


def _check(scores, k, label):
    got = da.topk(scores.to(DEV), k)
    torch.cuda.synchronize()
    want = otk.topk(scores.numpy(), k)
    got = got.cpu().numpy()
    bad = np.nonzero((got != want).any(axis=1))[0]
    print(f"{label}: rows {scores.shape[0]} n {scores.shape[1]} k {k} mismatching rows {bad.size}")
    assert bad.size == 0, (label, bad[:8].tolist())


@pytest.mark.parametrize("rows,n,kind", [
    (2048, 7680, "normal"),    # ratio-4 prefill chunk at position 30720
    (64, 2048, "normal"),      # ratio-4 decode batch at an 8K context
    (256, 3000, "coarse"),
    (256, 3000, "special"),
])
def test_topk_workload(rows, n, kind):
    _check(wl.indexer_scores(201, rows, n, kind), 512, f"{kind}")


@pytest.mark.parametrize("n,k", [
    (0, 5), (1, 1), (3, 8), (511, 512), (512, 512), (513, 512), (700, 1),
    (2048, 2048), (16384, 512), (16385, 512), (40000, 2048), (97, 33),
])
def test_topk_sizes(n, k):
    _check(wl.indexer_scores(202 + n, 6, n, "normal"), k, f"n{n}_k{k}")
    _check(wl.indexer_scores(203 + n, 6, n, "coarse"), k, f"n{n}_k{k}_coarse")


def test_topk_long_rows_with_specials():
    _check(wl.indexer_scores(204, 8, 50000, "special"), 700, "long special")


def test_topk_constant_rows():
    s = torch.full((3, 1000), -2.5)
    s[1] = 0.0
    s[2] = float("inf")
    _check(s, 100, "constant")


def test_topk_strided_rows():
    """Rows that sit inside a wider buffer, and an output with a wider row."""
    full = wl.indexer_scores(205, 40, 1300, "normal")
    view = full[:, 100:1100]
    d = full.to(DEV)[:, 100:1100]
    out = torch.full((40, 600), 12345, dtype=torch.int32, device=DEV)
    da.ds4attn_topk(d, 512, out[:, 40:552])
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.array_equal(o[:, 40:552], otk.topk(view.numpy(), 512))
    assert (o[:, :40] == 12345).all() and (o[:, 552:] == 12345).all()


def test_topk_feeds_indexed_attention():
    """Scores -> ds4attn_topk -> indexed ratio-4 decode, against the oracle's
    selection fed to the oracle's attention, on a sample of sequences."""
    w = wl.named("decode_r4")
    batch, n1 = w.q.shape[0], w.r1.n_rows
    scores = wl.indexer_scores(206, batch, n1, "normal")
    idx = da.topk(scores.to(DEV), wl.TOPK)
    torch.cuda.synchronize()
    want_idx = otk.topk(scores.numpy(), wl.TOPK)
    assert np.array_equal(idx.cpu().numpy(), want_idx)
    wg = dataclasses.replace(w, r1_index=idx.cpu().view(batch, 1, wl.TOPK))
    dp = pipeline.to_device(wg, DEV)
    out = pipeline.step(dp, "decode", 1)
    torch.cuda.synchronize()
    out = out.cpu().double().numpy()
    wo = dataclasses.replace(w, r1_index=torch.from_numpy(want_idx).view(batch, 1, wl.TOPK))
    seqs = [0, 5, 33, 63]
    want = ref.attention(ref.from_workload(wo), tokens=[(b, 0) for b in seqs])
    err = np.abs(out[seqs, 0] - want)
    print(f"topk->decode_r4: max abs {err.max():.3e} mean abs {err.mean():.3e}")
    assert err.max() <= 1e-2 and err.mean() <= 1e-3
