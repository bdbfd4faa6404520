"""GPU parity at the capacity limits of the matrix-core attention kernel, against
the float64 oracle (same bar as the other parity tests: max-abs 1e-2, mean-abs
1e-3):

* index lists of the largest supported length (2048 entries per token), in both
  decode work splits and in prefill;
* index lists that are unsorted, hold duplicates (a multiset: a row listed twice
  counts twice) and entries past the region's rows (unused);
* a dense region of exactly the largest block list the kernel keeps in LDS
  (2048 blocks = 65536 rows), and one row more, which the library runs on the
  vector-ALU kernel.
"""

import numpy as np
import pytest
import torch

from oracle import reference as ref
from query_flashattention_amd import ds4attn as da
from query_flashattention_amd import pipeline, workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(w, entry, bq, flags=0):
    dp = pipeline.to_device(w, DEV)
    dp.flags = flags
    out = pipeline.step(dp, entry, bq)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def _compare(out, want, label):
    err = np.abs(out - want)
    print(f"{label}: max abs {err.max():.3e} mean abs {err.mean():.3e} over {err.size} values")
    assert np.isfinite(out).all(), label
    assert err.max() <= 1e-2 and err.mean() <= 1e-3, label


@pytest.mark.parametrize("entry,bq,flags", [("decode", 1, da.FLAG_DECODE_DIMS), ("decode", 1, da.FLAG_DECODE_KEYS),
                                            ("prefill", 16, 0)], ids=["decode_dims", "decode_keys", "prefill"])
def test_longest_index_list(entry, bq, flags):
    w = wl.random_problem(601, batch=1, tokens=2 if entry == "decode" else 3, heads=16 if entry == "decode" else 64,
                          head_dim=512, n0=40, window=24, q_pos0=39, k_pos0=0, n1=4100, r1_mode="index",
                          r1_k=2048, idx_invalid_frac=0.05)
    _compare(_run(w, entry, bq, flags), ref.attention(ref.from_workload(w)), f"r1_k=2048 {entry}")


def _messy_index(w, seed):
    """Shuffle each list, repeat some entries and point some past the region's rows."""
    g = torch.Generator().manual_seed(seed)
    idx = w.r1_index.clone()
    b, t, k = idx.shape
    flat = idx.view(b * t, k)
    for r in range(b * t):
        flat[r] = flat[r, torch.randperm(k, generator=g)]
    dup = torch.rand(b * t, k, generator=g) < 0.2
    src = torch.randint(0, k, (b * t, k), generator=g)
    flat[dup] = torch.gather(flat, 1, src)[dup]
    far = torch.rand(b * t, k, generator=g) < 0.05
    flat[far] = w.r1.n_rows + torch.randint(0, 1000, (int(far.sum()),), generator=g, dtype=torch.int32)
    w.r1_index = flat.view(b, t, k)
    return w


@pytest.mark.parametrize("entry,bq,flags", [("decode", 1, da.FLAG_DECODE_DIMS), ("decode", 1, da.FLAG_DECODE_KEYS),
                                            ("prefill", 16, 0)], ids=["decode_dims", "decode_keys", "prefill"])
def test_unsorted_index_lists_with_duplicates_and_far_entries(entry, bq, flags):
    w = wl.random_problem(602, batch=2, tokens=1 if entry == "decode" else 5, heads=16 if entry == "decode" else 64,
                          head_dim=512, n0=50, n1=700, r1_mode="index", r1_k=256)
    w = _messy_index(w, 603)
    idx = w.r1_index.numpy()
    assert (idx >= w.r1.n_rows).any() and any(len(set(r)) < len(r) for r in idx.reshape(-1, idx.shape[-1]))
    _compare(_run(w, entry, bq, flags), ref.attention(ref.from_workload(w)), f"messy index {entry}")


@pytest.mark.parametrize("n0", [65536, 65537], ids=["list_cap_blocks", "one_row_more"])
def test_longest_dense_region(n0):
    w = wl.random_problem(604, batch=1, tokens=1, heads=16, head_dim=512, n0=n0)
    _compare(_run(w, "decode", 1), ref.attention(ref.from_workload(w)), f"n0={n0}")
