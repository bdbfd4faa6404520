"""GPU parity of the compressor step (ds4attn_compress) against the float64 oracle.

Pooled rows are compared element by element with the oracle within max-abs 1e-2
and mean-abs 1e-3 (float32 arithmetic, one float16 rounding of values below 5 in
magnitude: at most 2^-9 per element); the state update is a copy and is compared
bit for bit, as are rows the call must not touch.  Cases: the 2048-row prefill
chunk at ratio 4 and 128, the 64-sequence decode batch crossing a boundary (and
not crossing one), ragged counts, odd ratios, ratio 1 (the identity), and the
same rows fed in chunks (bit-identical to one call).
"""

import numpy as np
import pytest
import torch

from oracle import compress as ocp
from query_flashattention_amd import ds4attn as da
from query_flashattention_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(ci, comp_rows=None, sentinel=7.0):
    b, ratio, d = ci.state_kv.shape
    n_new = ci.kv_new.shape[1]
    n_out = (ci.n_state + n_new) // ratio
    rows = max(n_out, 1) + 2 if comp_rows is None else comp_rows
    st_kv = ci.state_kv.to(DEV).clone()
    st_sc = ci.state_score.to(DEV).clone()
    comp = torch.full((b, rows, d), sentinel, dtype=torch.float16, device=DEV)
    got = da.ds4attn_compress(st_kv, st_sc, ci.n_state, ci.kv_new.to(DEV), ci.score_new.to(DEV), ratio, comp)
    torch.cuda.synchronize()
    assert got == n_out
    return comp.cpu(), st_kv.cpu(), st_sc.cpu(), n_out


def _check(ci, comp, st_kv, st_sc, n_out):
    b, ratio, d = ci.state_kv.shape
    n_next = (ci.n_state + ci.kv_new.shape[1]) % ratio
    errs = []
    for s in range(b):
        pooled, s_kv, s_sc = ocp.compress_step(ci.state_kv[s, :ci.n_state].numpy(),
                                               ci.state_score[s, :ci.n_state].numpy(),
                                               ci.kv_new[s].numpy(), ci.score_new[s].numpy(), ratio)
        assert pooled.shape[0] == n_out
        errs.append(np.abs(comp[s, :n_out].double().numpy() - pooled))
        # the new state, bit for bit; rows past it untouched
        assert torch.equal(st_kv[s, :n_next], torch.from_numpy(s_kv))
        assert torch.equal(st_sc[s, :n_next], torch.from_numpy(s_sc))
        keep = slice(n_next, ratio)
        assert torch.equal(st_kv[s, keep], ci.state_kv[s, keep])
        assert torch.equal(st_sc[s, keep], ci.state_score[s, keep])
        # compressed rows past n_out untouched
        assert torch.all(comp[s, n_out:] == 7.0)
    if n_out:
        e = np.stack(errs)
        print(f"max abs err {e.max():.3e}, mean {e.mean():.3e}")
        assert e.max() <= 1e-2 and e.mean() <= 1e-3


CASES = [
    # label, batch, ratio, n_state, n_new, head_dim
    ("prefill_r4_chunk", 1, 4, 0, 2048, 512),
    ("prefill_r128_chunk", 1, 128, 0, 2048, 512),
    ("prefill_r128_with_state", 1, 128, 77, 2048, 512),
    ("decode_r4_boundary", 64, 4, 3, 1, 512),
    ("decode_r128_boundary", 64, 128, 127, 1, 512),
    ("decode_r128_no_boundary", 64, 128, 5, 1, 512),
    ("ragged_small", 3, 4, 2, 13, 64),
    ("odd_ratio", 2, 7, 6, 50, 256),
    ("groups_and_state", 2, 128, 100, 300, 512),
    ("d128", 5, 16, 9, 40, 128),
    ("exactly_one_group", 2, 32, 31, 1, 512),
]


@pytest.mark.parametrize("label,b,ratio,n_state,n_new,d", CASES, ids=[c[0] for c in CASES])
def test_compress_matches_oracle(label, b, ratio, n_state, n_new, d):
    ci = wl.compress_inputs(300 + [c[0] for c in CASES].index(label), b, ratio, n_state, n_new, d)
    _check(ci, *_run(ci))


def test_compress_wide_scores():
    """Scores with std 8: the weights span many orders of magnitude."""
    ci = wl.compress_inputs(11, 4, 128, 3, 381, 512, score_std=8.0)
    _check(ci, *_run(ci))


def test_ratio_one_copies_rows():
    ci = wl.compress_inputs(12, 3, 1, 0, 37, 512)
    comp, _, _, n_out = _run(ci)
    assert n_out == 37
    assert torch.equal(comp[:, :37], ci.kv_new)


@pytest.mark.parametrize("ratio,chunks", [(4, [3, 1, 5, 0, 7, 2, 64]), (128, [100, 27, 1, 300, 5, 128])])
def test_chunked_calls_equal_one_call(ratio, chunks):
    b, d = 2, 512
    n = sum(chunks)
    ci = wl.compress_inputs(13 + ratio, b, ratio, 0, n, d)
    whole, w_kv, w_sc, n_out = _run(ci)
    st_kv = ci.state_kv.to(DEV).clone()
    st_sc = ci.state_score.to(DEV).clone()
    kv, sc = ci.kv_new.to(DEV), ci.score_new.to(DEV)
    comp = torch.full((b, n_out + 2, d), 7.0, dtype=torch.float16, device=DEV)
    n_state, n_comp, at = 0, 0, 0
    for c in chunks:
        out = comp[:, n_comp:]
        k = da.ds4attn_compress(st_kv, st_sc, n_state, kv[:, at:at + c].contiguous(),
                                sc[:, at:at + c].contiguous(), ratio, out if out.shape[1] else None)
        n_comp += k
        n_state = (n_state + c) % ratio
        at += c
    torch.cuda.synchronize()
    assert n_comp == n_out
    assert torch.equal(comp.cpu(), whole)
    m = n % ratio
    assert torch.equal(st_kv.cpu()[:, :m], w_kv[:, :m])
    assert torch.equal(st_sc.cpu()[:, :m], w_sc[:, :m])
