"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each check is chosen so that a plausible slip in ``oracle.reference`` -- a dropped
scale, a sign, a transposed operand, an off-by-one window edge, an ignored
validity mask, a swapped status code -- fails at least one of them:

* an independent pure-Python brute force (``oracle.brute``) on tiny inputs of
  every mask kind;
* closed forms (two keys: a logistic weight; a single visible row; all keys
  equal; scale 0);
* softmax invariants (rows of P sum to 1, shift of K along a direction
  orthogonal to nothing, affine V, permutation of rows);
* mode cross-checks (index list == validity mask, window == materialised mask,
  two regions == one concatenated region);
* block-map census by interval arithmetic, and the padded layout by bits;
* constants printed on the pages (tests/golden/ds4_constants.json).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, reference as ref
from oracle.reference import Problem, Region
from query_flashattention_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(rng, b=2, t=3, h=3, d=6, n0=13, window=0, q_pos0=0, k_pos0=0,
                  valid0=False, n1=0, r1_mode="none", valid1=False, r1_k=0, scale=0.37):
    q = rng.standard_normal((b, t, h, d))
    k0 = rng.standard_normal((b, n0, d))
    v0 = rng.standard_normal((b, n0, d))
    va0 = (rng.random((b, n0)) < 0.7).astype(np.uint8) if valid0 else None
    r1 = None
    idx = None
    if r1_mode != "none":
        k1 = rng.standard_normal((b, n1, d))
        v1 = rng.standard_normal((b, n1, d))
        va1 = (rng.random((b, n1)) < 0.6).astype(np.uint8) if valid1 else None
        r1 = Region(k1, v1, n1, va1)
        if r1_mode == "index":
            idx = rng.integers(-2, n1 + 2, size=(b, t, r1_k))   # includes unused entries
    return Problem(q, scale, Region(k0, v0, n0, va0), window, q_pos0, k_pos0, r1, idx)


TINY_CASES = [
    dict(),
    dict(valid0=True),
    dict(window=4, q_pos0=9, k_pos0=0, n0=13, t=4),
    dict(window=3, q_pos0=5, k_pos0=2, valid0=True, t=4),
    dict(n1=9, r1_mode="all"),
    dict(n1=9, r1_mode="all", valid1=True, valid0=True),
    dict(n1=11, r1_mode="index", r1_k=5),
    dict(n1=11, r1_mode="index", r1_k=6, valid1=True, window=5, q_pos0=12, k_pos0=3),
    dict(n0=0, n1=7, r1_mode="all"),
    dict(n0=40, d=8, h=4, t=2, window=33, q_pos0=39, k_pos0=0),
]


@pytest.mark.parametrize("case", range(len(TINY_CASES)))
def test_reference_equals_brute_force(case):
    rng = np.random.default_rng(1000 + case)
    p = _rand_problem(rng, **TINY_CASES[case])
    got = ref.attention(p)
    want = np.array(brute.attention(p), dtype=np.float64)
    assert got.shape == want.shape
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_two_keys_logistic_closed_form():
    """Two visible keys: weight of key 0 is 1/(1+exp(-(s0-s1))) -- pins the scale,
    the sign of the max subtraction and that scores use K (not V)."""
    q = np.array([[[[0.5, -1.25, 2.0]]]])
    k = np.array([[[1.0, 0.5, -0.25], [-0.75, 1.5, 0.5]]])
    v = np.array([[[3.0, -1.0, 0.5], [-2.0, 4.0, 1.0]]])
    scale = 0.375
    p = Problem(q, scale, Region(k, v, 2))
    s0 = scale * (0.5 * 1.0 + -1.25 * 0.5 + 2.0 * -0.25)
    s1 = scale * (0.5 * -0.75 + -1.25 * 1.5 + 2.0 * 0.5)
    w0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
    want = w0 * v[0, 0] + (1 - w0) * v[0, 1]
    np.testing.assert_allclose(ref.attention(p)[0, 0, 0], want, rtol=0, atol=1e-15)


def test_single_visible_row_returns_that_row():
    rng = np.random.default_rng(7)
    p = _rand_problem(rng, b=1, t=1, h=4, d=5, n0=9, valid0=False)
    p.r0.valid = np.zeros((1, 9), dtype=np.uint8)
    p.r0.valid[0, 6] = 1
    out = ref.attention(p)[0, 0]
    for h in range(4):
        np.testing.assert_array_equal(out[h], p.r0.v[0, 6])


def test_equal_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(8)
    p = _rand_problem(rng, b=1, t=2, h=3, d=4, n0=10, window=6, q_pos0=7, k_pos0=0)
    p.r0.k[:] = p.r0.k[:, :1]
    out = ref.attention(p)
    for t in range(2):
        rows = [j for j in range(10) if 0 <= 7 + t - j < 6]
        np.testing.assert_allclose(out[0, t], np.broadcast_to(p.r0.v[0, rows].mean(0), (3, 4)),
                                   rtol=0, atol=1e-14)


def test_scale_zero_is_uniform_average():
    rng = np.random.default_rng(9)
    p = _rand_problem(rng, b=1, t=1, h=2, d=3, n0=12, valid0=True, scale=0.0)
    rows = np.nonzero(p.r0.valid[0])[0]
    np.testing.assert_allclose(ref.attention(p)[0, 0], np.broadcast_to(p.r0.v[0, rows].mean(0), (2, 3)),
                               atol=1e-14)


def test_probabilities_sum_to_one_and_one_hot_values_return_them():
    """V = identity (one-hot rows) makes O equal to the probability rows."""
    rng = np.random.default_rng(10)
    n = 6
    q = rng.standard_normal((1, 1, 3, n))
    k = rng.standard_normal((1, n, n))
    v = np.eye(n)[None]
    p = Problem(q, 0.8, Region(k, v, n))
    o, probs, rows0, rows1 = ref.attention_probs(p, 0, 0)
    np.testing.assert_allclose(probs.sum(axis=1), 1.0, atol=1e-15)
    assert (probs > 0).all()
    np.testing.assert_allclose(o, probs, atol=1e-15)


def test_shift_of_keys_and_affine_values():
    rng = np.random.default_rng(11)
    p = _rand_problem(rng, b=1, t=3, h=2, d=5, n0=11, window=7, q_pos0=9)
    base = ref.attention(p)
    # adding the same vector to every key adds q.u to every score of a row: no change
    p2 = Problem(p.q, p.scale, Region(p.r0.k + rng.standard_normal(5), p.r0.v, 11),
                 p.window, p.q_pos0, p.k_pos0)
    np.testing.assert_allclose(ref.attention(p2), base, atol=1e-12)
    a, c = -1.5, rng.standard_normal(5)
    p3 = Problem(p.q, p.scale, Region(p.r0.k, a * p.r0.v + c, 11), p.window, p.q_pos0, p.k_pos0)
    np.testing.assert_allclose(ref.attention(p3), a * base + c, atol=1e-12)


def test_ring_rotation_is_a_permutation():
    """A ring buffer in physical order and in logical order give the same output
    (the decode workloads store the ring with a seeded write pointer)."""
    w = wl.decode_raw_swa(batch=3)
    w.q = w.q[:, :, :8]   # fewer heads keep the check fast; the rows are what matters
    phys = ref.attention(ref.from_workload(w, logical_ring=False))
    logi = ref.attention(ref.from_workload(w, logical_ring=True))
    np.testing.assert_allclose(phys, logi, atol=1e-12)
    # and the rotation really moved rows
    assert not torch.equal(w.r0.k, w.r0.logical()[0])


def test_index_mode_equals_validity_mask():
    rng = np.random.default_rng(12)
    p = _rand_problem(rng, b=1, t=1, h=2, d=4, n0=5, n1=20, r1_mode="all")
    chosen = np.array([1, 4, 5, 11, 19])
    valid1 = np.zeros((1, 20), dtype=np.uint8)
    valid1[0, chosen] = 1
    p_valid = Problem(p.q, p.scale, p.r0, r1=Region(p.r1.k, p.r1.v, 20, valid1))
    p_index = Problem(p.q, p.scale, p.r0, r1=Region(p.r1.k, p.r1.v, 20),
                      r1_index=np.array([[[19, -1, 4, 1, 11, 5, 25]]]))
    np.testing.assert_allclose(ref.attention(p_index), ref.attention(p_valid), atol=1e-14)


def test_window_equals_materialised_validity():
    rng = np.random.default_rng(13)
    p = _rand_problem(rng, b=1, t=4, h=2, d=4, n0=30, window=9, q_pos0=20, k_pos0=3)
    out = ref.attention(p)
    for t in range(4):
        valid = np.array([[1 if 0 <= (20 + t) - (3 + j) <= 8 else 0 for j in range(30)]], np.uint8)
        pt = Problem(p.q[:, t:t + 1], p.scale, Region(p.r0.k, p.r0.v, 30, valid))
        np.testing.assert_allclose(ref.attention(pt)[0, 0], out[0, t], atol=1e-14)


def test_two_regions_equal_their_concatenation():
    rng = np.random.default_rng(14)
    p = _rand_problem(rng, b=2, t=1, h=3, d=4, n0=7, valid0=True, n1=9, r1_mode="all", valid1=True)
    k = np.concatenate([p.r0.k, p.r1.k], axis=1)
    v = np.concatenate([p.r0.v, p.r1.v], axis=1)
    valid = np.concatenate([p.r0.valid, p.r1.valid], axis=1)
    pc = Problem(p.q, p.scale, Region(k, v, 16, valid))
    np.testing.assert_allclose(ref.attention(p), ref.attention(pc), atol=1e-14)


def test_fully_masked_query_outputs_zero():
    rng = np.random.default_rng(15)
    p = _rand_problem(rng, b=1, t=2, h=2, d=3, n0=8, window=4, q_pos0=0, k_pos0=100)
    assert np.all(ref.attention(p) == 0.0)
    assert np.all(np.array(brute.attention(p)) == 0.0)


def test_window_keeps_exactly_128_rows_including_own():
    """A query deep in a long raw region sees exactly the 128-token window,
    its own row included ([P-DS4] Fixed Model Shape: 128-token sliding window)."""
    n = 300
    p = Problem(np.zeros((1, 1, 1, 1)), 1.0, Region(np.zeros((1, n, 1)), np.zeros((1, n, 1)), n),
                window=128, q_pos0=250, k_pos0=0)
    rows0, _ = ref.visible_rows(p, 0, 0)
    assert rows0.tolist() == list(range(123, 251))


# --------------------------------------------------------------------------- layout and block map

def test_pad_layout_bits():
    rng = np.random.default_rng(16)
    k = rng.standard_normal((2, 27, 8)).astype(np.float16)
    v = rng.standard_normal((2, 27, 8)).astype(np.float16)
    valid = (rng.random((2, 27)) < 0.5).astype(np.uint8)
    kp, vp, vap = ref.pad_layout(k, v, valid, 27)
    assert kp.shape == (2, 32, 8) and vap.shape == (2, 32)
    assert kp.view(np.uint16)[:, :27].tobytes() == k.view(np.uint16).tobytes()
    assert (kp.view(np.uint16)[:, 27:] == 0).all() and (vp.view(np.uint16)[:, 27:] == 0).all()
    assert (vap[:, :27] == valid).all() and (vap[:, 27:] == 0).all()
    kp2, _, vap2 = ref.pad_layout(k[:, :, :], v, None, 32 - 5)
    assert (vap2[:, :27] == 1).all()
    # already aligned: identity
    k64 = rng.standard_normal((1, 64, 4)).astype(np.float32)
    kp3, _, _ = ref.pad_layout(k64, k64, None, 64)
    assert kp3.tobytes() == k64.tobytes()


@pytest.mark.parametrize("case", range(len(TINY_CASES)))
@pytest.mark.parametrize("bq", [1, 2, 3])
def test_blockmap_equals_brute_force(case, bq):
    rng = np.random.default_rng(2000 + case)
    p = _rand_problem(rng, **TINY_CASES[case])
    assert ref.blockmap(p, bq).tolist() == brute.blockmap(p, bq)


def _census_by_intervals(tokens, n0, window, q_pos0, k_pos0, bq):
    """Counts of SKIP/PARTIAL/FULL for a causal-window raw region, from the
    visible interval of each token (no pair enumeration)."""
    nb = -(-n0 // 32)
    counts = [0, 0, 0]
    for qt in range(-(-tokens // bq)):
        toks = range(qt * bq, min(tokens, (qt + 1) * bq))
        for jb in range(nb):
            total = 0
            for t in toks:
                lo = max(q_pos0 + t - k_pos0 - window + 1, 32 * jb, 0)
                hi = min(q_pos0 + t - k_pos0, 32 * jb + 31, n0 - 1)
                total += max(0, hi - lo + 1)
            full = 32 * len(toks)
            counts[0 if total == 0 else (2 if total == full else 1)] += 1
    return counts


def _census(p, bq):
    m = ref.blockmap(p, bq)
    return [int((m == s).sum()) for s in (0, 1, 2)]


def _shape_only(tokens, n0, window, q_pos0, k_pos0, n1=0, indexed=False):
    q = np.zeros((1, tokens, 1, 1))
    r1 = Region(np.zeros((1, n1, 1)), np.zeros((1, n1, 1)), n1) if n1 else None
    idx = np.zeros((1, tokens, 1), np.int64) if indexed else None
    z = np.zeros((1, n0, 1))
    return Problem(q, 1.0, Region(z, z, n0), window, q_pos0, k_pos0, r1, idx)


@pytest.mark.parametrize("bq", [1, 16])
def test_blockmap_census_prefill_raw_swa(bq):
    p = _shape_only(2048, 2048, 128, 0, 0)
    want = _census_by_intervals(2048, 2048, 128, 0, 0, bq)
    assert _census(p, bq) == want
    if bq == 16:
        assert want == [7572, 248, 372]


@pytest.mark.parametrize("bq", [1, 16])
def test_blockmap_census_prefill_ratio4_raw_region(bq):
    p = _shape_only(2048, 2175, 128, 30720, 30593, n1=7680, indexed=True)
    want = _census_by_intervals(2048, 2175, 128, 30720, 30593, bq)
    assert _census(p, bq) == want
    assert ref.blockmap(p, bq).shape[2] == 68       # indexed rows are not in the map
    if bq == 16:
        assert want == [8064, 256, 384]


def test_blockmap_decode_closed_forms():
    # full 128-row ring, no mask: every block FULL
    p = _shape_only(1, 128, 0, 0, 0)
    assert ref.blockmap(p, 1).tolist() == [[[2, 2, 2, 2]]]
    # ring + 256 compressed slots, the last r invalid: 11 FULL blocks then 1 PARTIAL
    for r in (1, 17, 31):
        valid1 = (np.arange(256) < 256 - r).astype(np.uint8)[None]
        z = np.zeros((1, 256, 1))
        p = Problem(np.zeros((1, 1, 1, 1)), 1.0, Region(np.zeros((1, 128, 1)), np.zeros((1, 128, 1)), 128),
                    r1=Region(z, z, 256, valid1))
        assert ref.blockmap(p, 1).tolist() == [[[2] * 11 + [1]]]
    # 27 rows padded to 32: one PARTIAL block
    p = _shape_only(1, 27, 0, 0, 0)
    assert ref.blockmap(p, 1).tolist() == [[[1]]]


# --------------------------------------------------------------------------- constants from the pages

def _constants():
    with open(os.path.join(GOLDEN, "ds4_constants.json")) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


def test_workloads_use_the_pages_shapes():
    c = _constants()
    assert (wl.N_HEAD, wl.HEAD_DIM, wl.WINDOW, wl.TOPK, wl.PREFILL_CHUNK) == \
        (c["n_head"], c["head_dim"], c["swa_window"], c["indexer_topk"], c["prefill_chunk"])
    w = wl.decode_ratio128(batch=1)
    assert w.r1.n_rows == c["context_tokens"] // c["odd_layer_ratio"]
    assert w.q.shape == (1, 1, c["n_head"], c["head_dim"]) and w.r0.k.shape[0] == 1


def test_decode_rows_per_token_over_the_layer_schedule():
    """Rows one decode token attends across the 43 layers at a 32K context,
    counted through the oracle's visibility rules: 2 raw layers x 128,
    21 ratio-4 layers x (128 + 512), 20 ratio-128 layers x (128 + 256)."""
    c = _constants()
    ctx = c["context_tokens"]
    pos = ctx - 1
    total = 0
    for layer in range(c["n_layers"]):
        n0 = c["swa_window"]
        raw = Region(np.zeros((1, n0, 1)), np.zeros((1, n0, 1)), n0)
        q = np.zeros((1, 1, 1, 1))
        if layer in c["raw_only_layers"]:
            p = Problem(q, 1.0, raw, window=c["swa_window"], q_pos0=pos, k_pos0=pos - n0 + 1)
        elif layer % 2 == 0:
            n1 = ctx // c["even_layer_ratio"]
            comp = Region(np.zeros((1, n1, 1)), np.zeros((1, n1, 1)), n1)
            idx = np.arange(0, n1, n1 // c["indexer_topk"])[None, None, :c["indexer_topk"]]
            p = Problem(q, 1.0, raw, window=c["swa_window"], q_pos0=pos, k_pos0=pos - n0 + 1,
                        r1=comp, r1_index=idx)
        else:
            n1 = ctx // c["odd_layer_ratio"]
            comp = Region(np.zeros((1, n1, 1)), np.zeros((1, n1, 1)), n1)
            p = Problem(q, 1.0, raw, window=c["swa_window"], q_pos0=pos, k_pos0=pos - n0 + 1, r1=comp)
        r0, r1 = ref.visible_rows(p, 0, 0)
        total += len(r0) + len(r1)
    assert total == 2 * 128 + 21 * (128 + 512) + 20 * (128 + 256) == 21376
