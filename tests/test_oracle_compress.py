"""Pins of the compressor-pooling oracle (``oracle.compress``) against things other
than itself (CPU only):

* brute force: a pure-Python loop (``math.exp``, lists) over the definition, per
  group and element, on tiny inputs;
* closed forms: ratio 1 is the identity; equal scores in a group give the group's
  mean; one score far above the others gives that row exactly; a per-row score
  (the same for every element) gives the textbook softmax-weighted row average;
* invariants: a per-element shift of a group's scores, and a permutation of the
  rows inside a group (with their scores), leave the pooled row unchanged; a
  pooled element lies between the group's smallest and largest value;
* streaming: feeding the same rows in chunks of any sizes through the rolling
  state gives the same pooled rows, and the same final state, as one call;
* the ratios of the pages' layers (4 and 128) and their group counts for a
  2048-row chunk;
* planted mistakes (a softmax over elements instead of rows, a missing
  normalisation, weights without the max shift overflowing, a state that keeps
  the leading instead of the trailing rows) are each caught by one of the pins.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import compress as cp

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ds4_constants.json")


def _brute(kv, score, ratio):
    n, d = len(kv), len(kv[0])
    out = []
    for c in range(n // ratio):
        row = []
        for e in range(d):
            ss = [float(score[c * ratio + i][e]) for i in range(ratio)]
            mx = max(ss)
            ws = [math.exp(x - mx) for x in ss]
            tot = sum(ws)
            row.append(sum(w * float(kv[c * ratio + i][e]) for i, w in enumerate(ws)) / tot)
        out.append(row)
    return out


def _inputs(seed, n, d, scale=1.0):
    rng = np.random.default_rng(seed)
    kv = rng.standard_normal((n, d)).astype(np.float16)
    sc = (rng.standard_normal((n, d)) * scale).astype(np.float32)
    return kv, sc


@pytest.mark.parametrize("seed,n,d,ratio", [(0, 8, 4, 4), (1, 12, 3, 3), (2, 9, 5, 2), (3, 7, 6, 4),
                                            (4, 16, 2, 8), (5, 5, 3, 1)])
def test_pool_matches_brute_force(seed, n, d, ratio):
    kv, sc = _inputs(seed, n, d, scale=3.0)
    got = cp.pool_groups(kv, sc, ratio)
    want = np.array(_brute(kv.tolist(), sc.tolist(), ratio), dtype=np.float64).reshape(-1, d)
    assert got.shape == (n // ratio, d)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_ratio_one_is_identity():
    kv, sc = _inputs(10, 9, 7)
    np.testing.assert_array_equal(cp.pool_groups(kv, sc, 1), kv.astype(np.float64))


def test_equal_scores_give_the_mean():
    kv, _ = _inputs(11, 12, 5)
    sc = np.full((12, 5), 0.75, dtype=np.float32)
    got = cp.pool_groups(kv, sc, 4)
    want = kv.astype(np.float64).reshape(3, 4, 5).mean(axis=1)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_dominant_score_selects_its_row():
    kv, sc = _inputs(12, 8, 6)
    sc[:] = 0.0
    sc[2, :] = 1000.0          # group 0 -> row 2
    sc[7, :3] = 1000.0         # group 1 -> row 7 for elements 0..2, mean of rows 4..7 for the rest
    sc[5, 3:] = 1000.0         # ... and row 5 for elements 3..5
    got = cp.pool_groups(kv, sc, 4)
    k = kv.astype(np.float64)
    np.testing.assert_array_equal(got[0], k[2])
    np.testing.assert_array_equal(got[1, :3], k[7, :3])
    np.testing.assert_array_equal(got[1, 3:], k[5, 3:])


def test_per_row_scores_are_the_weighted_row_average():
    kv, _ = _inputs(13, 8, 4)
    w = np.array([0.1, -2.0, 1.5, 0.3, 2.0, 2.0, -1.0, 0.0])
    sc = np.repeat(w[:, None], 4, axis=1).astype(np.float32)
    got = cp.pool_groups(kv, sc, 4)
    k = kv.astype(np.float64)
    for c in range(2):
        e = np.exp(w[4 * c:4 * c + 4].astype(np.float32).astype(np.float64))
        p = e / e.sum()
        np.testing.assert_allclose(got[c], (p[:, None] * k[4 * c:4 * c + 4]).sum(axis=0), rtol=0, atol=1e-14)


def test_score_shift_and_row_permutation_invariance():
    kv, sc = _inputs(14, 16, 6, scale=2.0)
    base = cp.pool_groups(kv, sc, 8)
    shift = np.random.default_rng(15).standard_normal((1, 6)) * 5.0
    sc2 = sc.astype(np.float64).copy()
    sc2[:8] += shift           # a per-element shift of group 0's scores
    np.testing.assert_allclose(cp.pool_groups(kv, sc2, 8), base, rtol=0, atol=1e-12)
    perm = np.concatenate([np.random.default_rng(16).permutation(8), 8 + np.random.default_rng(17).permutation(8)])
    np.testing.assert_allclose(cp.pool_groups(kv[perm], sc[perm], 8), base, rtol=0, atol=1e-12)


def test_pooled_values_lie_between_the_group_extremes():
    kv, sc = _inputs(18, 128 * 3, 16, scale=4.0)
    got = cp.pool_groups(kv, sc, 128)
    g = kv.astype(np.float64).reshape(3, 128, 16)
    assert np.all(got >= g.min(axis=1) - 1e-12) and np.all(got <= g.max(axis=1) + 1e-12)


@pytest.mark.parametrize("ratio,chunks", [(4, [3, 1, 5, 0, 7, 2]), (4, [1] * 13), (8, [5, 11, 2, 6]),
                                          (128, [100, 27, 1, 300, 5])])
def test_streaming_matches_one_call(ratio, chunks):
    n = sum(chunks)
    kv, sc = _inputs(20 + ratio, n, 5)
    whole, st_kv, st_sc = cp.compress_step(kv[:0], sc[:0], kv, sc, ratio)
    pooled = []
    s_kv, s_sc = kv[:0], sc[:0]
    at = 0
    for c in chunks:
        p, s_kv, s_sc = cp.compress_step(s_kv, s_sc, kv[at:at + c], sc[at:at + c], ratio)
        pooled.append(p)
        at += c
        assert s_kv.shape[0] == at % ratio
    np.testing.assert_array_equal(np.concatenate(pooled, axis=0), whole)
    np.testing.assert_array_equal(s_kv, st_kv)
    np.testing.assert_array_equal(s_sc, st_sc)
    # the state holds the trailing rows of the stream
    np.testing.assert_array_equal(s_kv, kv[n - n % ratio:])


def test_state_must_hold_fewer_than_ratio_rows():
    kv, sc = _inputs(30, 4, 3)
    with pytest.raises(ValueError):
        cp.compress_step(kv, sc, kv[:0], sc[:0], 4)


def test_pages_ratios_and_chunk_group_counts():
    g = json.load(open(GOLDEN))
    for key, groups in (("even_layer_ratio", 512), ("odd_layer_ratio", 16)):
        ratio = g[key]["value"]
        kv, sc = _inputs(40, 2048, 2)
        assert cp.pool_groups(kv, sc, ratio).shape == (groups, 2)


# ---- planted mistakes: each must fail one of the pins above -------------------------

def _mutant_softmax_over_elements(kv, score, ratio):
    kv = np.asarray(kv, np.float64)
    s = np.asarray(score, np.float64)
    out = []
    for c in range(kv.shape[0] // ratio):
        g_s = s[c * ratio:(c + 1) * ratio]
        w = np.exp(g_s - g_s.max(axis=1, keepdims=True))
        w = w / w.sum(axis=1, keepdims=True)
        out.append((w * kv[c * ratio:(c + 1) * ratio]).sum(axis=0))
    return np.array(out).reshape(-1, kv.shape[1])


def _mutant_unnormalised(kv, score, ratio):
    kv = np.asarray(kv, np.float64)
    s = np.asarray(score, np.float64)
    out = []
    for c in range(kv.shape[0] // ratio):
        g_s = s[c * ratio:(c + 1) * ratio]
        w = np.exp(g_s - g_s.max(axis=0))
        out.append((w * kv[c * ratio:(c + 1) * ratio]).sum(axis=0))
    return np.array(out).reshape(-1, kv.shape[1])


def _mutant_no_shift(kv, score, ratio):
    kv = np.asarray(kv, np.float64)
    s = np.asarray(score, np.float64)
    out = []
    with np.errstate(over="ignore", invalid="ignore"):
        for c in range(kv.shape[0] // ratio):
            w = np.exp(s[c * ratio:(c + 1) * ratio])
            out.append((w * kv[c * ratio:(c + 1) * ratio]).sum(axis=0) / w.sum(axis=0))
    return np.array(out).reshape(-1, kv.shape[1])


@pytest.mark.parametrize("mutant", [_mutant_softmax_over_elements, _mutant_unnormalised, _mutant_no_shift])
def test_planted_pooling_mistakes_are_caught(mutant, monkeypatch):
    monkeypatch.setattr(cp, "pool_groups", mutant)
    failures = 0
    for check in (lambda: test_pool_matches_brute_force(0, 8, 4, 4),
                  test_equal_scores_give_the_mean,
                  test_dominant_score_selects_its_row):
        try:
            check()
        except AssertionError:
            failures += 1
    assert failures >= 1


def test_planted_state_mistake_is_caught(monkeypatch):
    real = cp.compress_step

    def leading_state(state_kv, state_score, kv_new, score_new, ratio):
        pooled, s_kv, s_sc = real(state_kv, state_score, kv_new, score_new, ratio)
        kv = np.concatenate([state_kv, kv_new], axis=0)
        sc = np.concatenate([state_score, score_new], axis=0)
        m = s_kv.shape[0]
        return pooled, kv[:m].copy(), sc[:m].copy()

    monkeypatch.setattr(cp, "compress_step", leading_state)
    with pytest.raises(AssertionError):
        test_streaming_matches_one_call(4, [3, 1, 5, 0, 7, 2])
