"""Pins of the top-k selection oracle (``oracle.topk``) against things other than
itself (CPU only):

* the defining property checked pair by pair on small rows: every selected index
  beats every unselected one under (larger key, then lower index), and exactly
  min(k, n) are selected -- no sort involved;
* Python's own float comparison on rows without signed zeros or NaNs (the key
  transform must order them the same way);
* closed forms: descending scores select the first k, ascending the last k,
  all-equal the first k; k >= n selects everything and pads with -1;
* the signed-zero / infinity / NaN order the reading fixes;
* order invariance: an exact positive scaling of the scores changes nothing;
* planted mistakes (descending tie-break, reversed order, a dropped sign flip in
  the key, an unsorted result) are each caught by one of the pins.
"""

import math
import struct

import numpy as np
import pytest

from oracle import topk as tk


def _beats(ka, ia, kb, ib):
    return ka > kb or (ka == kb and ia < ib)


def _check_property(scores, k, out):
    n = scores.shape[0]
    keys = [int(x) for x in tk.order_key(scores)]
    m = min(k, n)
    sel = [int(i) for i in out if i >= 0]
    assert len(sel) == m and len(set(sel)) == m
    assert all(int(i) == -1 for i in out[m:])
    assert sel == sorted(sel)
    rest = set(range(n)) - set(sel)
    for i in sel:
        for j in rest:
            assert _beats(keys[i], i, keys[j], j), (i, j)


@pytest.mark.parametrize("seed", range(12))
def test_selection_property_on_small_rows(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 40))
    k = int(rng.integers(1, 48))
    # coarse values so that ties are common
    scores = (rng.integers(-6, 7, size=n) * 0.5).astype(np.float32)
    out = tk.topk(scores[None, :], k)[0]
    _check_property(scores, k, out)


@pytest.mark.parametrize("seed", range(6))
def test_key_order_matches_float_comparison(seed):
    rng = np.random.default_rng(100 + seed)
    x = (rng.standard_normal(200) * 10.0 ** rng.integers(-3, 4, 200)).astype(np.float32)
    x = x[x != 0]
    keys = tk.order_key(x)
    for _ in range(400):
        a, b = rng.integers(0, x.size, 2)
        assert (keys[a] > keys[b]) == (float(x[a]) > float(x[b]))
        assert (keys[a] == keys[b]) == (float(x[a]) == float(x[b]))


def test_closed_forms():
    n, k = 50, 7
    desc = np.linspace(3, -3, n, dtype=np.float32)
    asc = desc[::-1].copy()
    same = np.full(n, 1.25, np.float32)
    out = tk.topk(np.stack([desc, asc, same]), k)
    assert out[0].tolist() == list(range(k))
    assert out[1].tolist() == list(range(n - k, n))
    assert out[2].tolist() == list(range(k))
    short = tk.topk(np.array([[0.5, -1.0, 2.0]], np.float32), 5)[0]
    assert short.tolist() == [0, 1, 2, -1, -1]
    assert tk.topk(np.zeros((2, 0), np.float32), 3).tolist() == [[-1, -1, -1]] * 2


def _f32(bits):
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def test_signed_zero_infinity_and_nan_order():
    pos_nan, neg_nan = _f32(0x7FC00000), _f32(0xFFC00000)
    row = np.array([-0.0, 0.0, -math.inf, math.inf, pos_nan, neg_nan, 1.0], np.float32)
    assert tk.topk(row[None], 1)[0].tolist() == [4]            # +NaN ranks highest
    assert tk.topk(row[None], 2)[0].tolist() == [3, 4]          # then +inf
    assert tk.topk(row[None], 4)[0].tolist() == [1, 3, 4, 6]    # then 1.0, then +0
    assert tk.topk(row[None], 5)[0].tolist() == [0, 1, 3, 4, 6]  # -0 ranks below +0
    assert tk.topk(row[None], 6)[0].tolist() == [0, 1, 2, 3, 4, 6]  # -NaN ranks lowest


def test_positive_scaling_changes_nothing():
    rng = np.random.default_rng(7)
    s = rng.standard_normal((5, 300)).astype(np.float32)
    t = s * np.float32(4.0)      # exact in float32: the order, ties included, is kept
    assert np.array_equal(tk.topk(s, 40), tk.topk(t, 40))


# --------------------------------------------------------------------------- planted mistakes

def _pins():
    return [lambda s=s: test_selection_property_on_small_rows(s) for s in range(12)] + [
        lambda s=s: test_key_order_matches_float_comparison(s) for s in range(2)] + [
        test_closed_forms, test_signed_zero_infinity_and_nan_order,
        test_positive_scaling_changes_nothing]


def _some_pin_fails():
    for pin in _pins():
        try:
            pin()
        except AssertionError:
            return True
    return False


def _higher_index_wins(monkeypatch):
    def topk(scores, k):
        s = np.asarray(scores, np.float32)
        rows, n = s.shape
        out = np.full((rows, k), -1, np.int32)
        m = min(k, n)
        for r in range(rows):
            key = tk.order_key(s[r]).astype(np.int64)
            order = np.lexsort((-np.arange(n), -key))
            out[r, :m] = np.sort(order[:m])
        return out
    monkeypatch.setattr(tk, "topk", topk)


def _smallest_instead(monkeypatch):
    orig = tk.topk
    monkeypatch.setattr(tk, "topk", lambda s, k: orig(-np.asarray(s, np.float32), k))


def _no_sign_flip(monkeypatch):
    monkeypatch.setattr(tk, "order_key",
                        lambda x: np.ascontiguousarray(x, np.float32).view(np.uint32).copy())


def _unsorted_result(monkeypatch):
    orig = tk.topk
    monkeypatch.setattr(tk, "topk", lambda s, k: orig(s, k)[:, ::-1].copy())


@pytest.mark.parametrize("plant", [_higher_index_wins, _smallest_instead, _no_sign_flip,
                                   _unsorted_result], ids=lambda f: f.__name__.strip("_"))
def test_planted_mistake_is_caught(plant, monkeypatch):
    assert not _some_pin_fails()
    plant(monkeypatch)
    assert _some_pin_fails()
