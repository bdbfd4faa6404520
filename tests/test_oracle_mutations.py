"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in ``oracle.reference`` (a window edge off by one,
a dropped scale, scores taken against V instead of K, an ignored validity mask,
swapped status codes, a non-zero pad fill) and checks that at least one pin of
``tests/test_oracle.py`` then fails.  Nothing here touches the GPU path.
"""

import numpy as np
import pytest

from oracle import reference as ref
from tests import test_oracle as pins


def _all_pins():
    checks = []
    for case in range(len(pins.TINY_CASES)):
        checks.append(lambda c=case: pins.test_reference_equals_brute_force(c))
        for bq in (1, 2, 3):
            checks.append(lambda c=case, q=bq: pins.test_blockmap_equals_brute_force(c, q))
    checks += [
        pins.test_two_keys_logistic_closed_form,
        pins.test_single_visible_row_returns_that_row,
        pins.test_equal_keys_give_mean_of_visible_values,
        pins.test_window_keeps_exactly_128_rows_including_own,
        pins.test_pad_layout_bits,
        lambda: pins.test_blockmap_census_prefill_raw_swa(16),
        pins.test_blockmap_decode_closed_forms,
        pins.test_decode_rows_per_token_over_the_layer_schedule,
    ]
    return checks


def _some_pin_fails():
    for check in _all_pins():
        try:
            check()
        except AssertionError:
            return True
    return False


def _window_off_by_one(monkeypatch):
    orig = ref.region0_allowed

    def wrong(p, b, t, rows):
        if p.window > 0:
            q = ref.Problem(p.q, p.scale, p.r0, p.window + 1, p.q_pos0, p.k_pos0, p.r1, p.r1_index)
            return orig(q, b, t, rows)
        return orig(p, b, t, rows)

    monkeypatch.setattr(ref, "region0_allowed", wrong)


def _dropped_scale(monkeypatch):
    orig_init = ref._Widened.__init__

    def init(self, p):
        orig_init(self, p)
        self.scale = 1.0

    monkeypatch.setattr(ref._Widened, "__init__", init)


def _scores_against_v(monkeypatch):
    orig_init = ref._Widened.__init__

    def init(self, p):
        orig_init(self, p)
        self.k0 = self.v0
        if p.r1 is not None:
            self.k1 = self.v1

    monkeypatch.setattr(ref._Widened, "__init__", init)


def _ignored_validity(monkeypatch):
    orig = ref.region0_allowed

    def wrong(p, b, t, rows):
        q = ref.Problem(p.q, p.scale, ref.Region(p.r0.k, p.r0.v, p.r0.n_rows, None), p.window,
                        p.q_pos0, p.k_pos0, p.r1, p.r1_index)
        return orig(q, b, t, rows)

    monkeypatch.setattr(ref, "region0_allowed", wrong)


def _swapped_status(monkeypatch):
    orig = ref.blockmap

    def wrong(p, bq):
        m = orig(p, bq)
        out = m.copy()
        out[m == ref.FULL] = ref.PARTIAL
        out[m == ref.PARTIAL] = ref.FULL
        return out

    monkeypatch.setattr(ref, "blockmap", wrong)


def _nonzero_pad(monkeypatch):
    orig = ref.pad_layout

    def wrong(k, v, valid, n):
        kp, vp, vap = orig(k, v, valid, n)
        kp[:, n:] = 1
        return kp, vp, vap

    monkeypatch.setattr(ref, "pad_layout", wrong)


def _max_not_subtracted(monkeypatch):
    """A softmax with the max added instead of subtracted overflows or skews."""
    orig_exp = np.exp

    def token(p, w, b, t, want):
        rows0, rows1 = ref.visible_rows(p, b, t)
        keys = [w.k0[b, rows0]]
        vals = [w.v0[b, rows0]]
        if len(rows1):
            keys.append(w.k1[b, rows1])
            vals.append(w.v1[b, rows1])
        kmat = np.concatenate(keys, 0)
        vmat = np.concatenate(vals, 0)
        if kmat.shape[0] == 0:
            return np.zeros(p.q.shape[2:])
        s = w.scale * (w.q[b, t] @ kmat.T)
        e = orig_exp(-s)          # sign slip
        pr = e / e.sum(1, keepdims=True)
        return pr @ vmat

    monkeypatch.setattr(ref, "_token", token)


@pytest.mark.parametrize("plant", [_window_off_by_one, _dropped_scale, _scores_against_v,
                                   _ignored_validity, _swapped_status, _nonzero_pad,
                                   _max_not_subtracted],
                         ids=lambda f: f.__name__.strip("_"))
def test_planted_mistake_is_caught(plant, monkeypatch):
    assert not _some_pin_fails(), "pins must pass on the unmodified oracle"
    plant(monkeypatch)
    assert _some_pin_fails(), f"no pin caught: {plant.__name__}"
