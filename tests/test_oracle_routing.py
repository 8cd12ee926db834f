"""Pins for the oracle's routing (vLLM "mega_moe" page, top_k_pick).

Pinned against: brute force on tiny inputs (selection by counting who beats
whom, independent of any sort), the zero-input closed form, hand-worked
examples, a forced-selection bias step, permutation equivariance, and the
normalisation identity.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import f32, route

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _beats(key, a, b):
    return key[a] > key[b] or (key[a] == key[b] and a < b)


@pytest.mark.parametrize("seed", range(40))
def test_bruteforce_selection(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(2, 13))
    k = int(rng.integers(1, E + 1))
    # few distinct values so that ties in the key are common
    logits = rng.choice([-1.0, 0.0, 0.5, 2.0], size=(3, E)).astype(np.float32)
    bias = rng.choice([0.0, 0.0, 0.125, -0.25], size=E).astype(np.float32)
    ids, w, s = route(logits, bias, k, 2.5)
    for t in range(3):
        z = [float(v) for v in logits[t]]
        sc = [float(np.float32(1.0 / (1.0 + math.exp(-v)))) for v in z]
        key = [float(np.float32(np.float32(a) + np.float32(b))) for a, b in zip(sc, bias)]
        chosen = {e for e in range(E) if sum(_beats(key, o, e) for o in range(E) if o != e) < k}
        assert set(ids[t].tolist()) == chosen
        # pick order: each id beats every later id
        for i in range(k - 1):
            assert _beats(key, ids[t, i], ids[t, i + 1])


def test_zero_inputs_closed_form():
    doc = json.load(open(os.path.join(GOLDEN, "routing_zero_inputs.json")))
    for c in doc["cases"]:
        E, k = c["experts"], c["top_k"]
        ids, w, _ = route(np.zeros((2, E), np.float32), np.zeros(E, np.float32), k, c["routed_scale"])
        assert ids.tolist() == [c["ids"]] * 2
        assert np.all(w == c["weight"])


def test_worked_examples():
    doc = json.load(open(os.path.join(GOLDEN, "routing_worked_example.json")))
    for c in doc["cases"]:
        logits = np.array([c["logits"]], np.float32)
        ids, w, _ = route(logits, np.array(c["bias"], np.float32), c["top_k"], c["routed_scale"])
        assert ids[0].tolist() == c["ids"]
        np.testing.assert_allclose(w[0], c["weights"], rtol=c["weights_rel_tol"])


def test_bias_selects_but_does_not_weigh():
    rng = np.random.default_rng(5)
    E, k = 32, 4
    logits = rng.standard_normal((1, E)).astype(np.float32)
    bias = np.zeros(E, np.float32)
    forced = [3, 17, 29, 30]
    bias[forced] = 10.0
    ids, w, s = route(logits, bias, k, 2.5)
    assert sorted(ids[0].tolist()) == forced
    sel = s[0, ids[0]]
    np.testing.assert_allclose(w[0], sel / sel.sum() * 2.5, rtol=1e-6)
    # the picks are ordered by the biased key, which here is the score order
    assert np.all(np.diff(sel) <= 0)


def test_permutation_equivariance():
    rng = np.random.default_rng(6)
    E, k = 64, 6
    logits = rng.standard_normal((4, E)).astype(np.float32) * 2
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    ids, w, _ = route(logits, bias, k, 2.5)
    perm = rng.permutation(E)
    inv = np.argsort(perm)
    ids_p, w_p, _ = route(logits[:, perm], bias[perm], k, 2.5)
    assert np.array_equal(perm[ids_p], ids)
    assert np.array_equal(w_p, w)
    del inv


def test_weights_sum_to_scale():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((16, 256)).astype(np.float32) * 2
    bias = (rng.standard_normal(256) * 0.1).astype(np.float32)
    _, w, _ = route(logits, bias, 8, 2.5)
    np.testing.assert_allclose(w.sum(axis=1), 2.5, rtol=1e-6)


def test_sigmoid_points():
    s = oracle.moe.sigmoid_f32(np.array([0.0, 50.0, -200.0, 1.0, -1.0]))
    assert s[0] == 0.5 and s[1] == 1.0 and s[2] == f32(np.exp(-200.0))
    assert abs(s[3] + s[4] - 1.0) <= 2.0**-24


def test_pins_catch_tie_break_mistake(monkeypatch):
    """Ties going to the higher index (a plausible slip) fails a pin."""
    real = oracle.moe.route

    def wrong(logits, bias, top_k, scale):
        E = np.asarray(logits).shape[1]
        rev = np.arange(E)[::-1]
        ids, w, s = real(np.asarray(logits)[:, rev], np.asarray(bias)[rev], top_k, scale)
        return rev[ids].astype(np.int32), w, s[:, rev]

    monkeypatch.setitem(globals(), "route", wrong)
    with pytest.raises(AssertionError):
        test_worked_examples()


def test_pins_catch_biased_weights(monkeypatch):
    """Normalising the biased keys instead of the scores fails a pin."""
    def wrong(logits, bias, top_k, scale):
        ids, w, s = oracle.moe.route(logits, bias, top_k, scale)
        key = f32(s + np.asarray(bias, np.float64)[None, :])
        kw = np.take_along_axis(key, ids.astype(np.int64), 1)
        return ids, f32(kw / kw.sum(1, keepdims=True) * scale), s

    monkeypatch.setitem(globals(), "route", wrong)
    with pytest.raises(AssertionError):
        test_worked_examples()
