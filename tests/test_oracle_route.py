"""Pins of the oracle's router epilogue (no GPU): brute-force ids, the closed
form sigma_i / sum_j sigma_j, the printed sum invariant, the all-negative
rows that produced NaN in the plain form, a dominating sink, and a mutation
(carrying the activated score instead of the raw logit) that must be caught.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import CONFIGS, make_batch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _closed_form(rows, ids, n_routed, n_sink, scale):
    """sigma_i / sum_j sigma_j in float64 via torch.sigmoid (a library
    routine, different formula from the oracle's log-sigmoid/LSE)."""
    x = torch.from_numpy(np.asarray(rows, np.float32).astype(np.float64))
    sel = torch.gather(x[:, :n_routed], 1, torch.from_numpy(ids))
    act = torch.cat([sel, x[:, n_routed:n_routed + n_sink]], 1)
    s = torch.sigmoid(act)
    w = s / s.sum(1, keepdim=True) * scale
    k = ids.shape[1]
    return w[:, :k].numpy(), w[:, k:].numpy()


def _brute_ids(rows, n_routed, k):
    return np.array([sorted(range(n_routed), key=lambda i: (-float(r[i]), i))[:k]
                     for r in rows], dtype=np.int64)


@pytest.mark.parametrize("T", [1, 37, 512])
def test_route_ids_and_weights_c5_rows(T):
    spec = CONFIGS["ep_lora_258"]
    lg = make_batch(spec, None, T).logits.numpy()
    ids, w, sw = O.route(lg, 256, 2, 8)
    assert np.array_equal(ids, _brute_ids(lg, 256, 8))
    cw, csw = _closed_form(lg, ids, 256, 2, 1.0)
    assert np.all(np.isfinite(w)) and np.all(np.isfinite(sw))
    np.testing.assert_allclose(w, cw, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(sw, csw, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(w.sum(1) + sw.sum(1), 1.0, rtol=0, atol=1e-12)


def test_route_tie_rows_resolve_to_lower_index():
    row = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, 2.0, 0.0, 3.0]], np.float32)
    ids, _, _ = O.route(row, 8, 0, 6)
    assert ids[0].tolist() == [1, 2, 4, 7, 3, 5]
    # 4 distinct values over 256 columns (the page's tie case)
    rng = np.random.default_rng(6)
    rows = rng.choice(np.array([-1.5, 0.25, 0.75, 2.0], np.float32), (64, 258))
    ids, w, sw = O.route(rows, 256, 2, 8)
    assert np.array_equal(ids, _brute_ids(rows, 256, 8))


def test_route_all_negative_rows_are_finite_and_normalised():
    # all K + S active logits below the fp32 sigmoid flush point (-104): the
    # plain sigma/sum(sigma) form is 0/0 in fp32 there
    for base in (-40.0, -90.0, -110.5, -200.0, -1000.0):
        rng = np.random.default_rng(int(-base))
        rows = (base + rng.standard_normal((16, 258))).astype(np.float32)
        ids, w, sw = O.route(rows, 256, 2, 8)
        assert np.all(np.isfinite(w)) and np.all(np.isfinite(sw))
        np.testing.assert_allclose(w.sum(1) + sw.sum(1), 1.0, atol=1e-12)
        if base > -700:                  # float64 sigmoid still representable
            cw, csw = _closed_form(rows, ids, 256, 2, 1.0)
            np.testing.assert_allclose(w, cw, rtol=1e-10)
    # the fp32 plain form really is NaN there (what the page fixed)
    x = torch.full((1, 10), -110.0, dtype=torch.float32)
    s = torch.sigmoid(x)
    assert torch.isnan(s / s.sum()).all()


def test_route_dominating_sink():
    rows = np.random.default_rng(7).standard_normal((8, 258)).astype(np.float32)
    rows[:, :256] -= 8.0
    rows[:, 256:] += 30.0
    _, w, sw = O.route(rows, 256, 2, 8)
    # sigmoid saturates at 1: each sink takes ~1/2, routed slots ~sigma(-6)/2
    assert np.all(sw.sum(1) > 0.95) and np.all(w < 0.01)
    np.testing.assert_allclose(w.sum(1) + sw.sum(1), 1.0, atol=1e-12)


def test_route_sum_invariant_printed_value():
    g = json.load(open(os.path.join(GOLD, "route_sum_invariant.json")))
    rows = np.random.default_rng(8).standard_normal((512, 258)).astype(np.float32)
    _, w, sw = O.route(rows, 256, 2, 6, g["route_scale"], g["global_scale"])
    tot = w.sum(1) + sw.sum(1)
    assert np.all(tot >= g["band_lo"]) and np.all(tot <= g["band_hi"])
    np.testing.assert_allclose(tot, g["expected_sum"], atol=2e-6)


def test_route_zero_sinks_and_T0():
    rows = np.random.default_rng(9).standard_normal((5, 64)).astype(np.float32)
    ids, w, sw = O.route(rows, 64, 0, 8)
    assert sw.shape == (5, 0)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-12)
    ids0, w0, sw0 = O.route(np.zeros((0, 64), np.float32), 64, 0, 8)
    assert ids0.shape == (0, 8) and w0.shape == (0, 8)


def test_mutation_activated_carry_is_caught(monkeypatch):
    """Planting the page's 'wrong carry' (sigmoid of the winner instead of
    its raw logit) in the oracle must break the closed-form pin, while the
    sum invariant alone still holds."""
    rows = np.random.default_rng(10).standard_normal((64, 258)).astype(np.float32)
    real_take = np.take_along_axis

    def carry_sigmoid(a, idx, axis):
        out = real_take(a, idx, axis)
        return 1.0 / (1.0 + np.exp(-out)) if out.shape[1] == 8 else out

    monkeypatch.setattr(O.np, "take_along_axis", carry_sigmoid)
    ids, w, sw = O.route(rows, 256, 2, 8)
    monkeypatch.undo()
    np.testing.assert_allclose(w.sum(1) + sw.sum(1), 1.0, atol=1e-12)
    cw, _ = _closed_form(rows, ids, 256, 2, 1.0)
    assert np.max(np.abs(w - cw)) > 1e-3
