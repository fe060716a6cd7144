"""Pins of the oracle's router GEMM, selection bias and packed output (no
GPU). Sources: "Enable and fuse the Inkling MoE gate epilogue on Intel XPU"
(sglang PR #36385), "3. Performance" and the router-epilogue commit message:
the ranking key is sigmoid(logits) + bias with the bias over the routed
columns only, the winner carries its raw logit, and the packed form is
(id << 16 | bf16 weight) read back with & 0xFFFF.

Each pin checks the oracle against something other than itself: exact sums
(math.fsum) and integer closed forms for the GEMM, a sort-based brute force
with torch's fp32 sigmoid for the ranking, hand-worked rows for saturation
and forced picks, the closed form sigma_i / sum_j sigma_j for the weights,
and hand-worked bit patterns for the packing.
"""
import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import CONFIGS, make_batch, make_gate


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _closed_form(raw_rows, ids, n_routed, n_sink, scale):
    x = torch.from_numpy(np.asarray(raw_rows, np.float32).astype(np.float64))
    sel = torch.gather(x[:, :n_routed], 1, torch.from_numpy(ids))
    act = torch.cat([sel, x[:, n_routed:n_routed + n_sink]], 1)
    s = torch.sigmoid(act)
    w = s / s.sum(1, keepdim=True) * scale
    k = ids.shape[1]
    return w[:, :k].numpy(), w[:, k:].numpy()


def _brute_biased_ids(rows, bias, n_routed, k):
    """Sort by (-key, column) with keys from torch's fp32 sigmoid plus the
    fp32 bias (a different routine and a sort instead of masked-max passes)."""
    x = torch.from_numpy(np.asarray(rows, np.float32)[:, :n_routed])
    key = (torch.sigmoid(x) + torch.from_numpy(np.asarray(bias, np.float32))).numpy()
    return np.array([sorted(range(n_routed), key=lambda i: (-float(r[i]), i))[:k]
                     for r in key], dtype=np.int64)


# ------------------------------------------------------------------ GEMM

def test_gate_logits_match_exact_sums():
    rng = np.random.default_rng(21)
    x = torch.from_numpy(rng.standard_normal((3, 64))).to(torch.bfloat16)
    wg = torch.from_numpy(rng.standard_normal((5, 64)) * 0.1).to(torch.bfloat16)
    lg = O.gate_logits(_bits(x), _bits(wg))
    xf, wf = x.double().numpy(), wg.double().numpy()
    for t in range(3):
        for c in range(5):
            exact = math.fsum(float(xf[t, h]) * float(wf[c, h]) for h in range(64))
            assert abs(lg[t, c] - exact) <= 1e-15 * max(1.0, abs(exact))


def test_gate_logits_integer_closed_form():
    # x[t, h] = t + 1, Wg[c, h] = c - 2 (small integers, exact in bf16):
    # logit = H (t + 1)(c - 2)
    H = 96
    x = torch.tensor([[t + 1.0] * H for t in range(4)]).to(torch.bfloat16)
    wg = torch.tensor([[c - 2.0] * H for c in range(7)]).to(torch.bfloat16)
    lg = O.gate_logits(_bits(x), _bits(wg))
    want = np.array([[H * (t + 1) * (c - 2) for c in range(7)] for t in range(4)], float)
    assert np.array_equal(lg, want)
    # transposed operand would give a wrong shape / values
    assert lg.shape == (4, 7)


def test_gate_route_rounds_the_gate_row_to_fp32_once():
    spec = CONFIGS["ep_lora_258"]
    gate = make_gate(spec)
    x = make_batch(spec, None, 6).x
    lg, ids, w, sw = O.gate_route(_bits(x), _bits(gate.wg), 256, 2, 8)
    exact = O.gate_logits(_bits(x), _bits(gate.wg))
    assert lg.dtype == np.float32
    assert np.array_equal(lg, exact.astype(np.float32))
    rid, rw, rsw = O.route(lg, 256, 2, 8)
    assert np.array_equal(ids, rid)
    np.testing.assert_array_equal(w, rw)


# ------------------------------------------------------- selection bias

@pytest.mark.parametrize("T", [1, 37, 200])
def test_biased_ids_match_sort_brute_force(T):
    spec = CONFIGS["ep_lora_258"]
    gate = make_gate(spec)
    rng = np.random.default_rng(T)
    rows = rng.standard_normal((T, 258)).astype(np.float32)
    ids, w, sw = O.route(rows, 256, 2, 8, sel_bias=gate.bias.numpy())
    assert np.array_equal(ids, _brute_biased_ids(rows, gate.bias.numpy(), 256, 8))
    # the bias changes the selected set of some rows but not of all
    plain, _, _ = O.route(rows, 256, 2, 8)
    if T >= 37:
        differ = np.array([set(a) != set(b) for a, b in zip(plain, ids)])
        assert 0 < differ.sum() < T


def test_biased_weights_carry_raw_logits():
    rng = np.random.default_rng(22)
    rows = rng.standard_normal((64, 258)).astype(np.float32)
    bias = (rng.random(256) * 0.4 - 0.2).astype(np.float32)
    ids, w, sw = O.route(rows, 256, 2, 8, 2.6, 4.0, sel_bias=bias)
    cw, csw = _closed_form(rows, ids, 256, 2, 2.6 * 4.0)
    np.testing.assert_allclose(w, cw, rtol=1e-6)
    np.testing.assert_allclose(sw, csw, rtol=1e-6)
    np.testing.assert_allclose(w.sum(1) + sw.sum(1), 10.4, rtol=1e-6)


def test_mutation_key_carry_is_caught(monkeypatch):
    """Carrying the ranking key (sigmoid + bias) out of the loop instead of
    the raw logit keeps the sum invariant but breaks the closed form."""
    rng = np.random.default_rng(23)
    rows = rng.standard_normal((64, 258)).astype(np.float32)
    bias = (rng.random(256) * 0.4 - 0.2).astype(np.float32)
    monkeypatch.setattr(O, "_carry", lambda raw, keys: keys)
    ids, w, sw = O.route(rows, 256, 2, 8, sel_bias=bias)
    monkeypatch.undo()
    np.testing.assert_allclose(w.sum(1) + sw.sum(1), 1.0, atol=1e-12)
    cw, _ = _closed_form(rows, ids, 256, 2, 1.0)
    assert np.max(np.abs(w - cw)) > 1e-3


def test_bias_forces_and_excludes_columns():
    row = np.zeros((1, 12), np.float32)
    row[0, :10] = [0.1, 0.9, 0.3, 2.5, -1.0, 0.5, 0.2, 0.8, -0.5, 0.0]
    row[0, 10:] = [0.4, -0.3]                       # two sinks
    bias = np.zeros(10, np.float32)
    bias[4] = 1.0                                   # lowest logit, forced first
    bias[3] = -1.0                                  # highest logit, pushed out
    ids, w, sw = O.route(row, 10, 2, 3, sel_bias=bias)
    # keys: col 4 sigma(-1)+1 = 1.269; col 1 sigma(0.9) = 0.711;
    # col 7 sigma(0.8) = 0.690; col 3 sigma(2.5)-1 = -0.076
    assert ids[0].tolist() == [4, 1, 7]
    s = 1.0 / (1.0 + np.exp(-np.array([-1.0, 0.9, 0.8, 0.4, -0.3])))
    np.testing.assert_allclose(np.concatenate([w[0], sw[0]]), s / s.sum(), rtol=1e-6)


def test_saturated_sigmoid_keys_tie_and_go_to_lower_column():
    # fp32 sigmoid is exactly 1 for these logits, so with zero bias the keys
    # tie and the lower column wins, unlike a ranking on the raw logit
    row = np.full((1, 24), -3.0, np.float32)
    row[0, 3], row[0, 9], row[0, 20] = 30.0, 25.0, 40.0
    ids, _, _ = O.route(row, 24, 0, 3, sel_bias=np.zeros(24, np.float32))
    assert ids[0].tolist() == [3, 9, 20]
    raw_ids, _, _ = O.route(row, 24, 0, 3)
    assert raw_ids[0].tolist() == [20, 3, 9]
    # a tiny bias breaks the tie in its favour
    b = np.zeros(24, np.float32)
    b[20] = 1e-3
    ids, _, _ = O.route(row, 24, 0, 3, sel_bias=b)
    assert ids[0].tolist() == [20, 3, 9]


def test_constant_bias_keeps_the_unbiased_order():
    rng = np.random.default_rng(24)
    rows = rng.standard_normal((50, 130)).astype(np.float32)
    plain, _, _ = O.route(rows, 128, 2, 6)
    shifted, _, _ = O.route(rows, 128, 2, 6, sel_bias=np.full(128, 0.25, np.float32))
    assert np.array_equal(plain, shifted)


def test_sinks_take_no_bias_and_never_rank():
    rng = np.random.default_rng(25)
    rows = rng.standard_normal((8, 258)).astype(np.float32)
    rows[:, 256:] = 50.0                            # sinks far above every column
    ids, w, sw = O.route(rows, 256, 2, 8, sel_bias=np.zeros(256, np.float32))
    assert np.all(ids < 256)
    assert np.all(sw > 0.0)


# -------------------------------------------------------------- packing

def test_pack_worked_bit_patterns():
    ids = np.array([[5, 0, 257]])
    w = np.array([[0.5, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9]])
    p = O.pack_topk(ids, w).view(np.uint32)
    # 0.5 = 0x3F00; 1 + 2^-8 is halfway between 0x3F80 and 0x3F81: even;
    # 1 + 3 * 2^-9 lies above the midpoint: 0x3F81
    assert p[0].tolist() == [0x00053F00, 0x00003F80, 0x01013F81]
    assert ((p >> 16) == ids).all()


def test_pack_round_trip_matches_torch_bfloat16():
    rng = np.random.default_rng(26)
    w = rng.random((40, 8)).astype(np.float32)
    ids = rng.integers(0, 1024, (40, 8))
    p = O.pack_topk(ids, w.astype(np.float64)).view(np.uint32)
    bf = torch.from_numpy(w).bfloat16().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(p & 0xFFFF, bf.astype(np.uint32))
    assert np.array_equal(p >> 16, ids.astype(np.uint32))
