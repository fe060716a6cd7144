"""Pins of the oracle's expert FFN and combine (no GPU): the SwiGLU epilogue
against library activations, LoRA invariants from the MoE-LoRA release
notes, and the whole layer against the independent brute-force formulation,
with planted mistakes that must be caught."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import brute
from oracle import moe_oracle as O
from synth import make_batch, make_layer, to_numpy_batch, to_numpy_layer
from tests.tinyspecs import TINY

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gu(n=20000, scale=8.0, seed=11):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(n, generator=g, dtype=torch.float64) * scale,
            torch.randn(n, generator=g, dtype=torch.float64) * scale)


def test_swiglu_defaults_reduce_to_silu_times_up():
    g, u = _gu()
    ours = O.swiglu(g.numpy(), u.numpy())
    np.testing.assert_allclose(ours, (F.silu(g) * u).numpy(), rtol=1e-13, atol=1e-300)


def test_swiglu_clamped_matches_page_formula():
    p = json.load(open(os.path.join(GOLD, "epilogue_params.json")))["clamped_swiglu"]
    g, u = _gu()
    L = p["limit"]
    ref = F.silu(torch.clamp(g, max=L)) * torch.clamp(u, -L, L)
    np.testing.assert_allclose(O.swiglu(g.numpy(), u.numpy(), 1.0, 0.0, L),
                               ref.numpy(), rtol=1e-13, atol=1e-300)


def test_swiglu_oai_matches_page_formula_and_bounds():
    p = json.load(open(os.path.join(GOLD, "epilogue_params.json")))["oai_swiglu"]
    a, b, L = p["alpha"], p["beta"], p["limit"]
    g, u = _gu()
    gc = torch.clamp(g, max=L)
    ref = gc * torch.sigmoid(a * gc) * (torch.clamp(u, min=-L, max=L) + b)
    h = O.swiglu(g.numpy(), u.numpy(), a, b, L)
    np.testing.assert_allclose(h, ref.numpy(), rtol=1e-13, atol=1e-300)
    # |h| <= max(L sigma(aL), max_x |x sigma(a x)| over x < 0) * (L + |b|)
    neg_peak = 0.27846454276107 / a
    bound = max(L / (1 + math.exp(-a * L)), neg_peak) * (L + abs(b))
    assert np.all(np.abs(h) <= bound * (1 + 1e-12))
    # above the limit the output no longer depends on g
    h1 = O.swiglu(np.array([L + 0.5, L + 50.0]), np.array([1.0, 1.0]), a, b, L)
    assert h1[0] == h1[1]


def _oracle_and_brute(spec, T, mutate=None, monkeypatch=None):
    layer = make_layer(spec)
    batch = make_batch(spec, layer, T)
    arr = to_numpy_layer(layer)
    nb = to_numpy_batch(batch)
    ref = np.array(brute.layer(spec, arr, nb["x_bits"], nb["logits"], nb["adapter_ids"]))
    if mutate is not None:
        mutate(monkeypatch)
    ours = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"], adapter_ids=nb["adapter_ids"])
    if monkeypatch is not None:
        monkeypatch.undo()
    return ours, ref


@pytest.mark.parametrize("name", list(TINY))
def test_oracle_layer_matches_brute_force(name):
    spec = TINY[name]
    ours, ref = _oracle_and_brute(spec, 5)
    scale = np.abs(ref).max()
    assert scale > 0
    assert np.max(np.abs(ours - ref)) <= 1e-9 * scale


def test_oracle_k1_single_expert_and_linearity():
    spec = TINY["bf16"].scaled(top_k=1, name="tiny_k1")
    ours, ref = _oracle_and_brute(spec, 5)
    assert np.max(np.abs(ours - ref)) <= 1e-9 * np.abs(ref).max()
    layer = make_layer(spec)
    batch = make_batch(spec, layer, 5)
    arr, nb = to_numpy_layer(layer), to_numpy_batch(batch)
    o1 = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"])
    o2 = O.moe_layer(spec.scaled(route_scale=2.0), arr, nb["x_bits"], nb["logits"])
    assert np.array_equal(o2, 2.0 * o1)


def _mut_swap_gate_up(mp):
    real = O.w13_dequant

    def swapped(spec, arr, e):
        w = real(spec, arr, e)
        return np.concatenate([w[spec.I:], w[:spec.I]])
    mp.setattr(O, "w13_dequant", swapped)


def _mut_drop_clamp(mp):
    real = O.swiglu
    mp.setattr(O, "swiglu", lambda g, u, a=1.0, b=0.0, L=math.inf: real(g, u, a, b))


def _mut_no_requant(mp):
    mp.setattr(O, "requant_fp8", lambda h, group=128: h)


def _row_amax_quant(v):
    """e4m3 quantisation with one scale per row (amax over the whole row)
    instead of one per 128 columns: the planted grouping mistake."""
    v = np.asarray(v, np.float64)
    amax = np.abs(v).max(axis=1).astype(np.float32) if v.shape[0] else \
        np.zeros(0, np.float32)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return s


def _mut_requant_per_row(mp):
    def per_row(h, group=128):
        s = _row_amax_quant(h).astype(np.float64)
        return O.e4m3_decode(O.e4m3_round(h / s[:, None])) * s[:, None]
    mp.setattr(O, "requant_fp8", per_row)


def _mut_quant_act_per_row(mp):
    def per_row(x_f32, group=128):
        x = np.asarray(x_f32, np.float32)
        s = _row_amax_quant(x)
        q = O.e4m3_round((x / s[:, None]).astype(np.float32).astype(np.float64))
        return q, np.repeat(s[:, None], x.shape[1] // group, axis=1)
    mp.setattr(O, "quant_act_fp8", per_row)


def _mut_w13_block_scale_rows_only(mp):
    """Weight block scales indexed by the row block only (the first K
    block's scale used for every K): a dropped index."""
    real = O.dequant_fp8_block

    def first_k_block(q, bs):
        b = np.asarray(bs)
        return real(q, np.repeat(b[:, :1], b.shape[1], axis=1))
    mp.setattr(O, "dequant_fp8_block", first_k_block)


def _mut_mx_floor_exponent(mp):
    """MXFP8 exponent from floor(log2 amax) - 8 (the largest element may then
    exceed 448 and is saturated) instead of the smallest e that keeps the
    group within 448."""
    def floor_exp(x_f32, group=32):
        x = np.asarray(x_f32, np.float32).astype(np.float64)
        T, H = x.shape
        xg = x.reshape(T, H // group, group)
        amax = np.abs(xg).max(axis=2)
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127)
        e = np.maximum(e, -127).astype(np.int64)
        q = O.e4m3_round(xg / np.ldexp(1.0, e.astype(np.int32))[:, :, None]).reshape(T, H)
        return q, (e + 127).astype(np.uint8)
    mp.setattr(O, "quant_act_mxfp8", floor_exp)


@pytest.mark.parametrize("mut,name", [
    (_mut_swap_gate_up, "fp8_clamp_shared"), (_mut_drop_clamp, "fp8_clamp_shared"),
    (_mut_drop_clamp, "fp8_oai"), (_mut_no_requant, "fp8_oai"),
    (_mut_requant_per_row, "fp8_2grp_shared"), (_mut_requant_per_row, "ep_lora_2grp"),
    (_mut_quant_act_per_row, "fp8_2grp_shared"),
    (_mut_w13_block_scale_rows_only, "fp8_2grp_shared"),
    (_mut_mx_floor_exponent, "mxfp4a8_oai")])
def test_planted_mistakes_are_caught_by_brute_force(mut, name, monkeypatch):
    spec = TINY[name]
    ours, ref = _oracle_and_brute(spec, 5, mut, monkeypatch)
    assert np.max(np.abs(ours - ref)) > 1e-6 * np.abs(ref).max()


def test_planted_missing_rebase_is_caught(monkeypatch):
    spec = TINY["ep_lora"]
    layer = make_layer(spec)
    batch = make_batch(spec, layer, 5)
    arr, nb = to_numpy_layer(layer), to_numpy_batch(batch)
    ref = np.array(brute.layer(spec, arr, nb["x_bits"], nb["logits"]))
    bad = O.moe_layer(spec.scaled(offset=0), arr, nb["x_bits"], nb["logits"])
    assert np.max(np.abs(bad - ref)) > 1e-6 * np.abs(ref).max()


# ---------------------------------------------------------------- LoRA pins

def _lora_setup(T=6):
    spec = TINY["ep_lora"]
    layer = make_layer(spec)
    batch = make_batch(spec, layer, T)
    return spec, layer, to_numpy_layer(layer), to_numpy_batch(batch)


def test_lora_zero_B_equals_base_and_no_adapter_equals_base():
    spec, layer, arr, nb = _lora_setup()
    base = O.moe_layer(spec.scaled(lora_rank=0), arr, nb["x_bits"], nb["logits"])
    arr0 = dict(arr, lora_B=np.zeros_like(arr["lora_B"]),
                lora_B2=np.zeros_like(arr["lora_B2"]))
    zero_b = O.moe_layer(spec, arr0, nb["x_bits"], nb["logits"])
    assert np.array_equal(base, zero_b)
    with_lora = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"])
    assert np.max(np.abs(with_lora - base)) > 1e-3 * np.abs(base).max()
    # zero down B: the up LoRA alone
    up_only = O.moe_layer(spec.scaled(lora_down=False), arr, nb["x_bits"], nb["logits"])
    arr2 = dict(arr, lora_B2=np.zeros_like(arr["lora_B2"]))
    assert np.array_equal(O.moe_layer(spec, arr2, nb["x_bits"], nb["logits"]), up_only)
    assert np.max(np.abs(with_lora - up_only)) > 1e-3 * np.abs(base).max()


def test_down_lora_is_linear_in_its_B():
    """Doubling B2 doubles the down delta: out(2 B2) - out(B2) = out(B2) -
    out(0) (exact up to float64 rounding)."""
    spec, layer, arr, nb = _lora_setup()
    f = lambda b2: O.moe_layer(spec, dict(arr, lora_B2=b2), nb["x_bits"], nb["logits"])
    b2 = arr["lora_B2"]
    twice = (torch.from_numpy(b2.view(np.int16)).view(torch.bfloat16).float() * 2
             ).bfloat16().view(torch.int16).numpy().view(np.uint16)
    o0, o1, o2 = f(np.zeros_like(b2)), f(b2), f(twice)
    np.testing.assert_allclose(o2 - o1, o1 - o0, rtol=0, atol=1e-9 * np.abs(o1).max())


def _mut_down_input_after_requant(mp):
    """Feed the down LoRA the re-quantised h (what the down GEMM reads)
    instead of the true-units SwiGLU output."""
    mp.setattr(O, "down_lora_input", lambda h: O.requant_fp8(h))


def _mut_down_input_gate_units(mp):
    """The pre-fix units: the up half (and so h and the down-LoRA input)
    left off by gate/up."""
    real = O.down_lora_delta
    mp.setattr(O, "down_lora_delta", lambda spec, arr, e, hl, adapters=None: real(
        spec, arr, e, hl * (float(arr["gs"][e][0]) / float(arr["gs"][e][1])), adapters))


def _mut_down_dropped(mp):
    mp.setattr(O, "down_lora_delta", lambda spec, arr, e, hl, adapters=None: 0.0)


@pytest.mark.parametrize("mut", [_mut_down_input_after_requant, _mut_down_input_gate_units,
                                 _mut_down_dropped])
def test_planted_down_lora_mistakes_are_caught(mut, monkeypatch):
    spec = TINY["ep_lora"]
    ours, ref = _oracle_and_brute(spec, 5, mut, monkeypatch)
    assert np.max(np.abs(ours - ref)) > 1e-6 * np.abs(ref).max()


def _resplit(spec, arr, factor):
    """Move a factor between the up half's global scale and its block scales:
    the dequantised weights stay the same."""
    a = dict(arr)
    gs = arr["gs"].copy()
    gs[:, 1] = (gs[:, 1] / np.float32(factor)).astype(np.float32)
    s = arr["w13_s"].copy()
    nb_half = spec.I // 128
    s[:, nb_half:, :] = (s[:, nb_half:, :] * np.float32(factor)).astype(np.float32)
    a["gs"], a["w13_s"] = gs, s
    return a


def test_lora_true_units_invariant_to_up_gate_split():
    spec, layer, arr, nb = _lora_setup()
    ref = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"])
    # power-of-two re-split: bit-identical
    out = O.moe_layer(spec, _resplit(spec, arr, 4.0), nb["x_bits"], nb["logits"])
    assert np.array_equal(out, ref)
    # arbitrary re-split: equal up to fp32 rounding of the moved scales
    out = O.moe_layer(spec, _resplit(spec, arr, 1.37), nb["x_bits"], nb["logits"])
    assert np.max(np.abs(out - ref)) <= 1e-5 * np.abs(ref).max()


def test_lora_old_units_bug_is_caught(monkeypatch):
    """The pre-fix behaviour (delta added before the up half is rescaled,
    i.e. the up delta multiplied by gs_up / gs_gate) breaks the invariance."""
    spec, layer, arr, nb = _lora_setup()
    real = O.lora_delta

    def buggy(spec_, arr_, e, xrows, adapters=None):
        d = real(spec_, arr_, e, xrows, adapters)
        gs = arr_["gs"][e].astype(np.float64)
        d[:, spec_.I:] *= gs[1] / gs[0]
        return d
    monkeypatch.setattr(O, "lora_delta", buggy)
    a = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"])
    b = O.moe_layer(spec, _resplit(spec, arr, 1.8), nb["x_bits"], nb["logits"])
    monkeypatch.undo()
    ref = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"])
    assert np.max(np.abs(a - b)) > 1e-3 * np.abs(ref).max()
    assert np.max(np.abs(a - ref)) > 1e-3 * np.abs(ref).max()


# ------------------------------------------------ boundary rounding decisions

def test_rounding_alternatives_fp8_marks_only_boundary_elements():
    # group amax 448 -> s = 1; values at and away from e4m3 midpoints
    h = np.zeros((1, 128))
    h[0, 0] = 448.0
    h[0, 1] = 1.0625          # midpoint of 1.0 and 1.125
    h[0, 2] = 1.03            # well inside (1.0 is nearest)
    h[0, 3] = 3 * 2.0 ** -10  # midpoint of subnormals 2^-9 and 2^-8
    h[0, 4] = 248.0           # midpoint of 240 and 256
    alt = O.rounding_alternatives(h, np.full_like(h, 1e-9), "fp8")
    np.testing.assert_allclose([alt[0, 1], alt[0, 3], alt[0, 4]],
                               [0.125, 2.0 ** -9, 16.0], rtol=1e-4)
    assert alt[0, 0] == 0 and alt[0, 2] == 0
    # a wider error band catches 1.03 too (distance to 1.0625 is 0.0325)
    alt = O.rounding_alternatives(h, np.full_like(h, 0.04), "fp8")
    assert alt[0, 2] >= 0.125


def test_rounding_alternatives_fp8_scale_per_128_columns():
    """Two rows, two 128-column groups each, with group amax 448, 300, 100
    and 420 (scales in ratios that are not powers of two): the same e4m3
    midpoints placed in every group, in that group's units, are found only
    when each group uses its own scale, and the admissible step scales with
    that group's s."""
    h = np.zeros((2, 256))
    amax = [[448.0, 300.0], [100.0, 420.0]]
    scale = lambda a: float(np.float32(np.float32(a) / np.float32(448.0)))
    for r in range(2):
        for gi in range(2):
            s = scale(amax[r][gi])
            c = 128 * gi
            h[r, c] = amax[r][gi]
            h[r, c + 1] = 1.0625 * s       # midpoint of 1 and 1.125 (times s)
            h[r, c + 2] = 248.0 * s        # midpoint of 240 and 256
            h[r, c + 3] = 1.03 * s         # inside: 1 is nearest
    alt = O.rounding_alternatives(h, np.full_like(h, 1e-12), "fp8")
    for r in range(2):
        for gi in range(2):
            s = scale(amax[r][gi])
            c = 128 * gi
            np.testing.assert_allclose([alt[r, c + 1], alt[r, c + 2]],
                                       [0.125 * s, 16.0 * s], rtol=1e-4)
            assert alt[r, c] == 0 and alt[r, c + 3] == 0
    # the re-quantisation itself: every group's amax element becomes 448 s of
    # that group and the midpoints go to the even neighbour in its units
    hq = O.requant_fp8(h)
    for r in range(2):
        for gi in range(2):
            s = scale(amax[r][gi])
            c = 128 * gi
            assert hq[r, c] == 448.0 * s
            assert hq[r, c + 1] == 1.0 * s and hq[r, c + 2] == 256.0 * s
            assert hq[r, c + 3] == 1.0 * s


def test_rounding_alternatives_bf16():
    h = np.array([[1.0 + 2.0 ** -8, 1.0 + 2.0 ** -9, 3.0]])   # midpoint, inside, exact
    alt = O.rounding_alternatives(h, np.full_like(h, 1e-12), "bf16")
    np.testing.assert_allclose(alt[0, 0], 2.0 ** -7, rtol=1e-3)
    assert alt[0, 1] == 0 and alt[0, 2] == 0


_BF16_CODES = np.array([c for c in range(1 << 16) if (c & 0x7F80) != 0x7F80])
_BF16_VALS = O.bf16_decode(_BF16_CODES.astype(np.uint16))


def _bf16_brute(v, near):
    """Nearest bf16 value by search over the finite bit patterns' values
    within `near` of the samples (ties to the even pattern): independent of
    bf16_round."""
    v = np.asarray(v, np.float64)
    keep = (_BF16_VALS >= v.min() - near) & (_BF16_VALS <= v.max() + near)
    vals, codes = _BF16_VALS[keep], _BF16_CODES[keep]
    d = np.abs(vals[None, :] - v[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = np.where(d == best, codes[None, :], 1 << 20)
    even = np.where((cand & 1) == 0, cand, 1 << 20).min(axis=1)
    pick = np.where(even < (1 << 20), even, cand.min(axis=1))
    return O.bf16_decode(pick.astype(np.uint16))


@pytest.mark.parametrize("h,err", [
    (5.6e-7, 1e-6),            # a band wider than the grid
    (0.0, 5e-6), (-0.0, 5e-6), # around zero the grid is far finer than at 1
    (0.5, 2.0 ** -11),         # just below a power of two the spacing halves
    (0.5 - 2.0 ** -10, 2.0 ** -12), (-2.0, 2.0 ** -8), (1.0 + 2.0 ** -9, 1e-9),
    (3.0, 1e-3), (1e-39, 1e-40)])
def test_rounding_alternatives_bf16_cover_every_rounding_in_the_band(h, err):
    """The bound equals the largest |bf16(v) - bf16(h)| over v in
    [h - err, h + err], found by sampling the band densely and rounding each
    sample by exhaustive search."""
    alt = O.rounding_alternatives(np.array([[h]]), np.array([[err]]), "bf16")[0, 0]
    e = err + abs(h) * O.EVAL_REL
    v = h + np.linspace(-e, e, 4001)
    near = 2 * e + abs(h) / 64 + 1e-37          # more than one grid step
    dev = np.abs(_bf16_brute(v, near) - _bf16_brute(np.array([h]), near)[0]).max()
    assert dev <= alt <= dev * (1 + 1e-9) + 1e-300


def test_allowance_is_zero_or_small_and_value_unchanged():
    spec = TINY["fp8_clamp_shared"]
    layer = make_layer(spec)
    batch = make_batch(spec, layer, 5)
    arr, nb = to_numpy_layer(layer), to_numpy_batch(batch)
    out = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"])
    out2, allow, nbnd = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"],
                                    with_allowance=True)
    assert np.array_equal(out, out2)
    assert np.all(allow >= 0)
    # boundary decisions are rare for an fp32-accurate kernel
    assert nbnd <= 0.01 * 5 * 3 * spec.I


# ------------------------------------------------------ a batch of adapters

def test_adapter_batch_matches_brute_force_and_single_adapter_runs():
    """Eight adapters, tokens picking one or none: the oracle equals the
    brute force (in test_oracle_layer_matches_brute_force too); tokens of
    adapter a give exactly the one-adapter layer built from adapter a's
    matrices; tokens with no adapter give the base layer."""
    spec = TINY["ep_lora_multi"]
    layer = make_layer(spec)
    batch = make_batch(spec, layer, 12)
    arr, nb = to_numpy_layer(layer), to_numpy_batch(batch)
    ad = nb["adapter_ids"]
    assert (ad == -1).any() and len(set(ad.tolist())) >= 4
    out = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"], adapter_ids=ad)
    one = spec.scaled(n_adapters=1)
    base = O.moe_layer(one.scaled(lora_rank=0), arr, nb["x_bits"], nb["logits"])
    for a in sorted(set(ad.tolist())):
        sel = ad == a
        if a < 0:
            np.testing.assert_array_equal(out[sel], base[sel])
            continue
        arr_a = dict(arr, **{k: arr[k][a] for k in ("lora_A", "lora_B", "lora_A2", "lora_B2")})
        ref = O.moe_layer(one, arr_a, nb["x_bits"], nb["logits"])
        np.testing.assert_array_equal(out[sel], ref[sel])
    # a wrong adapter for one token is seen
    bad = ad.copy()
    i = int(np.nonzero(ad >= 0)[0][0])
    bad[i] = (ad[i] + 1) % spec.n_adapters
    out_bad = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"], adapter_ids=bad)
    assert np.max(np.abs(out_bad[i] - out[i])) > 1e-6 * np.abs(out).max()
