"""Pins of the oracle's FP4 weight formats (no GPU).

NVFP4 is the weight format of the MoE-LoRA release ("FlashInfer 0.6.18
SM100a+SM103a MoE-LoRA AOT" release notes, "Changes since 1b699bf": gate
and up halves with distinct NVFP4 global scales); MXFP4 is its power-of-two
block-32 sibling. The pages name the formats without defining them, so the
oracle writes the public encodings from their bit fields; the pins check it
against other sources: the published list of the eight e2m1 magnitudes,
torch's own e8m0 decoding, hand-worked bytes, block boundaries that a wrong
block length would move, exact scaling laws of the layer, and the
independent brute-force formulation (which decodes e2m1 from the value list
and e4m3 from torch's table).
"""
import numpy as np
import pytest
import torch

from oracle import brute
from oracle import moe_oracle as O
from synth import make_batch, make_layer, to_numpy_batch, to_numpy_layer
from tinyspecs import TINY

# the e2m1 magnitudes of codes 0..7 as the format lists them
E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_all_sixteen_codes():
    v = O.e2m1_decode(np.arange(16))
    assert v[:8].tolist() == E2M1_VALUES
    assert v[8:].tolist() == [-x for x in E2M1_VALUES]
    assert np.signbit(v[8])                    # code 8 is -0


def test_e8m0_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    ours = O.e8m0_decode(codes)
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ours), ~fin)
    assert np.array_equal(ours[fin], ref[fin])


def test_nvfp4_worked_bytes():
    # byte 0x21: k0 = code 1 (0.5), k1 = code 2 (1.0); byte 0xF7: k2 = code 7
    # (6.0), k3 = code 15 (-6.0); byte 0x9C: k4 = code 12 (-2), k5 = code 9
    # (-0.5); the rest zero. Scale e4m3 0x40 = 2.0 for k 0..15.
    row = np.zeros((1, 8), np.uint8)
    row[0, :3] = [0x21, 0xF7, 0x9C]
    w = O.dequant_nvfp4(row, np.array([[0x40]], np.uint8))
    assert w[0, :6].tolist() == [1.0, 2.0, 12.0, -12.0, -4.0, -1.0]
    assert not w[0, 6:].any()


def test_nvfp4_scale_blocks_are_16_wide():
    # every element 1.0 (code 2, bytes 0x22); scales 1, 2, 4, 8 (e4m3 0x38,
    # 0x40, 0x48, 0x50) for k 0-15, 16-31, 32-47, 48-63: w[k] = 2^(k // 16)
    q = np.full((2, 32), 0x22, np.uint8)
    s = np.array([[0x38, 0x40, 0x48, 0x50]] * 2, np.uint8)
    w = O.dequant_nvfp4(q, s)
    assert np.array_equal(w, np.tile(2.0 ** (np.arange(64) // 16), (2, 1)))


def test_nvfp4_subnormal_and_largest_scales():
    # e4m3 0x01 = 2^-9 (smallest), 0x7E = 448 (largest); code 7 = 6.0
    q = np.full((1, 16), 0x77, np.uint8)
    w = O.dequant_nvfp4(q, np.array([[0x01, 0x7E]], np.uint8))
    assert np.array_equal(w[0], [6.0 * 2.0 ** -9] * 16 + [6.0 * 448.0] * 16)


def test_mxfp4_scale_blocks_are_32_wide():
    q = np.full((1, 32), 0x22, np.uint8)      # all 1.0
    w = O.dequant_mxfp4(q, np.array([[127, 130]], np.uint8))
    assert np.array_equal(w[0], [1.0] * 32 + [8.0] * 32)


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_fp4_dequant_matches_brute_force(fmt):
    rng = np.random.default_rng(5)
    q = rng.integers(0, 256, (6, 32), dtype=np.uint8)
    if fmt == "nvfp4":
        s = rng.integers(0, 0x7F, (6, 4), dtype=np.uint8)   # every finite code
        w = O.dequant_nvfp4(q, s)
    else:
        s = rng.integers(100, 150, (6, 2), dtype=np.uint8)
        w = O.dequant_mxfp4(q, s)
    ref = np.array(brute.dense_weight(fmt, q, s, 6, 64))
    assert np.array_equal(w, ref)


def _setup(name, T=5):
    spec = TINY[name]
    layer = make_layer(spec)
    batch = make_batch(spec, layer, T)
    return spec, to_numpy_layer(layer), to_numpy_batch(batch)


@pytest.mark.parametrize("name", ["nvfp4_lora", "mxfp4_shared", "mxfp4a8_oai"])
def test_fp4_layer_matches_brute_force(name):
    spec, arr, nb = _setup(name)
    ref = np.array(brute.layer(spec, arr, nb["x_bits"], nb["logits"]))
    ours = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"])
    assert np.abs(ref).max() > 0
    assert np.max(np.abs(ours - ref)) <= 1e-9 * np.abs(ref).max()


def test_w2_global_scale_scales_the_base_output_exactly():
    """Without LoRA the layer output is linear in W2, so doubling every W2
    global scale doubles it bit for bit; dropping the scale would not."""
    spec, arr, nb = _setup("nvfp4_lora")
    spec = spec.scaled(lora_rank=0, lora_down=False)
    a = dict(arr)
    base = O.moe_layer(spec, a, nb["x_bits"], nb["logits"])
    a["gs2"] = (arr["gs2"] * np.float32(2.0)).astype(np.float32)
    assert np.array_equal(O.moe_layer(spec, a, nb["x_bits"], nb["logits"]), 2.0 * base)
    a["gs2"] = None
    assert not np.allclose(O.moe_layer(spec, a, nb["x_bits"], nb["logits"]), base)


def test_nvfp4_true_units_invariant_to_a_power_of_two_resplit():
    """Moving a factor 2 from the up half's global scale into its NVFP4
    block scales (e4m3 codes one exponent step higher) leaves the layer,
    LoRA included, bit-identical: the delta is added in true units."""
    spec, arr, nb = _setup("nvfp4_lora")
    ref = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"])
    a = dict(arr)
    s = arr["w13_s"].copy()
    up = s[:, spec.I:, :]
    assert (up >= 0x08).all() and (up < 0x70).all()    # normal, positive codes
    s[:, spec.I:, :] = up + 0x08
    gs = arr["gs"].copy()
    gs[:, 1] *= np.float32(0.5)
    a["w13_s"], a["gs"] = s, gs
    assert np.array_equal(O.moe_layer(spec, a, nb["x_bits"], nb["logits"]), ref)


# ---------------------------------------------------------------- MXFP8 pins
# The W4A8 MXFP4 layers quantise the GEMM1 activations to MXFP8: per row and
# 32 columns an e8m0 power of two 2^e, the smallest that keeps the group's
# amax within 448 (e4m3's largest value), and e4m3 codes of x / 2^e.

def _mx(rows):
    q, e = O.quant_act_mxfp8(np.asarray(rows, np.float32))
    return q, e.astype(np.int64)


def test_mxfp8_exponent_closed_forms():
    rows = np.zeros((6, 32), np.float32)
    rows[0, 3] = 448.0                      # amax = 448 * 2^0: e = 0
    rows[1, 0] = -448.0 * 2.0 ** -20        # e = -20, sign kept
    rows[2, 7] = 450.0                      # next bf16 above 448: e = 1
    rows[3, 1] = 500.0                      # floor(log2) - 8 would give 0 and clip
    rows[4, 0] = 3.0e38                     # 448 * 2^119 = 2.98e38 < 3e38: e = 120
    # row 5 all zero: e8m0 code 0, every code 0
    q, e = _mx(rows)
    assert e[:, 0].tolist() == [127, 107, 128, 128, 247, 0]
    assert q[0, 3] == 0x7E and q[1, 0] == 0xFE          # +-448
    assert O.e4m3_decode(q[2, 7]) == 224.0              # 225 rounds to even 224
    assert O.e4m3_decode(q[3, 1]) == 256.0              # 250 -> 256 (step 16 below 256)
    assert not q[5].any()
    # amax exactly 448 * 2^e is kept; a hair above moves e up by one
    for k in (-30, -1, 0, 7, 40):
        a = np.float32(448.0 * 2.0 ** k)
        up = np.nextafter(a, np.float32(np.inf))
        _, e2 = _mx([[a] + [0.0] * 31, [up] + [0.0] * 31])
        assert e2[:, 0].tolist() == [127 + k, 128 + k]


def test_mxfp8_ties_go_to_the_even_code():
    # amax 448 (e = 0); 1.0625 lies midway between 1.0 (0x38) and 1.125
    # (0x39), 1.1875 between 1.125 and 1.25 (0x3A), 232 between 224 (0x76)
    # and 240 (0x77)
    row = np.zeros((1, 32), np.float32)
    row[0, :4] = [448.0, 1.0625, 1.1875, 232.0]
    q, e = _mx(row)
    assert e[0, 0] == 127
    assert q[0, :4].tolist() == [0x7E, 0x38, 0x3A, 0x76]


def test_mxfp8_groups_are_32_wide():
    # 1.0 everywhere, amax 448 in columns 0..31 only: the first group keeps
    # e = 0 (1.0 exact), the second has amax 1 (e = -8: 1.0 -> 256)
    row = np.ones((1, 64), np.float32)
    row[0, 31] = 448.0
    q, e = _mx(row)
    assert e[0].tolist() == [127, 119]
    v = O.e4m3_decode(q[0]) * np.repeat(O.e8m0_decode(e[0].astype(np.uint8)), 32)
    assert np.array_equal(v, row[0].astype(np.float64))


def _mx_against_brute():
    """Random bf16 rows whose magnitude changes from one 32-column group to
    the next (and zero, tiny and huge groups): the oracle's MXFP8 values
    and exponents against the brute-force scan-and-search."""
    rng = np.random.default_rng(11)
    T, H = 12, 256
    mag = np.ldexp(1.0, rng.integers(-40, 40, (T, H // 32)).repeat(32, axis=1))
    x = rng.standard_normal((T, H)) * mag * (rng.random((T, H)) < 0.9)
    x[3, :32] = 0.0
    x[4, 32:64] = 1e-39
    x[5, 64:96] *= 1e30
    xb = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    q, e = _mx(xb)
    ours = O.e4m3_decode(q) * np.repeat(O.e8m0_decode(e.astype(np.uint8)), 32, axis=1)
    ref = np.array([brute.mxfp8_row([float(v) for v in row]) for row in xb])
    exps = np.array([[brute.mxfp8_exponent(float(np.abs(xb[t, 32 * b:32 * b + 32]).max()))
                      for b in range(H // 32)] for t in range(T)])
    return np.array_equal(ours, ref) and np.array_equal(e - 127, exps)


def test_mxfp8_matches_brute_force():
    assert _mx_against_brute()


def _mut_mx_group_64(mp):
    real = O.quant_act_mxfp8

    def g64(x_f32, group=32):
        q, e = real(x_f32, 64)
        return q, np.repeat(e, 2, axis=1)
    mp.setattr(O, "quant_act_mxfp8", g64)


def _mut_mx_truncate(mp):
    """Codes truncated toward zero instead of rounded to nearest."""
    real = O.quant_act_mxfp8

    def trunc(x_f32, group=32):
        q, e = real(x_f32, group)
        x = np.asarray(x_f32, np.float32).astype(np.float64)
        v = x / np.repeat(O.e8m0_decode(e), group, axis=1)
        qv = O.e4m3_decode(q)
        down = np.abs(qv) > np.abs(v)               # rounded away from zero
        q = np.where(down & ((q & 0x7F) > 0), q - 1, q).astype(np.uint8)
        return q, e
    mp.setattr(O, "quant_act_mxfp8", trunc)


@pytest.mark.parametrize("mut", [_mut_mx_group_64, _mut_mx_truncate])
def test_planted_mxfp8_mistakes_are_caught(mut, monkeypatch):
    mut(monkeypatch)
    assert not _mx_against_brute()


def test_w4a8_layer_differs_from_w4a16_by_the_activation_rounding():
    """Same weights and inputs: the MXFP8 activation rounding moves the
    output (so it is applied), by about e4m3's relative precision."""
    spec, arr, nb = _setup("mxfp4a8_oai")
    a8 = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"])
    a16 = O.moe_layer(spec.scaled(fmt="mxfp4"), arr, nb["x_bits"], nb["logits"])
    rel = np.sqrt(np.mean((a8 - a16) ** 2) / np.mean(a16 ** 2))
    assert 1e-3 < rel < 0.1
