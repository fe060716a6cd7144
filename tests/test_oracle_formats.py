"""Pins of the oracle's number formats against library routines and the
pages' stated rules (no GPU)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # closed-form spot values of OCP e4m3fn
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9
    assert ours[0x38] == 1.0 and ours[0xB8] == -1.0 and ours[0x08] == 2.0 ** -6
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def test_e4m3_round_matches_torch_rne_inside_range():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(200000) * 60,
        rng.standard_normal(50000) * 1e-2,
        rng.standard_normal(20000) * 1e-3]).astype(np.float32)
    ours = O.e4m3_round(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ok = np.abs(v) < 448
    assert np.array_equal(ours[ok], ref[ok])


def test_e4m3_round_ties_and_saturation():
    # midpoints go to the even code
    assert O.e4m3_round([2.0 ** -10])[0] == 0x00      # 0 vs 2^-9 -> 0 (even)
    assert O.e4m3_round([3 * 2.0 ** -10])[0] == 0x02  # 2^-9 vs 2^-8 -> code 2
    assert O.e4m3_round([1.0625])[0] == 0x38          # 1 vs 1.125 -> 1.0
    assert O.e4m3_round([1.1875])[0] == 0x3A          # 1.125 vs 1.25 -> 1.25
    # 464 is the midpoint of 448 and (unrepresentable) 480: ties to 448;
    # everything larger saturates to 448 instead of NaN
    for v in (448.0, 460.0, 464.0, 465.0, 1e6, np.inf):
        assert O.e4m3_round([v])[0] == 0x7E
        assert O.e4m3_round([-v])[0] == 0xFE
    assert O.e4m3_round([np.nan])[0] & 0x7F == 0x7F


def test_bf16_round_and_decode_match_torch():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))) \
        .astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16)
    ours = O.bf16_round(v.astype(np.float64))
    assert np.array_equal(ours, ref.double().numpy())
    bits = ref.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_decode(bits), ref.double().numpy())


def test_int4_worked_example_from_page_rule():
    ex = json.load(open(os.path.join(GOLD, "int4_worked_example.json")))
    scale = torch.tensor([0.01171875], dtype=torch.bfloat16)  # exact bf16
    sbits = scale.view(torch.int16).numpy().view(np.uint16)
    packed = np.full((1, 16), ex["byte"], dtype=np.uint8)    # K = 32
    w = O.dequant_int4_g32(packed, sbits.reshape(1, 1))
    s = float(scale.double())
    assert np.all(w[0, 0::2] == ex["even_k_factor"] * s)
    assert np.all(w[0, 1::2] == ex["odd_k_factor"] * s)


def test_int4_all_bytes_and_group_scales():
    rng = np.random.default_rng(3)
    N, K = 4, 512
    packed = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    packed[0, :256] = np.arange(256, dtype=np.uint8)
    sc = torch.rand(N, K // 32, dtype=torch.float32).to(torch.bfloat16)
    w = O.dequant_int4_g32(packed, sc.view(torch.int16).numpy().view(np.uint16))
    scd = sc.double().numpy()
    for n in range(N):
        for k in range(K):
            byte = int(packed[n, k // 2])
            nib = (byte & 15) if k % 2 == 0 else (byte >> 4)
            assert w[n, k] == (nib - 8) * scd[n, k // 32]


def test_fp8_block_dequant_matches_torch_decode():
    rng = np.random.default_rng(4)
    q = rng.integers(0, 256, (256, 384), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x10
    bs = rng.uniform(1e-4, 1e-2, (2, 3)).astype(np.float32)
    w = O.dequant_fp8_block(q, bs)
    ref = torch.from_numpy(q).view(torch.float8_e4m3fn).double() * \
        torch.from_numpy(bs).double().repeat_interleave(128, 0).repeat_interleave(128, 1)
    assert np.array_equal(w, ref.numpy())


def test_quant_act_properties_and_torch_agreement():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(7, 512, generator=g).to(torch.bfloat16).float().numpy()
    x[3, 128:256] = 0.0                                    # zero group
    x[4, :128] *= 1e-30                                    # tiny group
    q, s = O.quant_act_fp8(x)
    assert s.dtype == np.float32 and s.shape == (7, 4)
    assert s[3, 1] == 1.0 and np.all(q[3, 128:256] & 0x7F == 0)
    amax = np.abs(x.reshape(7, 4, 128)).max(axis=2)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax / np.float32(448)).astype(np.float32)[nz])
    deq = O.e4m3_decode(q)
    assert np.all(np.abs(deq) <= 448)
    # same codes as torch's RNE conversion of the fp32 quotient (no saturation
    # needed here: |x / s| <= 448 up to fp32 rounding)
    quot = (x.reshape(7, 4, 128) / s[:, :, None]).astype(np.float32).reshape(7, 512)
    ref = torch.from_numpy(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    # reconstruction within half an e4m3 step (relative 2^-4 for normals)
    rec = deq * np.repeat(s, 128, axis=1)
    err = np.abs(rec - x)
    step = np.maximum(np.abs(x) * 2.0 ** -3, np.repeat(s, 128, axis=1) * 2.0 ** -9)
    assert np.all(err <= step / 2 + 1e-30)
