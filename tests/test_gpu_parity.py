"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Integer and index work is compared bit-exactly (routing ids, permutation,
activation codes and scales); floating-point outputs against the bars:
routing weights rtol = atol = 2e-3; layer outputs max|err| <= 1e-2 RMS and
cosine >= 0.9999 for FP8/INT4, max|err| <= 5e-3 RMS for BF16.
"""
import math

import numpy as np
import pytest
import torch

import mixture_experts_expert_sigmoid_amd as M
from oracle import moe_oracle as O
from synth import (CONFIGS, FP4_CONFIGS, make_batch, make_layer, to_numpy_batch,
                   to_numpy_layer)
from tests.gpu_helpers import StepCalls, compare, module_for, tolerance

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")]


def _log(*a):
    print("[case]", *a, flush=True)


# ------------------------------------------------------------------ route

ROUTE_CASES = [("ep_lora_258", 1), ("ep_lora_258", 37), ("ep_lora_258", 512),
               ("ep_lora_258", 8192), ("fp8_clamp_288", 64), ("fp8_oai_128_skew", 4096),
               ("int4_g32_64", 2048), ("k14_sink2", 300), ("routed_512", 300),
               ("routed_600", 300), ("k16_sink2", 300)]
# Beyond the five workloads: 512 and 600 routed experts (8 and 16 columns
# per lane) and 16 or 18 reported slots per row.
ROUTE_SPECS = {
    "k14_sink2": CONFIGS["ep_lora_258"].scaled(name="k14_sink2", top_k=14),
    "routed_512": CONFIGS["fp8_clamp_288"].scaled(name="routed_512", n_routed=512),
    "routed_600": CONFIGS["fp8_clamp_288"].scaled(name="routed_600", n_routed=600),
    "k16_sink2": CONFIGS["ep_lora_258"].scaled(name="k16_sink2", top_k=16),
}


@pytest.mark.parametrize("name,T", ROUTE_CASES)
def test_route_parity(name, T):
    _log("route", name, T)
    spec = ROUTE_SPECS.get(name) or CONFIGS[name]
    lg = make_batch(spec, None, T).logits
    N, S, k = spec.n_routed, spec.n_sink, spec.top_k
    # padded rows exercise the row stride
    pad = torch.full((T, N + S + 5), 7.0)
    pad[:, :N + S] = lg
    d = pad.cuda()[:, :N + S]
    ids = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, device="cuda")
    sw = torch.empty(T, S, device="cuda") if S else None
    M.moe_route(d, N, S, k, 2.6, 4.0, ids, w, sw)
    torch.cuda.synchronize()
    rid, rw, rsw = O.route(lg.numpy(), N, S, k, 2.6, 4.0)
    assert np.array_equal(ids.cpu().numpy(), rid)
    np.testing.assert_allclose(w.cpu().numpy(), rw, rtol=2e-3, atol=2e-3)
    assert np.max(np.abs(w.cpu().numpy() - rw)) < 1e-5 * 10.4
    if S:
        np.testing.assert_allclose(sw.cpu().numpy(), rsw, rtol=2e-3, atol=2e-3)
        tot = w.sum(1) + sw.sum(1)
    else:
        tot = w.sum(1)
    assert torch.isfinite(tot).all()
    np.testing.assert_allclose(tot.cpu().numpy(), 10.4, atol=1e-5)


# ---------------------------------------------------------------- permute

@pytest.mark.parametrize("T,k,E,off,E_loc,shared", [
    (0, 8, 256, 96, 32, 0), (1, 8, 256, 96, 32, 0), (37, 8, 256, 96, 32, 1),
    (1000, 4, 128, 0, 128, 0), (4096, 8, 288, 0, 288, 1), (8192, 8, 256, 96, 32, 0),
    (3000, 2, 1024, 0, 1023, 1)])
def test_permute_parity(T, k, E, off, E_loc, shared):
    _log("permute", T, k, E, off, E_loc, shared)
    g = torch.Generator().manual_seed(T * 31 + k)
    ids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).int() \
        if T else torch.zeros(0, k, dtype=torch.int32)
    G = E_loc + shared
    pc = T * k + (T if shared else 0)
    dev = dict(device="cuda", dtype=torch.int32)
    offsets = torch.full((G + 1,), -7, **dev)
    sp = torch.full((max(pc, 1),), -7, **dev)
    pr = torch.full((max(pc, 1),), -7, **dev)
    err = torch.zeros(1, **dev)
    ws = torch.empty(M.moe_permute_workspace_size(T, k, G), dtype=torch.uint8, device="cuda")
    M.moe_permute(ids.cuda(), k, E, off, E_loc, shared, offsets, sp, pr, err, ws)
    assert M.moe_read_device_error(err) == 0
    ro, rsp, rpr, rerr = O.permute(ids.numpy(), E, off, E_loc, shared)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    P = int(ro[-1])
    assert np.array_equal(sp.cpu().numpy()[:P], rsp)
    assert np.array_equal(pr.cpu().numpy()[:pc], rpr)


def test_permute_out_of_range_ids_flag_error():
    _log("permute-oob")
    ids = torch.tensor([[3, 300], [-1, 5], [7, 2]], dtype=torch.int32)
    dev = dict(device="cuda", dtype=torch.int32)
    offsets = torch.zeros(257, **dev)
    sp = torch.zeros(6, **dev)
    pr = torch.zeros(6, **dev)
    err = torch.zeros(1, **dev)
    ws = torch.empty(M.moe_permute_workspace_size(3, 2, 256), dtype=torch.uint8, device="cuda")
    M.moe_permute(ids.cuda(), 2, 256, 0, 256, 0, offsets, sp, pr, err, ws)
    assert M.moe_read_device_error(err) == M.MOE_DEVERR_GLOBAL_ID_OOB
    ro, rsp, rpr, _ = O.permute(ids.numpy(), 256, 0, 256, 0)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(sp.cpu().numpy()[:4], rsp)
    assert np.array_equal(pr.cpu().numpy(), rpr)


# ---------------------------------------------------------------- quant

@pytest.mark.parametrize("T,H", [(1, 128), (37, 2048), (512, 6144)])
def test_quant_act_bit_exact(T, H):
    _log("quant", T, H)
    g = torch.Generator().manual_seed(T + H)
    x = torch.randn(T, H, generator=g) * torch.exp(torch.randn(T, 1, generator=g) * 3)
    if T > 3:
        x[1, :128] = 0.0
        x[2, :] *= 1e-30
        x[3, 5] = 3e38
    xb = x.to(torch.bfloat16)
    xq = torch.empty(T, H, dtype=torch.uint8, device="cuda")
    xs = torch.empty(T, H // 128, device="cuda")
    M.moe_quantize_act_fp8(xb.cuda(), xq, xs)
    rq, rs = O.quant_act_fp8(xb.float().numpy())
    assert np.array_equal(xs.cpu().numpy(), rs)
    assert np.array_equal(xq.cpu().numpy(), rq)


@pytest.mark.parametrize("T,H", [(1, 128), (37, 2048), (512, 6144)])
def test_quant_act_mxfp8_bit_exact(T, H):
    """MXFP8 codes and e8m0 exponents of the W4A8 layers' activations,
    bit for bit, on rows whose magnitude changes every 32 columns (and zero,
    tiny and huge groups)."""
    _log("quant-mx", T, H)
    g = torch.Generator().manual_seed(7 * T + H)
    mag = torch.exp2(torch.randint(-30, 30, (T, H // 32), generator=g).float())
    x = torch.randn(T, H, generator=g) * mag.repeat_interleave(32, dim=1)
    if T > 3:
        x[1, :32] = 0.0
        x[2, 32:64] *= 1e-30
        x[3, 5] = 3e38
    xb = x.to(torch.bfloat16)
    xq = torch.empty(T, H, dtype=torch.uint8, device="cuda")
    xe = torch.empty(T, H // 32, dtype=torch.uint8, device="cuda")
    M.moe_quantize_act_mxfp8(xb.cuda(), xq, xe)
    rq, re = O.quant_act_mxfp8(xb.float().numpy())
    assert np.array_equal(xe.cpu().numpy(), re)
    assert np.array_equal(xq.cpu().numpy(), rq)


# ------------------------------------------------------------ whole layer

SMALL = {
    "tiny_bf16": (CONFIGS["tiny_bf16"], 16),
    "fp8_clamp_small": (CONFIGS["fp8_clamp_288"].scaled(
        name="fp8_clamp_small", H=512, I=384, n_routed=24, cfg_id=22), 300),
    "fp8_clamp_decode": (CONFIGS["fp8_clamp_288"].scaled(
        name="fp8_clamp_dec", H=512, I=384, n_routed=24, cfg_id=22), 5),
    "fp8_oai_small": (CONFIGS["fp8_oai_128_skew"].scaled(
        name="fp8_oai_small", H=384, I=256, n_routed=16, cfg_id=23), 200),
    # 600 routed experts + the shared one at T = 50: a decode-sized launch
    # (32-row class, the 4-wave 128-column GEMM2 tiles) whose tile prefix
    # covers more groups than the workgroup has threads
    "fp8_many_groups": (CONFIGS["fp8_clamp_288"].scaled(
        name="fp8_many_groups", H=256, I=256, n_routed=600, cfg_id=55), 50),
    "int4_small": (CONFIGS["int4_g32_64"].scaled(
        name="int4_small", H=512, I=256, n_routed=16, cfg_id=24), 100),
    "int4_decode": (CONFIGS["int4_g32_64"].scaled(
        name="int4_dec", H=512, I=256, n_routed=16, cfg_id=24), 3),
    # the EP share with the up LoRA only (as configured) and with the down
    # LoRA as well
    "ep_lora_small": (CONFIGS["ep_lora_258"].scaled(
        name="ep_lora_small", H=256, I=256, cfg_id=25, lora_down=True), 300),
    "ep_lora_up_small": (CONFIGS["ep_lora_258"].scaled(
        name="ep_lora_up_small", H=256, I=256, cfg_id=25), 300),
    "ep_lora_mid": (CONFIGS["ep_lora_258"].scaled(
        name="ep_lora_mid", H=256, I=256, cfg_id=25), 37),
    # decode shapes with long K: both FP8 GEMMs take the split-K (stream-K)
    # schedule with several partial slots per tile; the second also runs the
    # LoRA delta and both global scales in the split-K epilogue
    "fp8_oai_sk": (CONFIGS["fp8_oai_128_skew"].scaled(
        name="fp8_oai_sk", H=2048, I=2048, n_routed=16, cfg_id=26), 2),
    "ep_lora_sk": (CONFIGS["ep_lora_258"].scaled(
        name="ep_lora_sk", H=2048, I=2048, n_routed=64, offset=16, cfg_id=27,
        lora_down=True), 1),
    "ep_lora_up_sk": (CONFIGS["ep_lora_258"].scaled(
        name="ep_lora_up_sk", H=2048, I=2048, n_routed=64, offset=16, cfg_id=27), 1),
    # INT4 at the C4 shape with 16 experts, T = 2: 16 pairs, split-K on GEMM1
    "int4_sk": (CONFIGS["int4_g32_64"].scaled(
        name="int4_sk", n_routed=16, cfg_id=28), 2),
    # a batch of eight adapters (tokens pick one or none) with both LoRAs:
    # FP8 plain and split-K, INT4 plain and decode, BF16
    "ep_lora_multi": (CONFIGS["ep_lora_258"].scaled(
        name="ep_lora_multi", H=256, I=256, cfg_id=31, n_adapters=8, lora_down=True), 300),
    "ep_lora_multi_sk": (CONFIGS["ep_lora_258"].scaled(
        name="ep_lora_multi_sk", H=2048, I=2048, n_routed=64, offset=16, cfg_id=32,
        n_adapters=8, lora_down=True), 4),
    "int4_lora_multi": (CONFIGS["int4_g32_64"].scaled(
        name="int4_lora_multi", H=512, I=256, n_routed=16, cfg_id=33, lora_rank=16,
        lora_down=True, n_adapters=4), 100),
    "int4_lora_multi_dec": (CONFIGS["int4_g32_64"].scaled(
        name="int4_lora_multi_dec", n_routed=16, cfg_id=34, lora_rank=16,
        lora_down=True, n_adapters=4), 3),
    "bf16_lora_multi": (CONFIGS["tiny_bf16"].scaled(
        name="bf16_lora_multi", cfg_id=35, lora_rank=8, lora_down=True, n_adapters=4), 16),
    # NVFP4 (per-half W13 and per-expert W2 global scales, both LoRAs) on
    # 128-row tiles, 32-row tiles, the split-K schedule and a batch of
    # adapters; MXFP4 with a shared expert and the clamp, plain and split-K
    "nvfp4_lora_small": (FP4_CONFIGS["nvfp4_lora_258"].scaled(
        name="nvfp4_lora_small", H=256, I=256, cfg_id=41), 300),
    "nvfp4_lora_mid": (FP4_CONFIGS["nvfp4_lora_258"].scaled(
        name="nvfp4_lora_mid", H=384, I=256, cfg_id=41), 37),
    "nvfp4_lora_sk": (FP4_CONFIGS["nvfp4_lora_258"].scaled(
        name="nvfp4_lora_sk", H=2048, I=2048, n_routed=64, offset=16, cfg_id=42), 1),
    "nvfp4_multi": (FP4_CONFIGS["nvfp4_lora_258"].scaled(
        name="nvfp4_multi", H=256, I=256, cfg_id=43, n_adapters=8), 300),
    "mxfp4_small": (FP4_CONFIGS["mxfp4_g32_64"].scaled(
        name="mxfp4_small", H=512, I=256, n_routed=16, shared=1, limit=7.0, cfg_id=44), 100),
    "mxfp4_sk": (FP4_CONFIGS["mxfp4_g32_64"].scaled(
        name="mxfp4_sk", n_routed=16, cfg_id=45), 2),
    # MXFP4 weights with MXFP8 activations into GEMM1 on the block-scaled
    # matrix cores: 128-, 64- and 32-row tiles with a shared expert and the
    # clamp; OAI SwiGLU with an odd K-block count (H = 384); per-half W13
    # global scales with a LoRA on both projections; the decode split-K
    "mxfp4a8_small": (FP4_CONFIGS["mxfp4a8_g32_64"].scaled(
        name="mxfp4a8_small", H=512, I=256, n_routed=16, shared=1, limit=7.0, cfg_id=44), 300),
    "mxfp4a8_oai": (FP4_CONFIGS["mxfp4a8_g32_64"].scaled(
        name="mxfp4a8_oai", H=384, I=256, n_routed=16, alpha=1.702, beta=1.0, limit=7.0,
        cfg_id=53), 200),
    "mxfp4a8_lora": (FP4_CONFIGS["nvfp4_lora_258"].scaled(
        name="mxfp4a8_lora", fmt="mxfp4_a8", H=256, I=256, cfg_id=54), 300),
    "mxfp4a8_sk": (FP4_CONFIGS["mxfp4a8_g32_64"].scaled(
        name="mxfp4a8_sk", n_routed=16, cfg_id=45), 2),
    # adapter batches on 128-row tiles (all 16 experts local, ~150 rows
    # each): the tile's adapters' B blocks staged in LDS; with 40 adapters a
    # tile meets more than fit and reads B from memory; rank 32 halves the
    # slots
    "ep_lora_multi_big": (CONFIGS["ep_lora_258"].scaled(
        name="ep_lora_multi_big", H=256, I=256, n_routed=16, n_sink=0, E_loc=None,
        offset=0, cfg_id=47, n_adapters=8, lora_down=True), 300),
    "nvfp4_multi_many": (FP4_CONFIGS["nvfp4_lora_258"].scaled(
        name="nvfp4_multi_many", H=256, I=256, n_routed=16, n_sink=0, E_loc=None,
        offset=0, cfg_id=48, n_adapters=40), 300),
    "int4_lora32_multi": (CONFIGS["int4_g32_64"].scaled(
        name="int4_lora32_multi", H=512, I=256, n_routed=16, cfg_id=49, lora_rank=32,
        lora_down=True, n_adapters=8), 300),
    # the smallest FP4 layer (H = I = 128, one 128-K block) with a shared
    # expert (W2 global scale included, no LoRA on it) and a rank-4 LoRA
    "nvfp4_min_shared": (FP4_CONFIGS["nvfp4_lora_258"].scaled(
        name="nvfp4_min_shared", H=128, I=128, n_routed=8, n_sink=0, E_loc=None, offset=0,
        shared=1, lora_rank=4, cfg_id=51), 20),
}

_cache = {}


def _setup(name):
    if name not in _cache:
        spec, T = SMALL[name]
        layer = make_layer(spec)
        batch = make_batch(spec, layer, T)
        _cache[name] = (spec, T, layer, batch, to_numpy_layer(layer),
                        to_numpy_batch(batch))
    return _cache[name]


def check_layer(spec, out_gpu, arr, nb, tokens=None, routing=None):
    """The output bar as stated: max|out - ref| <= tol * RMS(ref) and cosine
    >= bar. The beyond-allowance figure (the error left after removing what
    boundary rounding decisions of h can explain, either neighbouring code
    being a correct result there) is logged beside it."""
    ref, allow, nbnd = O.moe_layer(spec, arr, nb["x_bits"], nb["logits"], tokens=tokens,
                                   routing=routing, with_allowance=True,
                                   adapter_ids=nb.get("adapter_ids"))
    tol, cmin = tolerance(spec.fmt)
    got = np.asarray(out_gpu, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    excess = np.abs(got - ref) - allow
    rel_raw, cos = compare(got, ref)
    rel = float(np.max(excess)) / rms if ref.size else 0.0
    _log(f"  max|err|/rms={rel_raw:.3e} beyond-allowance={rel:.3e} cos={cos:.8f} "
         f"boundary-h={nbnd}")
    assert rel_raw <= tol, (rel_raw, tol)
    assert rel <= tol, (rel, tol)
    assert cos >= cmin, cos
    return ref


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_parity_small(name):
    spec, T, layer, batch, arr, nb = _setup(name)
    _log("forward", name, "T", T, spec.fmt, "H", spec.H, "I", spec.I)
    mod = module_for(spec, layer)
    o = mod.forward(batch.x.cuda(), batch.logits.cuda(), adapter_ids=_ad(batch))
    torch.cuda.synchronize()
    assert M.moe_read_device_error(o["err_word"]) == 0
    rid, rw, rsw = O.route(nb["logits"], spec.n_routed, spec.n_sink, spec.top_k,
                           spec.route_scale, spec.global_scale)
    assert np.array_equal(o["topk_ids"].cpu().numpy(), rid)
    np.testing.assert_allclose(o["topk_w"].cpu().numpy(), rw, rtol=2e-3, atol=2e-3)
    check_layer(spec, o["out"].cpu().numpy(), arr, nb)


def _ad(batch):
    return None if batch.adapter_ids is None else batch.adapter_ids.cuda()


def _stepwise(spec, mod, batch, T):
    """route -> permute -> quant -> gemm1 -> gemm2+combine through the
    individual C-ABI calls; returns every intermediate on the host."""
    st = StepCalls(spec, mod, batch.x.cuda(), batch.logits.cuda(), _ad(batch))
    st.run()
    torch.cuda.synchronize()
    assert M.moe_read_device_error(st.err) == 0
    if st.fp8:
        hval = O.e4m3_decode(st.h.cpu().numpy()) * np.repeat(
            st.hs.cpu().numpy().astype(np.float64), 128, axis=1)
    else:
        hval = st.h.float().cpu().numpy().astype(np.float64)
    return dict(out=st.out, offsets=st.offsets.cpu().numpy(), sp=st.sp.cpu().numpy(),
                hval=hval, hs=None if st.hs is None else st.hs.cpu().numpy(),
                h_lora=None if st.h_lora is None or not st.fp8
                else st.h_lora.float().cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("name", ["tiny_bf16", "fp8_clamp_small", "fp8_oai_small",
                                  "int4_small", "ep_lora_small", "ep_lora_up_small",
                                  "fp8_oai_sk", "ep_lora_sk", "ep_lora_up_sk", "int4_sk",
                                  "ep_lora_multi",
                                  "ep_lora_multi_sk", "int4_lora_multi_dec",
                                  "bf16_lora_multi", "nvfp4_lora_small", "nvfp4_lora_sk",
                                  "nvfp4_multi", "mxfp4_small", "mxfp4_sk",
                                  "ep_lora_multi_big", "nvfp4_multi_many",
                                  "int4_lora32_multi", "mxfp4a8_small", "mxfp4a8_oai",
                                  "mxfp4a8_lora", "mxfp4a8_sk"])
def test_gemm1_h_codes(name):
    """GEMM1 output h (codes and scales) against the oracle: equal wherever
    the exact h is not within the kernel's error of a rounding boundary;
    boundary elements may take either neighbour."""
    spec, T, layer, batch, arr, nb = _setup(name)
    _log("gemm1-h", name, T)
    mod = module_for(spec, layer)
    r = _stepwise(spec, mod, batch, T)
    xhat, xb = O.gemm1_input(spec, nb["x_bits"])
    k = spec.top_k
    n_bad = n_bnd = n_tot = 0
    for g in range(spec.n_groups):
        rows = np.arange(r["offsets"][g], r["offsets"][g + 1])
        if len(rows) == 0:
            continue
        toks = np.array([p // k if p < T * k else p - T * k for p in r["sp"][rows]])
        ad = None if nb["adapter_ids"] is None else nb["adapter_ids"][toks]
        _, det = O.expert_ffn(spec, arr, g, xhat[toks], xb[toks], detail=True, adapters=ad)
        diff = np.abs(r["hval"][rows] - det["hhat"])
        # scales agree to fp32 accuracy of the group amax
        slack = 1e-5 * np.abs(det["hhat"]) + det["alt"] * (1 + 1e-5)
        bad = diff > slack
        n_bad += int(np.count_nonzero(bad))
        for i, j in zip(*np.nonzero(bad)):
            _log(f"  outside: group {g} row {i} col {j} h_exact={det['h'][i, j]!r} "
                 f"gpu={r['hval'][rows][i, j]!r} oracle={det['hhat'][i, j]!r} "
                 f"alt={det['alt'][i, j]!r}")
        n_bnd += det["n_boundary"]
        n_tot += diff.size
        if r["h_lora"] is not None and det["alt_lora"] is not None:
            # the FP8 layer's bf16 down-LoRA input: the bf16 rounding of the
            # exact h, either neighbour at a boundary
            dl = np.abs(r["h_lora"][rows] - O.down_lora_input(det["h"]))
            bad_l = dl > det["alt_lora"] * (1 + 1e-5)
            n_bad += int(np.count_nonzero(bad_l))
    _log(f"  h elements={n_tot} boundary={n_bnd} outside-admissible={n_bad}")
    assert n_bad == 0


@pytest.mark.parametrize("name", ["ep_lora_small", "fp8_oai_sk", "ep_lora_sk",
                                  "ep_lora_up_sk", "int4_sk",
                                  "ep_lora_multi_sk", "int4_lora_multi_dec",
                                  "nvfp4_lora_sk", "nvfp4_multi", "mxfp4_sk",
                                  "mxfp4a8_small", "mxfp4a8_lora", "mxfp4a8_sk"])
def test_stepwise_entry_points_match_forward_and_oracle(name):
    """route -> permute -> quant -> gemm1 -> gemm2+combine through the
    individual C-ABI calls gives moe_forward's output bit for bit (also on
    the split-K schedule, whose partial sums live in different workspaces)."""
    spec, T, layer, batch, arr, nb = _setup(name)
    _log("stepwise", spec.name, T)
    mod = module_for(spec, layer)
    ref_out = mod.forward(batch.x.cuda(), batch.logits.cuda(),
                          adapter_ids=_ad(batch))["out"].clone()
    r = _stepwise(spec, mod, batch, T)
    assert torch.equal(r["out"], ref_out)
    check_layer(spec, r["out"].cpu().numpy(), arr, nb)


def test_lora_zero_B_and_power_of_two_resplit_on_gpu():
    spec, T, layer, batch, arr, nb = _setup("ep_lora_small")
    _log("lora-invariants", spec.name, T)
    x, lg = batch.x.cuda(), batch.logits.cuda()
    base = module_for(spec, layer, lora_A=None, lora_B=None).forward(x, lg)["out"].clone()
    zb = module_for(spec, layer, lora_B=torch.zeros_like(layer.lora_B).cuda()) \
        .forward(x, lg)["out"].clone()
    assert torch.equal(base, zb)
    full = module_for(spec, layer).forward(x, lg)["out"].clone()
    assert (full - base).abs().max() > 1e-3 * base.abs().max()
    # move a factor 4 from the up half's block scales into its global scale
    gs = layer.gs.clone()
    gs[:, 1] = gs[:, 1] / 4.0
    s = layer.w13_s.clone()
    s[:, spec.I // 128:, :] *= 4.0
    moved = module_for(spec, layer, w13_s=s.cuda(), gscale=gs.cuda()).forward(x, lg)["out"]
    torch.cuda.synchronize()
    assert torch.equal(moved, full)


def test_down_lora_zero_B2_and_adapter_batch_on_gpu():
    """Zero down-B gives the layer without the down LoRA bit for bit; a batch
    of adapters where every token takes adapter a gives the one-adapter layer
    built from adapter a's matrices bit for bit (same sums in the same order),
    and tokens without an adapter give the layer without LoRA."""
    spec, T, layer, batch, arr, nb = _setup("ep_lora_small")
    _log("down-lora / adapter-batch invariants", spec.name, T)
    x, lg = batch.x.cuda(), batch.logits.cuda()
    no_down = module_for(spec, layer, lora_A2=None, lora_B2=None).forward(x, lg)["out"].clone()
    zb2 = module_for(spec, layer, lora_B2=torch.zeros_like(layer.lora_B2).cuda()) \
        .forward(x, lg)["out"].clone()
    assert torch.equal(no_down, zb2)
    spec, T, layer, batch, arr, nb = _setup("ep_lora_multi")
    x, lg = batch.x.cuda(), batch.logits.cuda()
    multi = module_for(spec, layer)
    for a in (3, -1):
        ids = torch.full((T,), a, dtype=torch.int32, device="cuda")
        got = multi.forward(x, lg, adapter_ids=ids)["out"].clone()
        if a >= 0:
            one = module_for(spec.scaled(n_adapters=1), layer,
                             lora_A=layer.lora_A[a].cuda(), lora_B=layer.lora_B[a].cuda(),
                             lora_A2=layer.lora_A2[a].cuda(), lora_B2=layer.lora_B2[a].cuda())
        else:
            one = module_for(spec.scaled(n_adapters=1), layer, lora_A=None, lora_B=None,
                             lora_A2=None, lora_B2=None)
        ref = one.forward(x, lg)["out"]
        torch.cuda.synchronize()
        assert torch.equal(got, ref), a


def test_zero_tokens_and_no_local_pairs():
    spec, _, layer, _, arr, _ = _setup("ep_lora_small")
    _log("edge T=0 / no local pairs")
    mod = module_for(spec, layer)
    x = torch.zeros(0, spec.H, dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros(0, spec.n_routed + spec.n_sink, device="cuda")
    o = mod.forward(x, lg)
    torch.cuda.synchronize()
    assert o["out"].shape == (0, spec.H)
    # a token whose top-8 are all outside [96, 128): output exactly zero
    b = make_batch(spec, layer, 2)
    lgt = b.logits.clone()
    lgt[:, 96:128] = lgt[:, :256].min(dim=1, keepdim=True).values - 10.0
    o = mod.forward(b.x.cuda(), lgt.cuda())
    torch.cuda.synchronize()
    assert torch.all(o["out"] == 0)
    ids = o["topk_ids"].cpu()
    assert torch.all((ids < 96) | (ids >= 128))


@pytest.mark.parametrize("fmt", ["nvfp4", "mxfp4"])
def test_fp4_small_block_scales_on_gpu(fmt):
    """Block scales at the small end of each format (NVFP4: e4m3 subnormal
    codes 1..7, MXFP4: exponents 104..112), so that many expanded weights
    are f16 subnormals; W13 global scales (2^4, 2^16) bring g and u back
    to their usual size. Checks that the f16 products and the matrix cores
    keep those subnormals exactly."""
    base = SMALL["nvfp4_lora_small" if fmt == "nvfp4" else "mxfp4_small"][0]
    spec = base.scaled(name=f"{fmt}_tiny_scales", cfg_id=46, lora_rank=0, lora_down=False,
                       gscale=True)
    T = 64
    layer = make_layer(spec)
    g = torch.Generator().manual_seed(46)
    sh = layer.w13_s.shape
    if fmt == "nvfp4":
        codes = torch.randint(1, 8, sh, generator=g, dtype=torch.int32).to(torch.uint8)
        layer.w13_s = codes.view(torch.float8_e4m3fn)
        gsv = 2.0 ** 4
    else:
        layer.w13_s = torch.randint(104, 113, sh, generator=g, dtype=torch.int32).to(torch.uint8)
        gsv = 2.0 ** 16
    layer.gs = torch.full((spec.n_groups, 2), gsv, dtype=torch.float32)
    batch = make_batch(spec, layer, T)
    arr, nb = to_numpy_layer(layer), to_numpy_batch(batch)
    _log("fp4-small-scales", fmt, T)
    mod = module_for(spec, layer)
    o = mod.forward(batch.x.cuda(), batch.logits.cuda())
    torch.cuda.synchronize()
    check_layer(spec, o["out"].cpu().numpy(), arr, nb)


@pytest.mark.parametrize("name,log2f", [("fp8_clamp_small", 100), ("fp8_clamp_small", -90),
                                         ("fp8_clamp_decode", 100), ("nvfp4_lora_small", 96),
                                         ("nvfp4_lora_small", -100)])
def test_gemm2_rows_far_from_unit_scale(name, log2f):
    """GEMM2's rows reach the combine as fp16 with a power-of-two scale per
    row and 16 columns. W2 scaled by 2^log2f (FP8: the block scales, NVFP4:
    the per-expert W2 global scales) puts y and the output far outside
    fp16's own range (about 1e30 and 1e-26 here); the output must still meet
    the bar against the oracle, which scales exactly."""
    spec, T = SMALL[name]
    if spec.fmt != "fp8":     # no LoRA: its delta would not scale with W2
        spec = spec.scaled(name=name + "_nolora", lora_rank=0, lora_down=False)
    layer = make_layer(spec)
    batch = make_batch(spec, layer, T)
    nb = to_numpy_batch(batch)
    f = 2.0 ** log2f
    if spec.fmt == "fp8":
        layer.w2_s = (layer.w2_s.double() * f).float()
    else:
        layer.gs2 = (layer.gs2.double() * f).float()
    arr = to_numpy_layer(layer)
    _log("gemm2-row-scale", name, T, log2f)
    mod = module_for(spec, layer)
    o = mod.forward(batch.x.cuda(), batch.logits.cuda(), adapter_ids=_ad(batch))
    torch.cuda.synchronize()
    assert M.moe_read_device_error(o["err_word"]) == 0
    out = o["out"].cpu().numpy()
    assert np.isfinite(out).all()
    ref = check_layer(spec, out, arr, nb)
    assert np.sqrt(np.mean(ref ** 2)) > 0


def test_mxfp4_exponents_outside_the_exact_window_are_flagged():
    """MXFP4 block exponents outside the exactly expanded 104..128 set
    MOE_DEVERR_W4_SCALE (and nothing else); the kernels clamp them to
    99..128, so a layer with some exponents 90 and 131 gives the oracle's
    result for the same layer with those set to 99 and 128."""
    spec = SMALL["mxfp4_small"][0].scaled(name="mxfp4_clamp", cfg_id=50)
    T = 40
    layer = make_layer(spec)
    g = torch.Generator().manual_seed(50)
    s13 = layer.w13_s.clone()
    pick = torch.rand(s13.shape, generator=g)
    s13[pick < 0.01] = 90
    s13[pick > 0.99] = 131
    layer.w13_s = s13
    batch = make_batch(spec, layer, T)
    nb = to_numpy_batch(batch)
    arr = to_numpy_layer(layer)
    arr["w13_s"] = np.clip(arr["w13_s"], 99, 128).astype(np.uint8)
    _log("mxfp4-clamp", T, "exponents 90 / 131:", int((pick < 0.01).sum()), int((pick > 0.99).sum()))
    mod = module_for(spec, layer)
    o = mod.forward(batch.x.cuda(), batch.logits.cuda())
    torch.cuda.synchronize()
    assert M.moe_read_device_error(o["err_word"]) == M.MOE_DEVERR_W4_SCALE
    check_layer(spec, o["out"].cpu().numpy(), arr, nb)


@pytest.mark.parametrize("case", ["int4_scale_big", "int4_scale_tiny", "nvfp4_nan_scale",
                                  "mxfp4a8_nan_scale", "x_beyond_f16", "h_beyond_f16",
                                  "in_range"])
def test_4bit_range_problems_set_error_bits(case):
    """In-range data that the 4-bit kernels cannot expand exactly sets its
    error bit: an INT4 scale of 2^13 or 2^-14, an NVFP4 NaN scale code, an
    activation beyond f16 (1e5, finite in bf16) and an h beyond f16 (huge
    gate and up values). Edge values just inside the ranges set nothing: a
    W2 scale of 8160 and a W13 scale of -2^-13 in every expert, and x =
    65280 in a column whose W13 weights are zero (so h stays ordinary)."""
    _log("4bit-range", case)
    base = {"nvfp4_nan_scale": "nvfp4_lora_small", "mxfp4a8_nan_scale": "mxfp4a8_small"}
    spec = SMALL[base.get(case, "int4_small")][0] \
        .scaled(name=f"range_{case}", cfg_id=52, lora_rank=0, lora_down=False)
    layer = make_layer(spec)
    batch = make_batch(spec, layer, 24)
    x = batch.x.clone()
    want = 0
    if case == "int4_scale_big":          # every expert, so a routed one meets it
        s = layer.w2_s.clone()
        s[:, 3, 1] = 8192.0
        layer.w2_s = s
        want = M.MOE_DEVERR_W4_SCALE
    elif case == "int4_scale_tiny":
        s = layer.w13_s.clone()
        s[:, 7, 2] = 2.0 ** -14
        layer.w13_s = s
        want = M.MOE_DEVERR_W4_SCALE
    elif case == "nvfp4_nan_scale":
        s = layer.w13_s.clone().view(torch.uint8)
        s[:, 5, 3] = 0xFF
        layer.w13_s = s.view(torch.float8_e4m3fn)
        want = M.MOE_DEVERR_W4_SCALE
    elif case == "mxfp4a8_nan_scale":    # e8m0 0xFF (NaN) in the block-scaled GEMM1
        s = layer.w13_s.clone()
        s[:, 5, 3] = 0xFF
        layer.w13_s = s
        want = M.MOE_DEVERR_W4_SCALE
    elif case == "x_beyond_f16":
        x[3, 17] = 1e5
        want = M.MOE_DEVERR_F16_RANGE
    elif case == "h_beyond_f16":
        # every W13 scale of every expert 8160: |g|, |u| in the thousands,
        # so h = silu(g) u reaches far beyond 65504 while the weights expand
        # exactly; x stays N(0, 1)
        layer.w13_s = torch.full_like(layer.w13_s, 8160.0)
        want = M.MOE_DEVERR_F16_RANGE
    else:
        s2 = layer.w2_s.clone()
        s2[:, 0, 0] = 8160.0
        layer.w2_s = s2
        s = layer.w13_s.clone()
        s[:, 1, 0] = -(2.0 ** -13)
        layer.w13_s = s
        q = layer.w13_q.clone()
        q[:, :, 0] = (q[:, :, 0] & 0xF0) | 0x08      # k = 0: nibble 8, weight 0
        layer.w13_q = q
        x[0, 0] = 65280.0
    mod = module_for(spec, layer)
    o = mod.forward(x.cuda(), batch.logits.cuda())
    torch.cuda.synchronize()
    assert M.moe_read_device_error(o["err_word"]) == want
