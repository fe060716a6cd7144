"""Seeded synthetic inputs for the routed MoE expert-FFN path.

This module only DRAWS inputs: random activations, router logits and expert
weights stored in the formats the path consumes (bf16, fp8-e4m3 with fp32
128x128 block scales, packed int4 with bf16 group-32 scales, packed e2m1
with e4m3 block-16 or e8m0 block-32 scales). It holds none of
the path's arithmetic: no routing, no permutation, no activation quantisation,
no GEMM, no SwiGLU, no combine. Weight quantisation to e4m3 uses torch's own
float8_e4m3fn conversion, as an offline quantiser would.

Both the HIP path (tests, bench) and the CPU oracle consume what this module
returns; neither is imported here.

Workload shapes follow the MoE layers named on the pages:
  * GLM-5.3-Flash FP8 layer (blockwise 128x128 FP8, 288 routed experts, top-8,
    one shared expert, swiglu_limit 10) -- sglang PR #39920, "Motivation".
  * MiniMax-M3 OAI-SwiGLU (alpha 1.702, up_bias 1.0, clamp 7.0) -- DeepGEMM
    PR #445, "Summary".
  * INT4 group-32 weights, w_packed [N, K/2] u8 with low nibble = even K and
    scale [N, K/32] bf16 -- batchgen PR #239, commit text.
  * NVFP4 expert weights with distinct per-half global scales -- the
    MoE-LoRA release notes, "Changes since 1b699bf" (and MXFP4 at the INT4
    layer's shape).
  * Inkling [T, 258] gate rows (256 routed + 2 shared-sink columns) with ties,
    all-negative rows and a dominating sink -- sglang PR #36385, "Correctness".
  * distinct gate/up global scales with up/gate ratio 0.52-1.22 and a rank-16
    LoRA, on one expert-parallel rank's share -- FlashInfer MoE-LoRA AOT
    release notes, "Changes since 1b699bf".
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

FMT_BF16 = "bf16"
FMT_FP8 = "fp8"
FMT_INT4 = "int4"
FMT_NVFP4 = "nvfp4"
FMT_MXFP4 = "mxfp4"
# MXFP4 weights with MXFP8 activations into GEMM1 (block-scaled matrix
# instructions); the weights are stored exactly as for FMT_MXFP4
FMT_MXFP4_A8 = "mxfp4_a8"
FP4_FORMATS = (FMT_NVFP4, FMT_MXFP4, FMT_MXFP4_A8)


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    cfg_id: int
    fmt: str
    H: int
    I: int
    n_routed: int            # routed experts, global count (E)
    top_k: int
    n_sink: int = 0          # trailing shared-sink logit columns
    E_loc: Optional[int] = None   # local experts on this GPU (None: all)
    offset: int = 0          # local_expert_offset
    shared: int = 0          # 1: one always-on shared expert
    alpha: float = 1.0
    beta: float = 0.0
    limit: float = math.inf
    route_scale: float = 1.0
    global_scale: float = 1.0
    shared_w: float = 1.0
    lora_rank: int = 0
    lora_scale: float = 1.0
    lora_down: bool = False  # the same adapter also carries a down-projection LoRA
    n_adapters: int = 1      # a batch of adapters: per-token ids in [-1, n_adapters)
    gscale: bool = False     # per-expert (gate, up) global scales
    logits: str = "normal"   # normal | skewed | router | mix258
    w13_std: Optional[float] = None
    w2_std: Optional[float] = None
    Ts: tuple = ()

    @property
    def n_local(self) -> int:
        return self.n_routed if self.E_loc is None else self.E_loc

    @property
    def n_groups(self) -> int:
        return self.n_local + self.shared

    def scaled(self, **kw) -> "LayerSpec":
        return dataclasses.replace(self, **kw)


# The five workloads. Sizes and value recipes are the ones the layer
# descriptions above fix; where a page gives no distribution the choice is
# stated in the design notes.
CONFIGS = {
    "tiny_bf16": LayerSpec(
        name="tiny_bf16", cfg_id=1, fmt=FMT_BF16, H=256, I=128, n_routed=8,
        top_k=2, logits="router", w13_std=0.02, w2_std=0.02, Ts=(16,)),
    "fp8_clamp_288": LayerSpec(
        name="fp8_clamp_288", cfg_id=2, fmt=FMT_FP8, H=6144, I=2048,
        n_routed=288, top_k=8, shared=1, limit=10.0, Ts=(1, 64, 4096)),
    "fp8_oai_128_skew": LayerSpec(
        name="fp8_oai_128_skew", cfg_id=3, fmt=FMT_FP8, H=3072, I=1536,
        n_routed=128, top_k=4, alpha=1.702, beta=1.0, limit=7.0,
        logits="skewed", Ts=(1, 64, 4096)),
    "int4_g32_64": LayerSpec(
        name="int4_g32_64", cfg_id=4, fmt=FMT_INT4, H=2048, I=768,
        n_routed=64, top_k=8, Ts=(1, 64, 2048)),
    "ep_lora_258": LayerSpec(
        name="ep_lora_258", cfg_id=5, fmt=FMT_FP8, H=2048, I=1024,
        n_routed=256, n_sink=2, top_k=8, E_loc=32, offset=96, lora_rank=16,
        gscale=True, logits="mix258", Ts=(1, 37, 512, 8192)),
}

# The expert-parallel LoRA layer with the same adapter also on the down
# projection (its input is the SwiGLU output in true units: the MoE-LoRA
# release notes, "Changes since 1b699bf"). Same seeds as ep_lora_258, so the
# base weights and the up LoRA are identical.
EXT_CONFIGS = {
    "ep_lora_258_down": CONFIGS["ep_lora_258"].scaled(
        name="ep_lora_258_down", lora_down=True),
}

# The same expert-parallel LoRA layer in the weight format the MoE-LoRA
# release serves (NVFP4 with distinct gate/up global scales), and the INT4
# layer's shape with MXFP4 weights.
FP4_CONFIGS = {
    "nvfp4_lora_258": LayerSpec(
        name="nvfp4_lora_258", cfg_id=6, fmt=FMT_NVFP4, H=2048, I=1024,
        n_routed=256, n_sink=2, top_k=8, E_loc=32, offset=96, lora_rank=16,
        lora_down=True,
        gscale=True, logits="mix258", Ts=(1, 37, 512, 8192)),
    "mxfp4_g32_64": LayerSpec(
        name="mxfp4_g32_64", cfg_id=7, fmt=FMT_MXFP4, H=2048, I=768,
        n_routed=64, top_k=8, Ts=(1, 64, 2048)),
}
# The same MXFP4 layer (same seeds: identical weights and inputs) with its
# activations entering GEMM1 as MXFP8, on the block-scaled matrix cores
FP4_CONFIGS["mxfp4a8_g32_64"] = FP4_CONFIGS["mxfp4_g32_64"].scaled(
    name="mxfp4a8_g32_64", fmt=FMT_MXFP4_A8)


def _seed(*parts: int) -> int:
    ss = np.random.SeedSequence([int(p) & 0xFFFFFFFF for p in parts])
    st = ss.generate_state(2, dtype=np.uint32)
    return int(st[0]) | (int(st[1] & 0x7FFFFFFF) << 32)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _fp8_block_quant(w: torch.Tensor):
    """Offline quantiser used to STORE synthetic weights: per 128x128 block,
    scale = amax/448, code = torch's round-to-nearest-even e4m3fn conversion."""
    N, K = w.shape
    blk = w.reshape(N // 128, 128, K // 128, 128)
    amax = blk.abs().amax(dim=(1, 3)).float()
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (blk / s[:, None, :, None]).reshape(N, K).to(torch.float8_e4m3fn)
    return q, s


@dataclasses.dataclass
class Layer:
    spec: LayerSpec
    w13_q: torch.Tensor           # [G, 2I, H] (bf16 | e4m3fn) or [G, 2I, H/2] u8
    w13_s: Optional[torch.Tensor]  # fp8: [G, 2I/128, H/128] f32; int4: [G, 2I, H/32] bf16;
                                   # nvfp4: [G, 2I, H/16] e4m3fn; mxfp4: [G, 2I, H/32] u8
    w2_q: torch.Tensor            # [G, H, I] or [G, H, I/2] u8
    w2_s: Optional[torch.Tensor]
    gs: Optional[torch.Tensor]    # [G, 2] f32 (gate, up) or None
    lora_A: Optional[torch.Tensor]  # [n_local, r, H] bf16 (routed experts only)
    lora_B: Optional[torch.Tensor]  # [n_local, 2I, r] bf16
    w_router: Optional[torch.Tensor]  # [H, E] f64 (router GEMM input recipe)
    lora_A2: Optional[torch.Tensor] = None  # [n_local, r, I] bf16 (down LoRA)
    lora_B2: Optional[torch.Tensor] = None  # [n_local, H, r] bf16
    gs2: Optional[torch.Tensor] = None      # [G] f32 W2 global scales (NVFP4)


@dataclasses.dataclass
class Batch:
    T: int
    x: torch.Tensor        # [T, H] bf16
    logits: torch.Tensor   # [T, n_routed + n_sink] f32
    adapter_ids: Optional[torch.Tensor] = None   # [T] int32 (a batch of adapters)


def _rand_weights(spec: LayerSpec, N: int, K: int, std: float, gen, device,
                  half_scale: Optional[torch.Tensor] = None,
                  fp4_scale_codes: tuple = (0x30, 0x68)):
    """One expert's [N, K] matrix in the spec's storage format."""
    if spec.fmt == FMT_BF16:
        w = torch.randn(N, K, generator=gen, device=device) * std
        return w.to(torch.bfloat16), None
    if spec.fmt == FMT_FP8:
        w = torch.randn(N, K, generator=gen, device=device) * std
        if half_scale is not None:
            # stored weight = W_true / gs_half, one scale per half of the rows
            w = w / half_scale.repeat_interleave(N // half_scale.numel())[:, None]
        return _fp8_block_quant(w)
    if spec.fmt == FMT_INT4:
        q = torch.randint(0, 256, (N, K // 2), generator=gen, device=device,
                          dtype=torch.int32).to(torch.uint8)
        s = (torch.rand(N, K // 32, generator=gen, device=device) * 0.015
             + 0.005).to(torch.bfloat16)
        return q, s
    if spec.fmt in FP4_FORMATS:
        # uniform e2m1 codes (RMS 2.93); the scale codes set the magnitude
        q = torch.randint(0, 256, (N, K // 2), generator=gen, device=device,
                          dtype=torch.int32).to(torch.uint8)
        if spec.fmt == FMT_NVFP4:
            # e4m3 codes lo..hi-1 (W13: 0.5 .. 120, W2: 0.25 .. 60); the
            # global scales bring the weights to their usual size, as an
            # NVFP4 quantiser's amax / (6 * 448) does
            lo, hi = fp4_scale_codes
            s = torch.randint(lo, hi, (N, K // 16), generator=gen, device=device,
                              dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
        else:
            # e8m0 exponents 119..123: 2^-8 .. 2^-4
            s = torch.randint(119, 124, (N, K // 32), generator=gen, device=device,
                              dtype=torch.int32).to(torch.uint8)
        return q, s
    raise ValueError(spec.fmt)


def make_layer(spec: LayerSpec, device="cpu") -> Layer:
    H, I, G = spec.H, spec.I, spec.n_groups
    std13 = spec.w13_std if spec.w13_std is not None else 4.0 / math.sqrt(H)
    std2 = spec.w2_std if spec.w2_std is not None else 1.0 / math.sqrt(I)
    gs = None
    if spec.gscale:
        g = _gen(device, spec.cfg_id, 7001)
        gate = torch.rand(G, generator=g, device=device) * 1.5 + 0.5
        ratio = torch.rand(G, generator=g, device=device) * 0.70 + 0.52
        gs = torch.stack([gate, gate * ratio], dim=1).float()
        if spec.fmt == FMT_NVFP4:
            gs = gs * 2.0 ** -9      # NVFP4 block scales are in the tens
        gs = gs.contiguous()
    q13, s13, q2, s2 = [], [], [], []
    for e in range(G):
        g = _gen(device, spec.cfg_id, 1000 + e)
        a, b = _rand_weights(spec, 2 * I, H, std13, g, device,
                             None if gs is None else gs[e])
        c, d = _rand_weights(spec, H, I, std2, g, device, fp4_scale_codes=(0x28, 0x60))
        q13.append(a); s13.append(b); q2.append(c); s2.append(d)
    st = lambda xs: None if xs[0] is None else torch.stack(xs).contiguous()
    # LoRA covers the local routed experts (the shared expert carries none);
    # a batch of adapters stacks them first: [n_adapters, n_local, ...]
    na = spec.n_adapters
    lead = (spec.n_local,) if na == 1 else (na, spec.n_local)
    lora_A = lora_B = None
    if spec.lora_rank:
        r = spec.lora_rank
        g = _gen(device, spec.cfg_id, 7002)
        lora_A = (torch.randn(*lead, r, H, generator=g, device=device)
                  / math.sqrt(H)).to(torch.bfloat16)
        # RMS(x.A^T) ~ 1 and RMS(g) ~ 4 (std13 * sqrt(H)); B std 0.5 gives
        # RMS(delta) ~ sqrt(r) * 0.5 = 2 ~ 0.5 * RMS(g).
        lora_B = (torch.randn(*lead, 2 * I, r, generator=g, device=device)
                  * 0.5).to(torch.bfloat16)
    w_router = None
    if spec.logits == "router":
        g = _gen("cpu", spec.cfg_id, 7003)
        w_router = torch.randn(H, spec.n_routed, generator=g,
                               dtype=torch.float64) * 0.02
    lora_A2 = lora_B2 = None
    if spec.lora_rank and spec.lora_down:
        r = spec.lora_rank
        g = _gen(device, spec.cfg_id, 7006)
        # RMS(h A2^T) ~ RMS(h) ~ RMS(y); B2 std 0.5 / sqrt(r) gives a delta
        # of about half the base down-projection output
        lora_A2 = (torch.randn(*lead, r, I, generator=g, device=device)
                   / math.sqrt(I)).to(torch.bfloat16)
        lora_B2 = (torch.randn(*lead, H, r, generator=g, device=device)
                   * (0.5 / math.sqrt(r))).to(torch.bfloat16)
    gs2 = None
    if spec.fmt == FMT_NVFP4:
        g = _gen(device, spec.cfg_id, 7007)
        gs2 = ((torch.rand(G, generator=g, device=device) + 0.5)
               * 2.0 ** -10).float().contiguous()
    return Layer(spec, st(q13), st(s13), st(q2), st(s2), gs, lora_A, lora_B,
                 w_router, lora_A2, lora_B2, gs2)


def _logits_mix258(spec: LayerSpec, T: int, g, device) -> torch.Tensor:
    """Row mix for the [T, 256 + 2] gate: plain N(0,1) rows, rows with every
    logit below -110, rows near -90 (fp32 sigmoid subnormal), tie rows with
    4 distinct values over the routed columns, and rows whose sink dominates."""
    N, S = spec.n_routed, spec.n_sink
    out = torch.randn(T, N + S, generator=g, device=device)
    kind = torch.randint(0, 8, (T,), generator=g, device=device)
    if T >= 5:   # make sure every kind appears in small batches too
        kind[:5] = torch.tensor([1, 2, 3, 4, 5], device=device)
    z = torch.randn(T, N + S, generator=g, device=device)
    neg200 = -200.0 + z
    neg111 = -111.0 - 5.0 * z.abs()
    neg90 = -90.0 + 0.5 * z
    vals = torch.tensor([-1.5, 0.25, 0.75, 2.0], device=device)
    tie_idx = torch.randint(0, 4, (T, N + S), generator=g, device=device)
    ties = vals[tie_idx]
    sink = out.clone()           # sink outranks every routed column
    sink[:, :N] -= 8.0
    sink[:, N:] += 30.0
    out = torch.where((kind == 1)[:, None], neg200, out)
    out = torch.where((kind == 2)[:, None], neg111, out)
    out = torch.where((kind == 3)[:, None], neg90, out)
    out = torch.where((kind == 4)[:, None], ties, out)
    out = torch.where((kind == 5)[:, None], sink, out)
    return out.float().contiguous()


def make_tokens(spec: LayerSpec, T: int, device="cpu", seed_extra: int = 0) -> torch.Tensor:
    """The activations x [T, H] bf16 of make_batch alone (same draw)."""
    g = _gen(device, spec.cfg_id, T, 11 + seed_extra)
    return torch.randn(T, spec.H, generator=g, device=device).to(torch.bfloat16).contiguous()


def make_batch(spec: LayerSpec, layer: Optional[Layer], T: int,
               device="cpu", seed_extra: int = 0) -> Batch:
    g = _gen(device, spec.cfg_id, T, 11 + seed_extra)
    x = torch.randn(T, spec.H, generator=g, device=device).to(torch.bfloat16)
    N, S = spec.n_routed, spec.n_sink
    if spec.logits == "router":
        lg = (x.double().cpu() @ layer.w_router).float().to(device)
    elif spec.logits == "skewed":
        lg = torch.randn(T, N + S, generator=g, device=device)
        gh = _gen("cpu", spec.cfg_id, 7004)
        hot = torch.randperm(N, generator=gh)[:8].to(device)
        lg[:, hot] += 3.0
    elif spec.logits == "mix258":
        lg = _logits_mix258(spec, T, g, device)
    else:
        lg = torch.randn(T, N + S, generator=g, device=device)
    ad = None
    if spec.lora_rank and spec.n_adapters > 1:
        # each token picks one of the adapters or none (-1), uniformly
        ga = _gen(device, spec.cfg_id, T, 13 + seed_extra)
        ad = (torch.randint(0, spec.n_adapters + 1, (T,), generator=ga, device=device)
              - 1).to(torch.int32).contiguous()
    return Batch(T, x.contiguous(), lg.float().contiguous(), ad)


@dataclasses.dataclass
class Gate:
    wg: torch.Tensor      # [n_routed + n_sink, H] bf16 router weight
    bias: torch.Tensor    # [n_routed] f32 selection bias


def make_gate(spec: LayerSpec, device="cpu", logit_std: float = 1.0,
              bias_amp: float = 0.02) -> Gate:
    """Router weight and selection bias for the gate GEMM. The pages fix the
    shape ([T, N + S] gate rows from an [N + S, H] weight) but no values:
    Wg ~ N(0, (logit_std / sqrt(H))^2) in bf16 gives N(0, logit_std^2)
    logits for N(0, 1) activations; the bias is U(-bias_amp, bias_amp), the
    size of the gaps between the top sigmoid values at logit_std 1, so it
    changes some selections and not others."""
    g = _gen(device, spec.cfg_id, 7005)
    N, S, H = spec.n_routed, spec.n_sink, spec.H
    wg = (torch.randn(N + S, H, generator=g, device=device)
          * (logit_std / math.sqrt(H))).to(torch.bfloat16)
    bias = (torch.rand(N, generator=g, device=device) * 2.0 - 1.0) * bias_amp
    return Gate(wg.contiguous(), bias.float().contiguous())


def to_numpy_layer(layer: Layer, experts=None) -> dict:
    """Host copies of the stored arrays, as raw codes: bf16 -> uint16 bits,
    e4m3fn -> uint8 codes. `experts` limits the copy to some groups."""
    def cp(t):
        if t is None:
            return None
        if experts is not None:
            t = t[experts]
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).numpy()
        return t.numpy()
    return {k: cp(getattr(layer, k)) for k in
            ("w13_q", "w13_s", "w2_q", "w2_s", "gs", "lora_A", "lora_B",
             "lora_A2", "lora_B2", "gs2")}


def to_numpy_batch(batch: Batch) -> dict:
    return {
        "x_bits": batch.x.detach().cpu().contiguous().view(torch.int16)
                  .numpy().view(np.uint16),
        "logits": batch.logits.detach().cpu().numpy(),
        "adapter_ids": (None if batch.adapter_ids is None
                        else batch.adapter_ids.detach().cpu().numpy()),
    }
