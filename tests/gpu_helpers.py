"""Glue between the seeded inputs (synth) and the C-ABI binding, plus the
parity metrics used by the GPU tests and the bench."""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_expert_sigmoid_amd as M
from synth import Layer, LayerSpec

FMT = {"bf16": M.MOE_W_BF16, "fp8": M.MOE_W_FP8_B128, "int4": M.MOE_W_INT4_G32,
       "nvfp4": M.MOE_W_NVFP4, "mxfp4": M.MOE_W_MXFP4, "mxfp4_a8": M.MOE_W_MXFP4_A8}


def _dev(t):
    if t is None:
        return None
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    return t.to("cuda").contiguous()


def module_for(spec: LayerSpec, layer: Layer, **over) -> M.MoeModule:
    kw = dict(
        fmt=FMT[spec.fmt], H=spec.H, I=spec.I, num_experts_global=spec.n_routed,
        top_k=spec.top_k, w13_q=_dev(layer.w13_q), w2_q=_dev(layer.w2_q),
        w13_s=_dev(layer.w13_s), w2_s=_dev(layer.w2_s), gscale=_dev(layer.gs),
        gscale2=_dev(layer.gs2),
        num_local_experts=spec.n_local, local_expert_offset=spec.offset,
        shared_expert=spec.shared, n_sink=spec.n_sink,
        route_scale=spec.route_scale, global_scale=spec.global_scale,
        shared_w=spec.shared_w, alpha=spec.alpha, beta=spec.beta,
        limit=spec.limit, lora_A=_dev(layer.lora_A), lora_B=_dev(layer.lora_B),
        lora_scale=spec.lora_scale, lora_A2=_dev(layer.lora_A2),
        lora_B2=_dev(layer.lora_B2))
    kw.update(over)
    return M.MoeModule(**kw)


class LazyExperts:
    """Per-group host copies of a (possibly device-resident) layer, fetched on
    demand, for the oracle's expert-at-a-time loop."""

    def __init__(self, layer: Layer):
        self.layer = layer

    def __getitem__(self, name):
        t = getattr(self.layer, name)
        if t is None:
            return None
        return _Rows(t)

    def get(self, name, default=None):
        return self[name] if getattr(self.layer, name) is not None else default


class _Rows:
    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        x = self.t[e].detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy().view(np.uint16)
        if x.dtype == torch.float8_e4m3fn:
            return x.view(torch.uint8).numpy()
        return x.numpy()


def compare(out_gpu: np.ndarray, ref: np.ndarray):
    """max |err| / RMS(ref) and cosine similarity."""
    ref = np.asarray(ref, np.float64)
    got = np.asarray(out_gpu, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    nr, ng = np.linalg.norm(ref), np.linalg.norm(got)
    cos = float(np.dot(ref.ravel(), got.ravel()) / (nr * ng)) if nr > 0 and ng > 0 else \
        (1.0 if nr == ng else 0.0)
    return err / rms if rms > 0 else err, cos


def tolerance(fmt: str):
    """Output bars: FP8/INT4 max|err| <= 1e-2 RMS and cosine >= 0.9999 (the
    FP4 formats, 4-bit weights like INT4, take INT4's); BF16 max|err| <=
    5e-3 RMS."""
    return (5e-3, 0.9999) if fmt == "bf16" else (1e-2, 0.9999)


class StepCalls:
    """The path through its individual C-ABI entry points (route ->
    permute -> activation quant -> GEMM1 + act -> GEMM2 + combine) on one
    batch, with every buffer allocated once; each step is a callable, so
    the steps can be run in order or timed one by one."""

    def __init__(self, spec: LayerSpec, mod: M.MoeModule, x, logits, adapter_ids=None):
        T = x.shape[0]
        mod.set_adapters(adapter_ids)
        self.spec, self.mod, self.T, self.x, self.lg = spec, mod, T, x, logits
        k, S, H, I = spec.top_k, spec.n_sink, spec.H, spec.I
        G = spec.n_groups
        self.fp8 = fp8 = spec.fmt == "fp8"
        self.mx = mx = spec.fmt == "mxfp4_a8"
        dev32 = dict(device="cuda", dtype=torch.int32)
        self.ids = torch.empty(T, k, **dev32)
        self.w = torch.empty(T, k, device="cuda")
        self.sw = torch.empty(T, S, device="cuda") if S else None
        self.pc = pc = T * k + (T if spec.shared else 0)
        self.offsets = torch.empty(G + 1, **dev32)
        self.sp = torch.empty(pc, **dev32)
        self.pr = torch.empty(pc, **dev32)
        self.err = torch.zeros(1, **dev32)
        self.wsp = torch.empty(M.moe_permute_workspace_size(T, k, G), dtype=torch.uint8,
                               device="cuda")
        if fp8:
            self.xin = torch.empty(T, H, dtype=torch.uint8, device="cuda")
            self.xs = torch.empty(T, H // 128, device="cuda")
            self.h = torch.empty(pc, I, dtype=torch.uint8, device="cuda")
            self.hs = torch.empty(pc, I // 128, device="cuda")
        else:
            self.xin, self.xs = x, None
            if mx:   # MXFP8 activation codes and their e8m0 codes
                self.xin = torch.empty(T, H, dtype=torch.uint8, device="cuda")
                self.xs = torch.empty(T, H // 32, dtype=torch.uint8, device="cuda")
            # rows of other ranks' experts stay 0
            self.h = torch.zeros(pc, I, dtype=torch.bfloat16, device="cuda")
            self.hs = None
        self.ws1 = torch.empty(max(M.moe_gemm1_workspace_size(mod.w13, pc, mod.lora), 1),
                               dtype=torch.uint8, device="cuda")
        # the down-LoRA input: FP8 layers write it beside the codes, the
        # others read h itself
        self.h_lora = None
        if mod.lora_down is not None:
            self.h_lora = (torch.zeros(pc, I, dtype=torch.bfloat16, device="cuda") if fp8
                           else self.h)
        self.out = torch.empty(T, H, device="cuda")
        self.ws2 = torch.empty(M.moe_gemm2_workspace_size(mod.w2, pc, mod.lora_down),
                               dtype=torch.uint8, device="cuda")

    def route(self):
        s = self.spec
        M.moe_route(self.lg, s.n_routed, s.n_sink, s.top_k, s.route_scale, s.global_scale,
                    self.ids, self.w, self.sw)

    def permute(self):
        s = self.spec
        M.moe_permute(self.ids, s.top_k, s.n_routed, s.offset, s.n_local, s.shared,
                      self.offsets, self.sp, self.pr, self.err, self.wsp)

    def quant(self):
        if self.fp8:
            M.moe_quantize_act_fp8(self.x, self.xin, self.xs)
        elif self.mx:
            M.moe_quantize_act_mxfp8(self.x, self.xin, self.xs)

    def gemm1(self):
        s, m = self.spec, self.mod
        M.moe_grouped_gemm1_act(m.w13, self.xin, self.xs, self.x, self.T, s.H, s.I, s.top_k,
                                self.pc, self.offsets, self.sp, m.act, m.lora, self.h, self.hs,
                                self.ws1, h_lora=self.h_lora if self.fp8 else None,
                                err_word=self.err)

    def gemm2(self):
        s, m = self.spec, self.mod
        M.moe_grouped_gemm2_combine(m.w2, self.h, self.hs, self.T, s.H, s.I, s.top_k,
                                    s.shared, self.pc, self.offsets, self.pr, self.w,
                                    s.shared_w, self.out, self.ws2, h_lora=self.h_lora,
                                    lora_down=m.lora_down, sorted_pair=self.sp,
                                    err_word=self.err)

    def steps(self):
        return [("route", self.route), ("permute", self.permute), ("quant", self.quant),
                ("gemm1", self.gemm1), ("gemm2_combine", self.gemm2)]

    def run(self):
        for _, f in self.steps():
            f()
