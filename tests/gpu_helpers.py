"""Glue between the seeded inputs (synth) and the C-ABI binding, plus the
parity metrics used by the GPU tests and the bench."""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_expert_sigmoid_amd as M
from synth import Layer, LayerSpec

FMT = {"bf16": M.MOE_W_BF16, "fp8": M.MOE_W_FP8_B128, "int4": M.MOE_W_INT4_G32,
       "nvfp4": M.MOE_W_NVFP4, "mxfp4": M.MOE_W_MXFP4}


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
    FP4 formats, 4-bit weights with bf16 activations like INT4, take INT4's);
    BF16 max|err| <= 5e-3 RMS."""
    return (5e-3, 0.9999) if fmt == "bf16" else (1e-2, 0.9999)
