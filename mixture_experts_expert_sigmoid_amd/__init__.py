"""Python binding of libmoe_mi355x.so: the routed MoE expert-FFN hot path
on MI355X (gfx950).

Argument marshalling only. Every step of the path runs in the library's HIP
kernels; torch supplies device memory (tensors) and the current stream. The
functions carry the C names (moe_route, moe_permute, moe_quantize_act_fp8,
moe_quantize_act_mxfp8,
moe_grouped_gemm1_act, moe_grouped_gemm2_combine, moe_forward, ...), take
torch tensors for the arrays, and raise MoeError on a negative status.
There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import POINTER, c_float, c_int, c_long, c_size_t, c_void_p
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe_mi355x.h")

MOE_W_BF16, MOE_W_FP8_B128, MOE_W_INT4_G32, MOE_W_NVFP4, MOE_W_MXFP4 = 0, 1, 2, 3, 4
MOE_W_MXFP4_A8 = 5
_PACKED4 = (MOE_W_INT4_G32, MOE_W_NVFP4, MOE_W_MXFP4, MOE_W_MXFP4_A8)
MOE_DEVERR_GLOBAL_ID_OOB = 0x1
MOE_DEVERR_F16_RANGE = 0x2
MOE_DEVERR_W4_SCALE = 0x4
STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE",
          -3: "MOE_ERR_FORMAT", -4: "MOE_ERR_LOCAL_RANGE", -5: "MOE_ERR_PARAM",
          -6: "MOE_ERR_WORKSPACE", -8: "MOE_ERR_HIP", -9: "MOE_ERR_SCRATCH"}
MOE_SCRATCH_BYTES = 32 << 20


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")
        self.status = status


class MoeActParams(ctypes.Structure):
    _fields_ = [("alpha", c_float), ("beta", c_float), ("limit", c_float)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("fmt", c_int), ("n_groups", c_int), ("N", c_int), ("K", c_int),
                ("q", c_void_p), ("scale", c_void_p), ("gscale", c_void_p)]


class MoeLora(ctypes.Structure):
    _fields_ = [("rank", c_int), ("n_groups", c_int), ("scale", c_float),
                ("A", c_void_p), ("B", c_void_p), ("n_adapters", c_int),
                ("adapter_ids", c_void_p)]


class MoeLayer(ctypes.Structure):
    _fields_ = [("H", c_int), ("I", c_int), ("num_experts_global", c_int),
                ("num_local_experts", c_int), ("local_expert_offset", c_int),
                ("shared_expert", c_int), ("top_k", c_int), ("n_sink", c_int),
                ("route_scale", c_float), ("global_scale", c_float),
                ("shared_w", c_float), ("w13", MoeWeights), ("w2", MoeWeights),
                ("act", MoeActParams), ("lora", POINTER(MoeLora)),
                ("lora_down", POINTER(MoeLora))]


_lib = None

_SIGS = {
    "moe_route": (c_int, [c_void_p, c_long, c_long, c_int, c_int, c_int, c_void_p,
                          c_float, c_float, c_void_p, c_void_p, c_void_p, c_void_p,
                          c_void_p]),
    "moe_gate_route_workspace_size": (c_size_t, [c_long, c_int, c_int, c_int]),
    "moe_gate_route": (c_int, [c_void_p, c_void_p, c_long, c_int, c_int, c_int, c_int,
                               c_void_p, c_float, c_float, c_void_p, c_void_p,
                               c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                               c_void_p]),
    "moe_permute": (c_int, [c_void_p, c_long, c_int, c_int, c_int, c_int, c_int,
                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_size_t, c_void_p]),
    "moe_permute_workspace_size": (c_size_t, [c_long, c_int, c_int]),
    "moe_quantize_act_fp8": (c_int, [c_void_p, c_long, c_int, c_void_p, c_void_p,
                                     c_void_p]),
    "moe_quantize_act_mxfp8": (c_int, [c_void_p, c_long, c_int, c_void_p, c_void_p,
                                       c_void_p]),
    "moe_grouped_gemm1_act": (c_int, [POINTER(MoeWeights), c_void_p, c_void_p,
                                      c_void_p, c_long, c_int, c_int, c_int,
                                      c_long, c_void_p, c_void_p,
                                      POINTER(MoeActParams), POINTER(MoeLora),
                                      c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_size_t, c_void_p]),
    "moe_gemm1_workspace_size": (c_size_t, [POINTER(MoeWeights), c_long, POINTER(MoeLora)]),
    "moe_grouped_gemm2_combine": (c_int, [POINTER(MoeWeights), c_void_p, c_void_p,
                                          c_void_p, POINTER(MoeLora),
                                          c_long, c_int, c_int, c_int, c_int,
                                          c_long, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_float, c_void_p, c_void_p,
                                          c_void_p, c_size_t, c_void_p]),
    "moe_gemm2_workspace_size": (c_size_t, [POINTER(MoeWeights), c_long,
                                            POINTER(MoeLora)]),
    "moe_forward": (c_int, [POINTER(MoeLayer), c_void_p, c_void_p, c_long, c_long,
                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_void_p, c_size_t, c_void_p]),
    "moe_workspace_size": (c_size_t, [POINTER(MoeLayer), c_long]),
    "moe_forward_no_workspace": (c_int, [POINTER(MoeLayer), c_void_p, c_void_p, c_long,
                                         c_long, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p]),
    "moe_scratch_error": (ctypes.c_char_p, []),
    "moe_read_device_error": (c_int, [c_void_p, POINTER(c_int), c_void_p]),
    "moe_status_string": (ctypes.c_char_p, [c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
}


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m mixture_experts_expert_sigmoid_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        L = lib()
        raise MoeError(status, where, L.moe_status_string(status).decode()
                       + ("; " + L.moe_last_error().decode() if status == -8 else ""))


# ---------------------------------------------------------------- descriptors

def weights(fmt: int, q: torch.Tensor, scale: Optional[torch.Tensor] = None,
            gscale: Optional[torch.Tensor] = None) -> MoeWeights:
    """Descriptor of a stacked [G][N][K] weight (4-bit formats: q is
    [G][N][K/2]). gscale: W13 [G][2] (gate, up), W2 [G] (FP4 formats)."""
    G, N, Kq = q.shape
    K = 2 * Kq if fmt in _PACKED4 else Kq
    w = MoeWeights(fmt, G, N, K, q.data_ptr(),
                   None if scale is None else scale.data_ptr(),
                   None if gscale is None else gscale.data_ptr())
    w._keep = (q, scale, gscale)
    return w


def act_params(alpha=1.0, beta=0.0, limit=math.inf) -> MoeActParams:
    return MoeActParams(alpha, beta, limit)


def lora_desc(A: torch.Tensor, B: torch.Tensor, scale=1.0,
              adapter_ids: Optional[torch.Tensor] = None) -> MoeLora:
    """A [G][r][K] (one adapter) or [n_adapters][G][r][K] (a batch, with
    per-token adapter_ids int32 [T] set here or per call)."""
    na = 1 if A.dim() == 3 else A.shape[0]
    G, r = A.shape[-3], A.shape[-2]
    d = MoeLora(r, G, scale, A.data_ptr(), B.data_ptr(), na,
                None if adapter_ids is None else adapter_ids.data_ptr())
    d._keep = (A, B, adapter_ids)
    return d


def layer_desc(H, I, num_experts_global, num_local_experts, local_expert_offset,
               shared_expert, top_k, n_sink, route_scale, global_scale, shared_w,
               w13: MoeWeights, w2: MoeWeights, act: MoeActParams,
               lora: Optional[MoeLora] = None,
               lora_down: Optional[MoeLora] = None) -> MoeLayer:
    L = MoeLayer(H, I, num_experts_global, num_local_experts, local_expert_offset,
                 shared_expert, top_k, n_sink, route_scale, global_scale,
                 shared_w, w13, w2, act, _lp(lora), _lp(lora_down))
    L._keep = (w13, w2, lora, lora_down)
    return L


# ------------------------------------------------------------ entry points

def moe_route(logits, n_routed, n_sink, top_k, route_scale, global_scale,
              topk_ids, topk_w, sink_w=None, stream=None, sel_bias=None,
              packed=None):
    T, ld = logits.shape
    _check(lib().moe_route(_p(logits), T, logits.stride(0), n_routed, n_sink,
                           top_k, _p(sel_bias), route_scale, global_scale,
                           _p(topk_ids), _p(topk_w), _p(sink_w), _p(packed),
                           _stream(stream)), "moe_route")


def moe_gate_route_workspace_size(T, H, n_routed, n_sink) -> int:
    return lib().moe_gate_route_workspace_size(T, H, n_routed, n_sink)


def moe_gate_route(x_bf16, wg_bf16, n_routed, n_sink, top_k, route_scale,
                   global_scale, topk_ids, topk_w, sink_w=None, sel_bias=None,
                   logits=None, packed=None, ws=None, stream=None):
    T, H = x_bf16.shape
    _check(lib().moe_gate_route(_p(x_bf16), _p(wg_bf16), T, H, n_routed, n_sink,
                                top_k, _p(sel_bias), route_scale, global_scale,
                                _p(logits), _p(topk_ids), _p(topk_w), _p(sink_w),
                                _p(packed), _p(ws),
                                0 if ws is None else ws.numel() * ws.element_size(),
                                _stream(stream)), "moe_gate_route")


def moe_permute_workspace_size(T, top_k, n_groups) -> int:
    return lib().moe_permute_workspace_size(T, top_k, n_groups)


def moe_permute(topk_ids, top_k, num_experts_global, local_expert_offset,
                num_local_experts, shared_expert, offsets, sorted_pair, pair_row,
                err_word, ws, stream=None):
    T = topk_ids.shape[0]
    _check(lib().moe_permute(_p(topk_ids), T, top_k, num_experts_global,
                             local_expert_offset, num_local_experts,
                             shared_expert, _p(offsets), _p(sorted_pair),
                             _p(pair_row), _p(err_word), _p(ws),
                             ws.numel() * ws.element_size(), _stream(stream)),
           "moe_permute")


def moe_quantize_act_fp8(x_bf16, xq, xs, stream=None):
    T, H = x_bf16.shape
    _check(lib().moe_quantize_act_fp8(_p(x_bf16), T, H, _p(xq), _p(xs),
                                      _stream(stream)), "moe_quantize_act_fp8")


def moe_quantize_act_mxfp8(x_bf16, xq, xe, stream=None):
    T, H = x_bf16.shape
    _check(lib().moe_quantize_act_mxfp8(_p(x_bf16), T, H, _p(xq), _p(xe),
                                        _stream(stream)), "moe_quantize_act_mxfp8")


def moe_gemm1_workspace_size(w13: MoeWeights, p_cap, lora: Optional[MoeLora] = None) -> int:
    return lib().moe_gemm1_workspace_size(
        ctypes.byref(w13), p_cap, ctypes.pointer(lora) if lora is not None else None)


def _lp(lora):
    return ctypes.pointer(lora) if lora is not None else None


def moe_grouped_gemm1_act(w13: MoeWeights, x, xs, x_bf16, T, H, I, top_k, p_cap,
                          offsets, sorted_pair, act: MoeActParams,
                          lora: Optional[MoeLora], h, hs, ws, stream=None,
                          h_lora=None, err_word=None):
    _check(lib().moe_grouped_gemm1_act(
        ctypes.byref(w13), _p(x), _p(xs), _p(x_bf16), T, H, I, top_k, p_cap,
        _p(offsets), _p(sorted_pair), ctypes.byref(act), _lp(lora), _p(h), _p(hs),
        _p(h_lora), _p(err_word), _p(ws),
        0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)), "moe_grouped_gemm1_act")


def moe_gemm2_workspace_size(w2: MoeWeights, p_cap,
                             lora_down: Optional[MoeLora] = None) -> int:
    return lib().moe_gemm2_workspace_size(ctypes.byref(w2), p_cap, _lp(lora_down))


def moe_grouped_gemm2_combine(w2: MoeWeights, h, hs, T, H, I, top_k,
                              shared_expert, p_cap, offsets, pair_row, topk_w,
                              shared_w, out, ws, stream=None, h_lora=None,
                              lora_down: Optional[MoeLora] = None, sorted_pair=None,
                              err_word=None):
    _check(lib().moe_grouped_gemm2_combine(
        ctypes.byref(w2), _p(h), _p(hs), _p(h_lora), _lp(lora_down), T, H, I,
        top_k, shared_expert, p_cap, _p(offsets), _p(sorted_pair), _p(pair_row),
        _p(topk_w), shared_w, _p(out), _p(err_word), _p(ws),
        ws.numel() * ws.element_size(), _stream(stream)), "moe_grouped_gemm2_combine")


def moe_workspace_size(layer: MoeLayer, T_max) -> int:
    n = lib().moe_workspace_size(ctypes.byref(layer), T_max)
    if n == 0:
        raise MoeError(-2, "moe_workspace_size", "invalid layer descriptor")
    return n


def moe_forward(layer: MoeLayer, x_bf16, logits, out, topk_ids, topk_w, sink_w,
                err_word, ws, stream=None):
    T = x_bf16.shape[0]
    _check(lib().moe_forward(ctypes.byref(layer), _p(x_bf16), _p(logits), T,
                             logits.stride(0), _p(out), _p(topk_ids), _p(topk_w),
                             _p(sink_w), _p(err_word), _p(ws),
                             ws.numel() * ws.element_size(), _stream(stream)),
           "moe_forward")


def moe_forward_no_workspace(layer: MoeLayer, x_bf16, logits, out, topk_ids, topk_w,
                             sink_w, err_word, stream=None):
    """moe_forward with the library's static device scratch as workspace."""
    T = x_bf16.shape[0]
    L = lib()
    st = L.moe_forward_no_workspace(ctypes.byref(layer), _p(x_bf16), _p(logits), T,
                                    logits.stride(0), _p(out), _p(topk_ids), _p(topk_w),
                                    _p(sink_w), _p(err_word), _stream(stream))
    if st == -9:
        raise MoeError(st, "moe_forward_no_workspace", L.moe_scratch_error().decode())
    _check(st, "moe_forward_no_workspace")


def moe_read_device_error(err_word, stream=None) -> int:
    bits = c_int(0)
    _check(lib().moe_read_device_error(_p(err_word), ctypes.byref(bits),
                                       _stream(stream)), "moe_read_device_error")
    return bits.value


# ------------------------------------------------------------ layer object

class MoeModule:
    """Device tensors of one layer plus its descriptor; forward() allocates
    the outputs and a workspace with torch and calls moe_forward."""

    def __init__(self, *, fmt, H, I, num_experts_global, top_k, w13_q, w2_q,
                 w13_s=None, w2_s=None, gscale=None, gscale2=None,
                 num_local_experts=None,
                 local_expert_offset=0, shared_expert=0, n_sink=0,
                 route_scale=1.0, global_scale=1.0, shared_w=1.0, alpha=1.0,
                 beta=0.0, limit=math.inf, lora_A=None, lora_B=None,
                 lora_scale=1.0, lora_A2=None, lora_B2=None):
        self.fmt, self.H, self.I, self.top_k, self.n_sink = fmt, H, I, top_k, n_sink
        self.shared_expert = shared_expert
        E_loc = num_experts_global if num_local_experts is None else num_local_experts
        self.w13 = weights(fmt, w13_q, w13_s, gscale)
        self.w2 = weights(fmt, w2_q, w2_s, gscale2)
        self.act = act_params(alpha, beta, limit)
        self.lora = lora_desc(lora_A, lora_B, lora_scale) if lora_A is not None else None
        self.lora_down = (lora_desc(lora_A2, lora_B2, lora_scale)
                          if lora_A2 is not None else None)
        self.desc = layer_desc(H, I, num_experts_global, E_loc, local_expert_offset,
                               shared_expert, top_k, n_sink, route_scale,
                               global_scale, shared_w, self.w13, self.w2, self.act,
                               self.lora, self.lora_down)
        self._ws = None

    def workspace(self, T):
        need = moe_workspace_size(self.desc, T)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        return self._ws

    def alloc_outputs(self, T):
        dev = "cuda"
        return dict(
            out=torch.empty(T, self.H, dtype=torch.float32, device=dev),
            topk_ids=torch.empty(T, self.top_k, dtype=torch.int32, device=dev),
            topk_w=torch.empty(T, self.top_k, dtype=torch.float32, device=dev),
            sink_w=(torch.empty(T, self.n_sink, dtype=torch.float32, device=dev)
                    if self.n_sink else None),
            err_word=torch.zeros(1, dtype=torch.int32, device=dev))

    def set_adapters(self, adapter_ids: Optional[torch.Tensor]):
        """Per-token adapter ids (int32 [T], -1 none) for a batch of adapters."""
        for d in (self.lora, self.lora_down):
            if d is not None and d.n_adapters > 1:
                d.adapter_ids = None if adapter_ids is None else adapter_ids.data_ptr()
                d._keep = d._keep[:2] + (adapter_ids,)

    def forward(self, x_bf16, logits, outs=None, stream=None, adapter_ids=None):
        T = x_bf16.shape[0]
        if adapter_ids is not None:
            self.set_adapters(adapter_ids)
        o = outs if outs is not None else self.alloc_outputs(T)
        moe_forward(self.desc, x_bf16, logits, o["out"], o["topk_ids"], o["topk_w"],
                    o["sink_w"], o["err_word"], self.workspace(T), stream)
        return o
