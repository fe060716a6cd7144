"""The C-ABI library loads, exports every symbol the header declares, and its
host-side validation rejects bad arguments before touching the device
(no GPU needed: every call here returns before any HIP call)."""
import ctypes
import math
import os
import re

import pytest

import mixture_experts_expert_sigmoid_amd as M

pytestmark = pytest.mark.skipif(not os.path.exists(M.LIB_PATH),
                                reason="library not built")


def _declared():
    src = open(M.HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert "moe_forward" in names and "moe_route" in names
    L = ctypes.CDLL(M.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    # the four steps of the path and the one-shot layer call are all declared
    for n in ("moe_route", "moe_permute", "moe_grouped_gemm1_act",
              "moe_grouped_gemm2_combine", "moe_forward"):
        assert n in names


def test_binding_covers_every_declared_symbol():
    for n in _declared():
        assert n in M._SIGS, n


def _w(fmt=M.MOE_W_FP8_B128, G=4, N=256, K=256, q=1, s=1):
    return M.MoeWeights(fmt, G, N, K, q, s, None)


def test_route_validation():
    L = M.lib()
    # (logits, T, ld, n_routed, n_sink, top_k, sel_bias, scales, ids, w, sw, packed)
    f = lambda lg, T, ld, N, S, k, rs=1.0, sw=None: L.moe_route(
        lg, T, ld, N, S, k, None, rs, 1.0, 1, 1, sw, None, None)
    # top_k > n_routed, top_k + n_sink > 64, ld too small, T < 0
    assert f(1, 4, 8, 8, 0, 9) == -2
    assert f(1, 4, 100, 60, 8, 60, sw=1) == -2
    assert f(1, 4, 7, 8, 0, 2) == -2
    assert f(1, -1, 8, 8, 0, 2) == -2
    assert f(1, 4, 8, 8, 0, 2, rs=math.nan) == -5
    assert f(None, 4, 8, 8, 0, 2) == -1
    assert f(1, 4, 10, 8, 2, 2) == -1   # sinks need sink_w


def test_gate_route_validation():
    L = M.lib()
    ws = ctypes.c_void_p(256)

    def f(x=256, wg=256, T=4, H=2048, N=256, S=2, k=8, rs=1.0, sw=1, ws_=ws,
          nb=1 << 30):
        return L.moe_gate_route(x, wg, T, H, N, S, k, None, rs, 1.0, None, 1, 1,
                                sw, None, ws_, nb, None)
    assert f(H=2040) == -2                  # H % 32
    assert f(H=0) == -2
    assert f(k=9, S=8) == -2                # top_k + n_sink > 16
    assert f(N=500, S=13) == -2             # more than 512 columns
    assert f(k=300) == -2                   # top_k > n_routed
    assert f(T=-1) == -2
    assert f(rs=math.inf) == -5
    assert f(x=None) == -1
    assert f(sw=None) == -1                 # sinks need sink_w
    assert f(x=264) == -5                   # not 16-byte aligned
    assert f(ws_=None) == -6                # split path needs the workspace
    assert f(nb=16) == -6
    # T = 0 is a no-op; large T needs no workspace (one fused launch)
    assert f(T=0, x=None, wg=None, ws_=None, nb=0) == 0
    assert L.moe_gate_route_workspace_size(1, 2048, 256, 2) >= 272 * 4
    assert L.moe_gate_route_workspace_size(8192, 2048, 256, 2) == 0
    assert L.moe_gate_route_workspace_size(4, 2040, 256, 2) == 0   # invalid H


def test_permute_validation_local_range():
    L = M.lib()
    ws = ctypes.c_void_p(1)
    # missing / invalid local range is an error, not a silent out-of-bounds read
    assert L.moe_permute(1, 4, 8, 256, 96, 0, 0, 1, 1, 1, 1, ws, 1 << 20, None) == -4
    assert L.moe_permute(1, 4, 8, 256, -1, 32, 0, 1, 1, 1, 1, ws, 1 << 20, None) == -4
    assert L.moe_permute(1, 4, 8, 256, 240, 32, 0, 1, 1, 1, 1, ws, 1 << 20, None) == -4
    assert L.moe_permute(1, 4, 8, 256, 96, 32, 0, 1, 1, 1, 1, None, 0, None) == -6
    assert L.moe_permute(1, 4, 8, 256, 96, 32, 0, 1, 1, 1, 1, ws, 16, None) == -6
    assert L.moe_permute(1, 4, 8, 2048, 0, 1100, 0, 1, 1, 1, 1, ws, 1 << 20, None) == -2
    assert L.moe_permute_workspace_size(4096, 8, 289) > 4096 * 8 * 4


def test_quantize_validation():
    L = M.lib()
    for f in (L.moe_quantize_act_fp8, L.moe_quantize_act_mxfp8):
        assert f(1, 4, 100, 1, 1, None) == -2      # H % 128
        assert f(1, -1, 128, 1, 1, None) == -2
        assert f(None, 4, 128, 1, 1, None) == -1
        assert f(1, 4, 128, 1, None, None) == -1
        assert f(None, 0, 128, None, None, None) == 0   # T = 0: nothing to do


def test_gemm_validation():
    L = M.lib()
    act = M.act_params(1.0, 0.0, math.inf)
    w = _w(N=2 * 128, K=256)
    g1 = lambda w_, act_, H=256, I=128, lora=None, hl=None, err=1: L.moe_grouped_gemm1_act(
        ctypes.byref(w_), 1, 1, None, 4, H, I, 2, 8, 1, 1, ctypes.byref(act_),
        lora, 1, 1, hl, err, ctypes.c_void_p(1), 1 << 20, None)
    assert g1(_w(N=256, K=250), act, H=250) == -2        # H % 128
    assert g1(_w(N=256, K=256), act, H=256, I=100) == -2   # I % 128
    assert g1(_w(N=512, K=256), act) == -2               # N != 2I
    assert g1(M.MoeWeights(7, 4, 256, 256, 1, 1, None), act) == -3
    assert g1(M.MoeWeights(6, 4, 256, 256, 1, 1, None), act) == -3
    assert g1(M.MoeWeights(-1, 4, 256, 256, 1, 1, None), act) == -3
    # 4-bit codes are read 16 bytes at a time, NVFP4 scales as 2-byte pairs
    for f in (M.MOE_W_INT4_G32, M.MOE_W_NVFP4, M.MOE_W_MXFP4, M.MOE_W_MXFP4_A8):
        assert g1(M.MoeWeights(f, 4, 256, 256, 264, 256, None), act) == -5
    assert g1(M.MoeWeights(M.MOE_W_NVFP4, 4, 256, 256, 256, 257, None), act) == -5
    assert g1(M.MoeWeights(M.MOE_W_NVFP4, 4, 256, 256, 256, None, None), act) == -1
    assert g1(M.MoeWeights(1, 4, 256, 256, 1, None, None), act) == -1   # fp8 needs scales
    # 4-bit layers report range problems through the error word: required
    for f in (M.MOE_W_INT4_G32, M.MOE_W_NVFP4, M.MOE_W_MXFP4, M.MOE_W_MXFP4_A8):
        assert g1(M.MoeWeights(f, 4, 256, 256, 256, 256, None), act, err=None) == -1
    # MXFP4 W4A8: GEMM1 takes the MXFP8 codes' e8m0 exponents in xs
    mxw = M.MoeWeights(M.MOE_W_MXFP4_A8, 4, 256, 256, 256, 256, None)
    assert L.moe_grouped_gemm1_act(ctypes.byref(mxw), 1, None, None, 4, 256, 128, 2, 8, 1, 1,
                                   ctypes.byref(act), None, 1, None, None, 1,
                                   ctypes.c_void_p(1), 1 << 20, None) == -1
    # and needs no f16 copy of the activations in its workspace
    big13 = M.MoeWeights(M.MOE_W_MXFP4_A8, 64, 1536, 2048, 256, 256, None)
    big13i = M.MoeWeights(M.MOE_W_MXFP4, 64, 1536, 2048, 256, 256, None)
    assert L.moe_gemm1_workspace_size(ctypes.byref(big13), 16384, None) == 0
    assert L.moe_gemm1_workspace_size(ctypes.byref(big13i), 16384, None) >= 16384 * 2048 * 2
    assert g1(w, M.act_params(1.0, 0.0, 0.0)) == -5       # limit must be > 0
    assert g1(w, M.act_params(1.0, 0.0, math.nan)) == -5
    assert g1(w, M.act_params(math.inf, 0.0, 7.0)) == -5
    assert g1(w, M.act_params(1.0, math.nan, 7.0)) == -5
    lo = M.MoeLora(64, 4, 1.0, 256, 256, 1, None)
    assert g1(w, act, lora=ctypes.pointer(lo)) == -2      # rank > 32
    # the bf16 down-LoRA input is an FP8-only output of GEMM1
    assert g1(_w(fmt=M.MOE_W_BF16, N=256, K=256), act, hl=ctypes.c_void_p(256)) == -5
    w2 = _w(N=256, K=128)
    g2 = lambda hl=None, ld=None, ws=None, nb=0, sp=1, k=2, w_=w2, err=1: \
        L.moe_grouped_gemm2_combine(ctypes.byref(w_), 1, 1, hl, ld, 4, 256, 128, k, 0,
                                    4 * k, 1, sp, 1, 1, 1.0, 1, err, ws, nb, None)
    assert g2() == -6                                    # workspace
    # top_k <= 64: the split-K combine holds a token's pairs in LDS
    assert g2(k=65) == -2 and g2(k=64) == -6 and g2(k=0) == -2
    w2i = M.MoeWeights(M.MOE_W_INT4_G32, 4, 256, 128, 256, 256, None)
    assert g2(w_=w2i, err=None) == -1                     # 4-bit: error word required
    ld = M.MoeLora(16, 4, 1.0, 256, 256, 1, None)
    big = dict(ws=ctypes.c_void_p(256), nb=1 << 30)
    assert g2(ld=ctypes.pointer(ld), **big) == -1         # no h_lora
    assert g2(ld=ctypes.pointer(ld), hl=ctypes.c_void_p(256), sp=None, **big) == -1
    assert g2(ld=ctypes.pointer(M.MoeLora(40, 4, 1.0, 256, 256, 1, None)),
              hl=ctypes.c_void_p(256), **big) == -2       # rank > 32
    # a batch of adapters needs the per-token ids
    assert g2(ld=ctypes.pointer(M.MoeLora(16, 4, 1.0, 256, 256, 8, None)),
              hl=ctypes.c_void_p(256), **big) == -1
    assert g2(ld=ctypes.pointer(M.MoeLora(16, 4, 1.0, 256, 264, 1, None)),
              hl=ctypes.c_void_p(256), **big) == -5     # B not 16-byte aligned
    # W2 global scales are an FP4-format input
    w2g = M.MoeWeights(M.MOE_W_FP8_B128, 4, 256, 128, 1, 1, 256)
    assert L.moe_grouped_gemm2_combine(ctypes.byref(w2g), 1, 1, None, None, 4, 256, 128, 2,
                                       0, 8, 1, 1, 1, 1, 1.0, 1, None, ctypes.c_void_p(256),
                                       1 << 30, None) == -3
    assert L.moe_gemm2_workspace_size(ctypes.byref(w2), 100, None) >= 100 * 256 * 4
    assert (L.moe_gemm2_workspace_size(ctypes.byref(w2), 100, ctypes.pointer(ld)) -
            L.moe_gemm2_workspace_size(ctypes.byref(w2), 100, None)) >= 100 * 16 * 4
    assert L.moe_gemm2_workspace_size(None, 100, None) == 0
    # FP8 at decode sizes (few tiles for the CUs): room for the split-K
    # partial sums; at large p_cap plain rows only
    w13f = _w(fmt=M.MOE_W_FP8_B128, G=289, N=4096, K=6144)      # 9 x 16 tiles
    assert L.moe_gemm1_workspace_size(ctypes.byref(w13f), 9, None) >= 4 * 9 * 4096 * 4
    assert L.moe_gemm1_workspace_size(ctypes.byref(w13f), 36864, None) == 0
    w2f = _w(fmt=M.MOE_W_FP8_B128, G=128, N=3072, K=1536)       # 4 x 12 tiles
    assert L.moe_gemm2_workspace_size(ctypes.byref(w2f), 4, None) >= 4 * 4 * 3072 * 4
    assert L.moe_gemm2_workspace_size(ctypes.byref(w2f), 16384, None) == 16384 * 3072 * 4
    w13b = _w(fmt=M.MOE_W_BF16, G=289, N=4096, K=6144)
    assert L.moe_gemm1_workspace_size(ctypes.byref(w13b), 9, None) == 0   # BF16: none
    assert L.moe_gemm1_workspace_size(None, 9, None) == 0


def _layer(**kw):
    w13 = _w(N=256, K=256, G=kw.pop("G", 4))
    w2 = _w(N=256, K=128, G=w13.n_groups)
    d = dict(H=256, I=128, E=8, E_loc=4, off=4, shared=0, k=2, S=0)
    d.update(kw)
    return M.layer_desc(d["H"], d["I"], d["E"], d["E_loc"], d["off"], d["shared"],
                        d["k"], d["S"], 1.0, 1.0, 1.0, w13, w2, M.act_params())


def test_forward_validation_and_workspace():
    L = M.lib()
    good = _layer()
    assert L.moe_workspace_size(ctypes.byref(good), 64) > 0
    bad_range = _layer(off=6)                 # 6 + 4 > 8
    assert L.moe_workspace_size(ctypes.byref(bad_range), 64) == 0
    r = L.moe_forward(ctypes.byref(bad_range), 1, 1, 4, 8, 1, 1, 1, None, 1,
                      ctypes.c_void_p(1), 1 << 30, None)
    assert r == -4
    r = L.moe_forward(ctypes.byref(good), 1, 1, 4, 8, 1, 1, 1, None, 1,
                      ctypes.c_void_p(1), 16, None)
    assert r == -6
    r = L.moe_forward(ctypes.byref(good), 1, 1, 4, 8, 1, 1, 1, None, None,
                      ctypes.c_void_p(1), 1 << 30, None)
    assert r == -1                            # err_word is required
    groups_mismatch = _layer(G=5)
    assert L.moe_workspace_size(ctypes.byref(groups_mismatch), 64) == 0
    assert L.moe_status_string(-4) == b"missing or invalid local expert range"
