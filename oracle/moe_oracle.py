"""fp64 CPU oracle of the routed MoE expert-FFN path.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module. The product path (the HIP library and
its Python binding) never imports, calls or links it, and shares no code with
it: number formats, routing, permutation, quantisation, dequantisation,
epilogue and combine are written out here a second time, plainly, in float64.

What each step computes, and the passage it follows (the pages are cited by
title and section):

  route      -- sigmoid-gate top-k with log-sigmoid renormalisation and
                shared-sink columns: "Enable and fuse the Inkling MoE gate
                epilogue on Intel XPU" (sglang PR #36385), "2. Correctness"
                (w = exp(lp - logsumexp(lp)), lp = logsigmoid(x)) and
                "3. Performance" plus the epilogue commit message (iterative
                masked-max top-k, raw logit carried, trailing SHARED_SINK
                columns join the normaliser, global_scale).
  gate       -- the router GEMM in front of that epilogue (the "258-column
                gate GEMM" of the same PR, its fp32 [T, 258] gate row), an
                optional selection bias [N] that shifts the ranking key to
                sigmoid(x) + bias while the winner still carries its raw
                logit, and the packed (id << 16 | bf16 weight) output: the
                same PR, router-epilogue commit message.
  permute    -- expert-parallel rebase: routing ids are global, per-expert
                tables are rank-local, rebase by local_expert_offset and
                bounds-check: "FlashInfer 0.6.18 SM100a+SM103a MoE-LoRA AOT"
                release notes, "Changes since 1b699bf"; tokens grouped per
                expert ("per-expert sorted-token dispatch"): "Fused INT4
                grouped + SiLU Triton kernel" (batchgen PR #239), commit text.
  quant_act  -- per-token, per-128-column fp8 e4m3 activation quantisation
                that goes with blockwise 128x128 FP8 weights ("DeepSeekFp8"):
                sglang PR #39920, "Modifications"; rounding read as
                round-to-nearest-even with saturation at +-448.
  dequant    -- FP8 q * block scale; INT4 (nibble - 8) * scale[n, k/32],
                low nibble = even k: batchgen PR #239, commit text. NVFP4
                expert weights with distinct per-half global scales (the
                format the MoE-LoRA AOT release notes serve, "Changes since
                1b699bf"): e2m1 codes times an e4m3 scale per 16 K times
                the fp32 global scale (W13: gate, up; W2: one per expert);
                MXFP4: e2m1 codes times a power-of-two e8m0 scale per 32 K.
  quant_mx   -- the W4A8 variant of the MXFP4 layers: activations enter
                GEMM1 as MXFP8 (e4m3 codes with a power-of-two e8m0 scale
                per 32 columns, the smallest that keeps the group's amax
                within 448), the form the block-scaled matrix instructions
                take; a design choice of this library (the pages fix no
                activation format for 4-bit weights), h stays bf16.
                The pages name these formats without defining them; the
                element and scale encodings are the public ones, written
                here from their bit fields.
  swiglu     -- g' = min(g, L), u' = clamp(u, -L, L),
                h = g' * sigmoid(alpha g') * (u' + beta); defaults alpha = 1,
                beta = 0, no clamp: sglang PR #39920 "Modifications" and
                "fix(sm90): support parameterized SwiGLU in FP8 MegaMoE"
                (DeepGEMM PR #445), "Summary" and "Compatibility".
  lora       -- delta added to gate and up in true units, i.e. after each
                half's own global scale: MoE-LoRA AOT release notes,
                "Changes since 1b699bf"; the down-projection LoRA consumes
                activation_lora_input, the SwiGLU output in those true
                units (same section: the pre-fix kernels left it off by
                gate/up), its delta added to the expert's output.
  combine    -- out[t] = sum over t's local slots of w[t, j] * y[t, j], fp32
                accumulation on the device ("slot-specific routing-weight
                reduction"): batchgen PR #239, commit text.

Readings taken where the pages leave a step open are listed in the design
notes; the code states each one where it is used.

Parity of the whole layer against a printed page output is unpinned (the pages
print no layer outputs); each step is pinned separately by the tests.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

E4M3_MAX = 448.0


# ----------------------------------------------------------------------------
# number formats (OCP e4m3fn, bfloat16), written from their definitions
# ----------------------------------------------------------------------------

def _e4m3_from_fields(codes) -> np.ndarray:
    """OCP e4m3fn code -> value: sign * 2^(e-7) * (1 + m/8) for e >= 1,
    sign * 2^-6 * m/8 for e == 0; 0x7F / 0xFF are NaN (no infinities)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m / 8.0, -6),
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32)))
    val = np.where((e == 15) & ((c & 7) == 7), np.nan, val)
    return sign * val


# the formula above evaluated once per code; decoding is a lookup in it
_E4M3_VALUES = _e4m3_from_fields(np.arange(256))


def e4m3_decode(codes) -> np.ndarray:
    """OCP e4m3fn code -> value (float64), looked up in the 256 values of the
    bit-field formula."""
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_round(v) -> np.ndarray:
    """Nearest e4m3fn code to the exact value v (float64), ties to the even
    code, magnitudes >= 448 saturated to +-448. Returns uint8 codes."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    # subnormal range: multiples of 2^-9 below 2^-6 (m = 8 is the first normal)
    sub = a < 2.0 ** -6
    code_sub = np.rint(np.where(sub, a, 0.0) * 512.0).astype(np.int64)
    # normal range: 4 significant bits
    an = np.where(sub | ~np.isfinite(a), 1.0, a)
    _, ex = np.frexp(an)
    e = (ex - 1).astype(np.int64)                # an = 1.f * 2^e
    mant = np.rint(np.ldexp(an, (3 - e).astype(np.int32))).astype(np.int64)
    e = np.where(mant >= 16, e + 1, e)           # rounding carried into e
    mant = np.where(mant >= 16, 8, mant)
    code_norm = ((e + 7) << 3) | (mant - 8)
    code = np.where(sub, code_sub, code_norm)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.where(np.isnan(v), 0x7F, code | sign)
    return code.astype(np.uint8)


def bf16_decode(bits) -> np.ndarray:
    """bfloat16 bits (uint16) -> float64: the top half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round(v) -> np.ndarray:
    """Nearest bfloat16 value (8 significant bits, ties to even) of float64 v,
    returned as float64. Normal range only (|v| >= 2^-126), which covers every
    value rounded here; smaller magnitudes round on the 2^-133 grid."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(np.where(a == 0, 1.0, a))
    e = np.maximum(ex - 1, -126)
    q = np.ldexp(np.rint(np.ldexp(a, (7 - e).astype(np.int32))),
                 (e - 7).astype(np.int32))
    return np.where(np.signbit(v), -q, q)


# ----------------------------------------------------------------------------
# router epilogue (sglang PR #36385)
# ----------------------------------------------------------------------------

def logsigmoid(x) -> np.ndarray:
    """log(sigmoid(x)) = min(x, 0) - log1p(exp(-|x|)), the overflow-free form."""
    x = np.asarray(x, dtype=np.float64)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def topk_masked_max(keys, k):
    """k passes of argmax over the keys not yet taken; equal keys resolve to
    the lower column index. Slot j holds the j-th pick."""
    keys = np.asarray(keys, dtype=np.float64)
    T, N = keys.shape
    ids = np.zeros((T, k), dtype=np.int64)
    remaining = np.ones((T, N), dtype=bool)
    for j in range(k):
        masked = np.where(remaining, keys, np.nan)
        pick = np.nanargmax(masked, axis=1)       # first index of the max
        ids[:, j] = pick
        remaining[np.arange(T), pick] = False
    return ids


def selection_keys(logits_routed, sel_bias):
    """Ranking key under a selection bias, in the page's precision (fp32):
    sigmoid of the fp32 logit rounded to fp32, plus the fp32 bias, the sum
    rounded to fp32 (round to nearest even). Bias [N] covers the routed
    columns only; sink columns never enter the ranking."""
    x = np.asarray(logits_routed, dtype=np.float32).astype(np.float64)
    s32 = sigmoid(x).astype(np.float32)
    b32 = np.asarray(sel_bias, dtype=np.float32)
    return (s32 + b32[None, :]).astype(np.float32)


def _carry(raw, keys):
    """The value a winner carries out of the top-k loop: its raw logit, not
    its ranking key."""
    return raw


def route(logits, n_routed, n_sink, top_k, route_scale=1.0, global_scale=1.0,
          sel_bias=None):
    """Top-k over the n_routed columns of each fp32 logit row, then weights
    over the k winners and the n_sink trailing sink columns:
        lp = logsigmoid(x),  w = exp(lp - logsumexp(lp)) * route_scale * global_scale,
    x the winners' RAW logits. Ranking key: with no selection bias the raw
    logit (sigmoid is strictly increasing, so this is the order of
    sigmoid(x)); with a bias [n_routed], selection_keys(). Equal keys go to
    the lower column.
    Returns ids [T, k] (global column ids), w [T, k], sink_w [T, n_sink]."""
    lg = np.asarray(logits, dtype=np.float32)
    T = lg.shape[0]
    raw = lg[:, :n_routed].astype(np.float64)
    keys = raw if sel_bias is None else \
        selection_keys(lg[:, :n_routed], sel_bias).astype(np.float64)
    ids = topk_masked_max(keys, top_k)
    chosen = _carry(np.take_along_axis(raw, ids, axis=1),
                    np.take_along_axis(keys, ids, axis=1))
    sinks = lg[:, n_routed:n_routed + n_sink].astype(np.float64)
    lp = logsigmoid(np.concatenate([chosen, sinks], axis=1))
    if T == 0:
        return ids, np.zeros((0, top_k)), np.zeros((0, n_sink))
    m = lp.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(lp - m).sum(axis=1, keepdims=True))
    scale = float(np.float32(route_scale)) * float(np.float32(global_scale))
    w = np.exp(lp - lse) * scale
    return ids, w[:, :top_k], w[:, top_k:]


def gate_logits(x_bits, wg_bits):
    """Router GEMM: logits[t, c] = sum_h x[t, h] * Wg[c, h] over bf16 x
    [T, H] and bf16 Wg [N + S, H] (bit patterns). Each product of two bf16
    values is exact in float64 and the float64 sum keeps ~1e-16 relative
    error, so this is the exact dot product for all practical purposes."""
    x = bf16_decode(x_bits)
    w = bf16_decode(wg_bits)
    return x @ w.T


def gate_route(x_bits, wg_bits, n_routed, n_sink, top_k, route_scale=1.0,
               global_scale=1.0, sel_bias=None):
    """The gate row is the fp32 [T, N + S] matrix of logits (each the exact
    dot product rounded once to fp32); the epilogue is route() on it.
    Returns (logits fp32, ids, w, sink_w)."""
    lg = gate_logits(x_bits, wg_bits).astype(np.float32)
    ids, w, sw = route(lg, n_routed, n_sink, top_k, route_scale, global_scale,
                       sel_bias)
    return lg, ids, w, sw


def bf16_bits(v) -> np.ndarray:
    """Bit pattern (uint16) of the nearest bfloat16 (ties to even) of v."""
    q = bf16_round(v).astype(np.float32)
    return (q.view(np.uint32) >> 16).astype(np.uint16)


def pack_topk(ids, w) -> np.ndarray:
    """Packed routing output: (id << 16) | bf16 bits of the routed weight,
    one int32 per slot; a consumer recovers the id as p >> 16 and the weight
    from p & 0xFFFF."""
    ids = np.asarray(ids, dtype=np.int64)
    p = (ids << 16) | bf16_bits(w).astype(np.int64)
    return p.astype(np.uint32).view(np.int32)


# ----------------------------------------------------------------------------
# permutation by expert with expert-parallel rebase
# ----------------------------------------------------------------------------

ERR_GLOBAL_ID_OOB = 0x1


def permute(ids, num_experts_global, local_offset, num_local, shared):
    """Group the (token, slot) pairs by local expert.

    Pair id p = t*k + j for routed slots; the always-on shared expert (if any)
    is group num_local with pair ids T*k + t. A global id is rebased to
    e = id - local_offset and kept iff 0 <= e < num_local; ids outside
    [0, num_experts_global) set ERR_GLOBAL_ID_OOB and are skipped.
    Within a group pairs are ordered by p. Returns (offsets [G+1],
    sorted_pair [P], pair_row [T*k (+T)], err)."""
    ids = np.asarray(ids)
    T, k = ids.shape
    G = num_local + (1 if shared else 0)
    groups = [[] for _ in range(G)]
    err = 0
    for t in range(T):
        for j in range(k):
            gid = int(ids[t, j])
            if gid < 0 or gid >= num_experts_global:
                err |= ERR_GLOBAL_ID_OOB
                continue
            e = gid - local_offset
            if 0 <= e < num_local:
                groups[e].append(t * k + j)
    if shared:
        groups[num_local] = [T * k + t for t in range(T)]
    offsets = [0]
    sorted_pair = []
    for g in range(G):
        sorted_pair.extend(groups[g])
        offsets.append(len(sorted_pair))
    n_pairs = T * k + (T if shared else 0)
    pair_row = -np.ones(n_pairs, dtype=np.int64)
    pair_row[np.asarray(sorted_pair, dtype=np.int64)] = np.arange(len(sorted_pair))
    return (np.asarray(offsets, dtype=np.int64),
            np.asarray(sorted_pair, dtype=np.int64), pair_row, err)


# ----------------------------------------------------------------------------
# fp8 activation quantisation (per token, per 128 columns)
# ----------------------------------------------------------------------------

def quant_act_fp8(x_f32, group=128):
    """amax over each 128-column group in fp32, s = fp32(amax / 448) (s = 1
    when amax = 0), q = e4m3 RNE of the fp32 quotient fp32(x / s), saturated.
    Returns (codes uint8 [T, H], s float32 [T, H/128])."""
    x = np.asarray(x_f32, dtype=np.float32)
    T, H = x.shape
    xg = x.reshape(T, H // group, group)
    amax = np.abs(xg).max(axis=2) if T else np.zeros((0, H // group), np.float32)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX),
                 np.float32(1.0)).astype(np.float32)
    quot = (xg / s[:, :, None]).astype(np.float32)          # fp32 division
    q = e4m3_round(quot.astype(np.float64)).reshape(T, H)
    return q, s


def quant_act_mxfp8(x_f32, group=32):
    """MXFP8 activations (the GEMM1 input of the MXFP4 W4A8 layers): per row
    and 32 columns, amax = max |x| (fp32), e = the smallest integer with
    amax <= 448 * 2^e, held as the e8m0 code e + 127 (e is raised to -127
    when smaller, e.g. for an all-zero group), and codes = e4m3 RNE of the
    exact quotient x / 2^e (never above 448, so never saturated). Returns
    (codes uint8 [T, H], e8m0 codes uint8 [T, H/32])."""
    x = np.asarray(x_f32, dtype=np.float32).astype(np.float64)
    T, H = x.shape
    xg = x.reshape(T, H // group, group)
    amax = np.abs(xg).max(axis=2) if T else np.zeros((0, H // group))
    # candidate from the logarithm, then corrected against the exact bound
    e = np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / E4M3_MAX)).astype(np.int64)
    for _ in range(2):
        e = np.where(amax > E4M3_MAX * np.ldexp(1.0, e.astype(np.int32)), e + 1, e)
        e = np.where(amax <= E4M3_MAX * np.ldexp(1.0, (e - 1).astype(np.int32)), e - 1, e)
    e = np.where(amax > 0, np.maximum(e, -127), -127)
    q = e4m3_round(xg / np.ldexp(1.0, e.astype(np.int32))[:, :, None]).reshape(T, H)
    return q, (e + 127).astype(np.uint8)


def requant_fp8(h, group=128):
    """The FP8 path's intermediate rounding of h [P, I] (float64): per row and
    128-column group, amax taken to fp32, s = fp32(amax / 448) (1 if zero),
    q = e4m3 RNE of h / s, saturated. Returns the value q * s (float64)."""
    h = np.asarray(h, dtype=np.float64)
    P, I = h.shape
    hg = h.reshape(P, I // group, group)
    amax = np.abs(hg).max(axis=2).astype(np.float32) if P else \
        np.zeros((0, I // group), np.float32)
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX),
                 np.float32(1.0)).astype(np.float32).astype(np.float64)
    q = e4m3_round(hg / s[:, :, None])
    return (e4m3_decode(q) * s[:, :, None]).reshape(P, I)


# ----------------------------------------------------------------------------
# weight dequantisation, one expert at a time, exact in float64
# ----------------------------------------------------------------------------

def dequant_fp8_block(q, bs):
    """w[n, k] = e4m3(q[n, k]) * bs[n // 128, k // 128]."""
    w = e4m3_decode(q)
    N, K = w.shape
    b = np.asarray(bs, np.float64)
    return (w.reshape(N // 128, 128, K // 128, 128) * b[:, None, :, None]).reshape(N, K)


def dequant_int4_g32(packed, scale_bits):
    """Byte j of row n holds k = 2j in its low nibble and k = 2j + 1 in its
    high nibble; w[n, k] = (nibble - 8) * scale[n, k // 32] (bf16 scale)."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    N, Kh = b.shape
    nib = np.empty((N, 2 * Kh), dtype=np.float64)
    nib[:, 0::2] = (b & 0xF) - 8
    nib[:, 1::2] = (b >> 4) - 8
    return nib * np.repeat(bf16_decode(scale_bits), 32, axis=1)


def e2m1_decode(codes) -> np.ndarray:
    """4-bit e2m1 element code -> value: bit 3 sign, bits 2..1 exponent e
    (bias 1), bit 0 mantissa m; sign * 2^(e-1) * (1 + m/2) for e >= 1 and
    sign * m/2 for e == 0 (no infinities or NaN). The eight magnitudes are
    0, 0.5, 1, 1.5, 2, 3, 4, 6."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    val = np.where(e == 0, m / 2.0,
                   np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int32)))
    return sign * val


def _nibbles(packed):
    """[N][K/2] bytes -> [N][K] 4-bit codes; byte j holds k = 2j in its low
    nibble and k = 2j + 1 in its high nibble."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    N, Kh = b.shape
    nib = np.empty((N, 2 * Kh), dtype=np.int64)
    nib[:, 0::2] = b & 0xF
    nib[:, 1::2] = b >> 4
    return nib


def dequant_nvfp4(packed, scale_codes):
    """NVFP4: w[n, k] = e2m1(code[n, k]) * e4m3(scale[n, k // 16]); the
    per-tensor fp32 global scale (here per expert, per half of W13) is
    applied by the caller."""
    return e2m1_decode(_nibbles(packed)) * np.repeat(e4m3_decode(scale_codes), 16, axis=1)


def e8m0_decode(codes) -> np.ndarray:
    """e8m0 scale code -> 2^(e - 127); 0xFF is NaN."""
    e = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(e == 0xFF, np.nan, np.ldexp(1.0, (e - 127).astype(np.int32)))


def dequant_mxfp4(packed, scale_codes):
    """MXFP4: w[n, k] = e2m1(code[n, k]) * 2^(scale[n, k // 32] - 127)."""
    return e2m1_decode(_nibbles(packed)) * np.repeat(e8m0_decode(scale_codes), 32, axis=1)


def dequant(fmt, q, s):
    if fmt == "bf16":
        return bf16_decode(q)
    if fmt == "fp8":
        return dequant_fp8_block(q, s)
    if fmt == "int4":
        return dequant_int4_g32(q, s)
    if fmt == "nvfp4":
        return dequant_nvfp4(q, s)
    if fmt in ("mxfp4", "mxfp4_a8"):
        return dequant_mxfp4(q, s)
    raise ValueError(fmt)


# ----------------------------------------------------------------------------
# parameterized SwiGLU epilogue
# ----------------------------------------------------------------------------

def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    ez = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + ez), ez / (1.0 + ez))


def swiglu(g, u, alpha=1.0, beta=0.0, limit=math.inf):
    """Clamp first (gate from above only, up on both sides), alpha scales the
    clamped gate inside the sigmoid, beta is added to the clamped up."""
    gp = np.minimum(g, limit)
    up = np.clip(u, -limit, limit)
    return gp * sigmoid(alpha * gp) * (up + beta)


# ----------------------------------------------------------------------------
# one expert over its pairs, and the whole layer
# ----------------------------------------------------------------------------

def w13_dequant(spec, arr, e):
    """Dequantised fused [gate | up] weight of group e: rows 0..I-1 gate,
    I..2I-1 up, each half times its own global scale when present."""
    w = dequant(spec.fmt, arr["w13_q"][e],
                None if arr["w13_s"] is None else arr["w13_s"][e])
    if arr.get("gs") is not None:
        I = spec.I
        gs = np.asarray(arr["gs"][e], dtype=np.float32).astype(np.float64)
        w[:I] *= gs[0]
        w[I:] *= gs[1]
    return w


def w2_dequant(spec, arr, e):
    """Dequantised down weight of group e, times its global scale when
    present (FP4 layers: one fp32 per expert)."""
    w = dequant(spec.fmt, arr["w2_q"][e],
                None if arr["w2_s"] is None else arr["w2_s"][e])
    if arr.get("gs2") is not None:
        w *= float(np.float32(arr["gs2"][e]))
    return w


def lora_mat(spec, arr, name, a, e):
    """Adapter a's matrix of group e: arrays are [G, ...] for one adapter and
    [n_adapters, G, ...] for a batch of adapters."""
    return arr[name][e] if spec.n_adapters == 1 else arr[name][a][e]


def _per_adapter(spec, rows, adapters, fn):
    """fn(a, row_selection) for every adapter a >= 0 that some row uses;
    rows whose adapter is -1 (or out of range) get no delta (zero rows)."""
    m = rows.shape[0]
    ad = np.zeros(m, np.int64) if adapters is None else np.asarray(adapters, np.int64)
    out = None
    for a in np.unique(ad):
        if a < 0 or a >= spec.n_adapters:
            continue
        sel = ad == a
        d = fn(int(a), sel)
        if out is None:
            out = np.zeros((m, d.shape[1]))
        out[sel] = d
    return out


def lora_delta(spec, arr, e, x_bf16_rows, adapters=None):
    """Rank-r delta on [gate | up] in true units: z = x A_e^T (kept in full
    precision), delta = lora_scale * z B_e^T, shape [m, 2I]; with a batch of
    adapters each row uses its token's adapter (none: zero)."""
    def one(a, sel):
        A = bf16_decode(lora_mat(spec, arr, "lora_A", a, e))    # [r, H]
        B = bf16_decode(lora_mat(spec, arr, "lora_B", a, e))    # [2I, r]
        return float(np.float32(spec.lora_scale)) * ((x_bf16_rows[sel] @ A.T) @ B.T)
    d = _per_adapter(spec, x_bf16_rows, adapters, one)
    return np.zeros((x_bf16_rows.shape[0], 2 * spec.I)) if d is None else d


def down_lora_input(h):
    """activation_lora_input: the SwiGLU output in true units (formed from
    the gate and up halves after their own global scales and the up-delta),
    rounded to bf16, before any re-quantisation for the down GEMM."""
    return bf16_round(h)


def down_lora_delta(spec, arr, e, h_lora_rows, adapters=None):
    """Rank-r delta on the down projection: z2 = h_lora A2_e^T (full
    precision), delta = lora_scale * z2 B2_e^T, shape [m, H]; added to the
    expert's output row before the routing-weighted combine. Per-row
    adapters as in lora_delta."""
    def one(a, sel):
        A2 = bf16_decode(lora_mat(spec, arr, "lora_A2", a, e))  # [r, I]
        B2 = bf16_decode(lora_mat(spec, arr, "lora_B2", a, e))  # [H, r]
        return float(np.float32(spec.lora_scale)) * ((h_lora_rows[sel] @ A2.T) @ B2.T)
    d = _per_adapter(spec, h_lora_rows, adapters, one)
    return np.zeros((h_lora_rows.shape[0], spec.H)) if d is None else d


# ----------------------------------------------------------------------------
# rounding decisions of h taken from an fp32 kernel
# ----------------------------------------------------------------------------
# The quantised code of h (FP8 layers) or its bf16 rounding is an integer
# decided by floating point. A kernel that forms g and u with fp32 sums of
# exact products reaches h only to within a small error, so where the exact h
# lies within that error of a rounding boundary both neighbouring codes are
# correct results. These constants bound the kernel-side error used to find
# such boundary elements (they widen the set of admissible results; they do
# not change the oracle's own value):
ACC_REL = 2e-6     # |fp32 sum - exact| <= ACC_REL * sum |terms| (g, u, delta)
EVAL_REL = 2e-6    # relative error of the fp32 SwiGLU evaluation and of s
# GEMM1 of the MXFP4 W4A8 layers runs on a block-scaled matrix instruction
# whose 128-deep sums are not fp32-accurate: a kernel reaches g and u only
# to within ACC_REL_MX * sum |terms| (measured on gfx950: at most 2.0e-5 of
# the block's sum of |products|, 2e-6 over 16 chained blocks)
ACC_REL_MX = 3e-5


def acc_rel(fmt):
    """The kernel-side accumulation bound of a layer format."""
    return ACC_REL_MX if fmt == "mxfp4_a8" else ACC_REL


def swiglu_slopes(g, u, alpha=1.0, beta=0.0, limit=math.inf):
    """|dh/dg|, |dh/du| (one-sided bounds at the clamps)."""
    gp = np.minimum(g, limit)
    up = np.clip(u, -limit, limit)
    sg = sigmoid(alpha * gp)
    dg = np.abs(sg * (1.0 + alpha * gp * (1.0 - sg)) * (up + beta))
    du = np.abs(gp * sg)
    return dg, du


def _e4m3_neighbours(codes):
    """Magnitudes of the next smaller / larger e4m3 values (0 at the ends)."""
    c = np.asarray(codes, np.int64) & 0x7F
    lo = np.where(c > 0, np.abs(e4m3_decode(np.maximum(c - 1, 0))), 0.0)
    hi = np.where(c < 0x7E, np.abs(e4m3_decode(np.minimum(c + 1, 0x7E))), 0.0)
    return lo, hi


def rounding_alternatives(h, err_h, fmt, group=128):
    """For every h element whose exact value lies within err_h of a rounding
    boundary, a bound on |admissible rounded value - oracle's rounded value|
    (every rounding of a value in [h - err_h, h + err_h] is admissible:
    one step plus twice the error); 0 for every other element."""
    h = np.asarray(h, np.float64)
    if fmt == "fp8":
        P, I = h.shape
        hg = h.reshape(P, I // group, group)
        amax = np.abs(hg).max(axis=2).astype(np.float32) if P else \
            np.zeros((0, I // group), np.float32)
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX),
                     np.float32(1.0)).astype(np.float32).astype(np.float64)
        v = np.abs(hg / s[:, :, None])
        ev = np.asarray(err_h, np.float64).reshape(P, I // group, group) / s[:, :, None] \
            + v * EVAL_REL
        q = e4m3_round(v)
        qv = np.abs(e4m3_decode(q))
        lo, hi = _e4m3_neighbours(q)
        near_lo = (q & 0x7F) > 0
        near_lo &= (v - (qv + lo) / 2) <= ev
        near_hi = ((q & 0x7F) < 0x7E) & (((qv + hi) / 2 - v) <= ev)
        step = np.maximum(np.where(near_lo, qv - lo, 0.0), np.where(near_hi, hi - qv, 0.0))
        alt = np.where(near_lo | near_hi, step + 2.0 * ev, 0.0)
        return (alt * s[:, :, None]).reshape(P, I)
    # bf16: rounding is monotone, so the roundings of the values within e of
    # h lie between those of h - e and h + e; the largest step from the
    # oracle's own rounding is at one of the two ends (zero when no rounding
    # boundary lies in the band, whatever the grid spacing there: near 0 and
    # below a power of two it is finer than at h)
    e = np.asarray(err_h) + np.abs(h) * EVAL_REL
    r = bf16_round(h)
    return np.maximum(np.abs(bf16_round(h + e) - r), np.abs(bf16_round(h - e) - r))


def expert_ffn(spec, arr, e, xhat_rows, x_bf16_rows, detail=False, adapters=None):
    """y = round_h(swiglu(g, u)) W2_e^T for the rows of one group.
    xhat_rows are the GEMM1 input values (fp8-dequantised for FP8 layers,
    the bf16 values otherwise); x_bf16_rows feed the LoRA input; adapters
    (per row, with a batch of adapters) select each row's adapter.
    detail=True also returns the bound on y from boundary rounding decisions
    of h (see rounding_alternatives) and the intermediates."""
    I = spec.I
    w13 = w13_dequant(spec, arr, e)
    gu = xhat_rows @ w13.T                         # [m, 2I]
    g, u = gu[:, :I].copy(), gu[:, I:].copy()
    lora = spec.lora_rank and e < spec.n_local
    if lora:
        d = lora_delta(spec, arr, e, x_bf16_rows, adapters)
        g += d[:, :I]
        u += d[:, I:]
    f32 = lambda v: float(np.float32(v))
    al, be, L = f32(spec.alpha), f32(spec.beta), f32(spec.limit)
    h = swiglu(g, u, al, be, L)
    hhat = requant_fp8(h) if spec.fmt == "fp8" else bf16_round(h)
    w2 = w2_dequant(spec, arr, e)
    y = hhat @ w2.T                                # [m, H]
    down = lora and spec.lora_down
    if down:
        y = y + down_lora_delta(spec, arr, e, down_lora_input(h), adapters)
    if not detail:
        return y
    mag = np.abs(xhat_rows) @ np.abs(w13).T
    if lora:
        def mag_one(a, sel):
            A = np.abs(bf16_decode(lora_mat(spec, arr, "lora_A", a, e)))
            B = np.abs(bf16_decode(lora_mat(spec, arr, "lora_B", a, e)))
            return abs(spec.lora_scale) * ((np.abs(x_bf16_rows[sel]) @ A.T) @ B.T)
        mm = _per_adapter(spec, x_bf16_rows, adapters, mag_one)
        if mm is not None:
            mag = mag + mm
    dg, du = swiglu_slopes(g, u, al, be, L)
    err_h = acc_rel(spec.fmt) * (dg * mag[:, :I] + du * mag[:, I:]) + EVAL_REL * np.abs(h)
    alt = rounding_alternatives(h, err_h, spec.fmt)
    y_allow = alt @ np.abs(w2).T
    alt_l = None
    if down:   # boundary decisions of the bf16 down-LoRA input
        alt_l = rounding_alternatives(h, err_h, "bf16")

        def allow_one(a, sel):
            A2 = np.abs(bf16_decode(lora_mat(spec, arr, "lora_A2", a, e)))
            B2 = np.abs(bf16_decode(lora_mat(spec, arr, "lora_B2", a, e)))
            return abs(spec.lora_scale) * ((alt_l[sel] @ A2.T) @ B2.T)
        ya = _per_adapter(spec, alt_l, adapters, allow_one)
        if ya is not None:
            y_allow = y_allow + ya
    return y, dict(h=h, hhat=hhat, alt=alt, y_allow=y_allow,
                   n_boundary=int(np.count_nonzero(alt)), alt_lora=alt_l)


def gemm1_input(spec, x_bits):
    """Values that enter GEMM1: the bf16 x, or for FP8 layers the dequantised
    per-token per-128-column e4m3 codes, or for MXFP4 W4A8 layers the
    dequantised MXFP8 codes (e4m3 times 2^(e - 127) per 32 columns)."""
    x = bf16_decode(x_bits)
    if spec.fmt == "fp8":
        q, s = quant_act_fp8(x.astype(np.float32))
        return e4m3_decode(q) * np.repeat(s.astype(np.float64), 128, axis=1), x
    if spec.fmt == "mxfp4_a8":
        q, e = quant_act_mxfp8(x.astype(np.float32))
        return e4m3_decode(q) * np.repeat(e8m0_decode(e), 32, axis=1), x
    return x, x


def moe_layer(spec, arr, x_bits, logits, tokens=None, routing=None,
              with_allowance=False, adapter_ids=None, workers=1):
    """Output rows out[t, :] (float64) for the tokens asked for (all by
    default): route, rebase, per-expert FFN, then for each token
    sum_j w[t, j] y[t, j] over its local slots in ascending j, plus
    shared_w * y_shared last. `arr` maps array names to per-group indexable
    arrays (a dict of full arrays, or lazy accessors).
    with_allowance=True also returns, per output element, the largest change
    that boundary rounding decisions of h (either neighbour admissible) can
    make: sum_j |w[t, j]| * |alt_h| |W2|^T, and the count of such elements.
    adapter_ids [T] (a batch of adapters): each token's LoRA adapter, -1 for
    none. workers > 1 runs the independent per-expert FFNs on that many
    threads (numpy releases the interpreter lock in its array work); each
    expert's arithmetic and the combine order are unchanged."""
    T = x_bits.shape[0]
    if routing is None:
        routing = route(logits, spec.n_routed, spec.n_sink, spec.top_k,
                        spec.route_scale, spec.global_scale)
    ids, w, _ = routing
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    pairs = {}            # group -> list of (row in output, slot or -1)
    for i, t in enumerate(tokens):
        for j in range(spec.top_k):
            e = int(ids[t, j]) - spec.offset
            if 0 <= int(ids[t, j]) < spec.n_routed and 0 <= e < spec.n_local:
                pairs.setdefault(e, []).append((i, j))
        if spec.shared:
            pairs.setdefault(spec.n_local, []).append((i, -1))
    xhat, xb = gemm1_input(spec, x_bits[tokens])
    contrib, allow = {}, {}
    n_boundary = 0

    def one_expert(e):
        rows = [i for i, _ in pairs[e]]
        ad = None if adapter_ids is None else np.asarray(adapter_ids)[tokens[rows]]
        if with_allowance:
            y, det = expert_ffn(spec, arr, e, xhat[rows], xb[rows], detail=True,
                                adapters=ad)
            return y, det["y_allow"], det["n_boundary"]
        return expert_ffn(spec, arr, e, xhat[rows], xb[rows], adapters=ad), None, 0

    groups = sorted(pairs)
    if workers > 1 and len(groups) > 1:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(one_expert, groups))
    else:
        results = [one_expert(e) for e in groups]
    for e, (y, y_allow, nb) in zip(groups, results):
        n_boundary += nb
        if with_allowance:
            for (i, j), arow in zip(pairs[e], y_allow):
                allow[(i, j)] = arow
        for (i, j), yrow in zip(pairs[e], y):
            contrib[(i, j)] = yrow
    out = np.zeros((len(tokens), spec.H))
    out_allow = np.zeros((len(tokens), spec.H))
    sw = float(np.float32(spec.shared_w))
    for i, t in enumerate(tokens):
        acc = np.zeros(spec.H)
        for j in range(spec.top_k):
            if (i, j) in contrib:
                acc = acc + w[t, j] * contrib[(i, j)]
                if with_allowance:
                    out_allow[i] += abs(w[t, j]) * allow[(i, j)]
        if (i, -1) in contrib:
            acc = acc + sw * contrib[(i, -1)]
            if with_allowance:
                out_allow[i] += abs(sw) * allow[(i, -1)]
        out[i] = acc
    if with_allowance:
        return out, out_allow, n_boundary
    return out
