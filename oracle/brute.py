"""Brute-force dense formulation of the MoE layer for tiny shapes.

TEST INFRASTRUCTURE, independent of moe_oracle.py (it imports nothing from
it): pure-Python scalar loops over every expert, with its own number-format
handling:
  * e4m3 values come from torch's float8_e4m3fn decoding (a library table),
    e2m1 values from the list of its eight magnitudes, e8m0 as ldexp,
    and rounding to e4m3 is a nearest-value search over that table (ties to
    the even code, saturation at 448);
  * bfloat16 rounding is Python's round-half-even on the scaled value;
  * MXFP8 activations (the W4A8 MXFP4 layers) scan for the smallest power
    of two that keeps a 32-column group within 448 and round each element
    by that same table search;
  * routing sorts the routed columns by (-logit, index) and forms the
    weights as sigmoid(x_i) / sum_j sigmoid(x_j) (the plain form the
    log-sigmoid renormalisation is algebraically equal to, sglang PR #36385,
    "2. Correctness"), valid while float64 sigmoid does not underflow;
  * every expert's output is computed densely; the combine then picks the
    routed ones (so a wrong gather or scatter in the oracle shows up here).
Intended for T <= 8, H, I <= 256.
"""
from __future__ import annotations

import math
import struct

import torch

_E4M3_ALL = torch.arange(256, dtype=torch.int32).to(torch.uint8) \
    .view(torch.float8_e4m3fn).double().tolist()
_E4M3 = [(c, v) for c, v in enumerate(_E4M3_ALL)
         if not math.isnan(v) and c < 0x80]


# the eight e2m1 magnitudes, codes 0..7
_E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _e4m3_table():
    return _E4M3


def e4m3_value(code):
    return _E4M3_ALL[code]


def e4m3_nearest(v):
    """Nearest e4m3 value by exhaustive search; ties go to the even code."""
    if v != v:
        return float("nan")
    a = min(abs(v), 448.0)
    best = None
    for c, val in _e4m3_table():
        d = abs(a - val)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c, val)
    return math.copysign(best[2], v)


def mxfp8_exponent(amax):
    """The smallest e >= -127 with amax <= 448 * 2^e, by scanning upwards."""
    e = -127
    while amax > 448.0 * 2.0 ** e:
        e += 1
    return e


def mxfp8_row(row):
    """MXFP8 values of one activation row: per 32 columns the exponent above
    and the nearest e4m3 value of each element divided by 2^e, times 2^e."""
    out = []
    for c0 in range(0, len(row), 32):
        grp = row[c0:c0 + 32]
        e = mxfp8_exponent(max(abs(v) for v in grp))
        out.extend(e4m3_nearest(v / 2.0 ** e) * 2.0 ** e for v in grp)
    return out


def bf16_nearest(v):
    if v == 0:
        return 0.0
    m, e = math.frexp(abs(v))          # |v| = m * 2^e, m in [0.5, 1)
    q = round(abs(v) * 2.0 ** (8 - e)) * 2.0 ** (e - 8)
    return math.copysign(q, v)


def bf16_bits_value(b):
    """bfloat16 bits are the upper 16 bits of a big-endian binary32."""
    return struct.unpack(">f", bytes([(b >> 8) & 0xFF, b & 0xFF, 0, 0]))[0]


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z)) if z >= 0 else math.exp(z) / (1.0 + math.exp(z))


def route_row(row, n_routed, n_sink, k, scale):
    order = sorted(range(n_routed), key=lambda i: (-row[i], i))[:k]
    act = [row[i] for i in order] + [row[n_routed + s] for s in range(n_sink)]
    sg = [_sig(a) for a in act]
    tot = sum(sg)
    w = [scale * s / tot for s in sg]
    return order, w[:k], w[k:]


def dense_weight(fmt, q, s, N, K, gsc=None):
    """[N][K] list of floats from the stored codes."""
    W = [[0.0] * K for _ in range(N)]
    for n in range(N):
        for kk in range(K):
            if fmt == "bf16":
                v = bf16_bits_value(int(q[n][kk]))
            elif fmt == "fp8":
                v = e4m3_value(int(q[n][kk])) * float(s[n // 128][kk // 128])
            elif fmt == "int4":
                byte = int(q[n][kk // 2])
                nib = byte & 0xF if kk % 2 == 0 else byte >> 4
                v = (nib - 8) * bf16_bits_value(int(s[n][kk // 32]))
            else:                      # nvfp4 | mxfp4(_a8): e2m1 from its value list
                byte = int(q[n][kk // 2])
                nib = byte & 0xF if kk % 2 == 0 else byte >> 4
                v = _E2M1[nib & 7] * (-1.0 if nib & 8 else 1.0)
                if fmt == "nvfp4":
                    v *= e4m3_value(int(s[n][kk // 16]))
                else:
                    v *= math.ldexp(1.0, int(s[n][kk // 32]) - 127)
            if gsc is not None:
                v *= gsc[n]
            W[n][kk] = v
    return W


def layer(spec, arr, x_bits, logits, adapter_ids=None):
    """out[t][h] for every token, float64 Python lists. adapter_ids [T]
    (a batch of adapters): each token's LoRA adapter, -1 for none."""
    T = len(x_bits)
    H, I, k = spec.H, spec.I, spec.top_k
    f32 = lambda v: float(torch.tensor(v, dtype=torch.float32))
    alpha, beta, L = f32(spec.alpha), f32(spec.beta), f32(spec.limit)
    x = [[bf16_bits_value(int(b)) for b in row] for row in x_bits]
    xin = []
    for t in range(T):
        if spec.fmt == "mxfp4_a8":
            xin.append(mxfp8_row(x[t]))
        elif spec.fmt == "fp8":
            row = []
            for c0 in range(0, H, 128):
                grp = [float(torch.tensor(v, dtype=torch.float32)) for v in x[t][c0:c0 + 128]]
                amax = max(abs(v) for v in grp)
                s = float(torch.tensor(amax, dtype=torch.float32) / 448.0) if amax > 0 else 1.0
                for v in grp:
                    qv = float(torch.tensor(v, dtype=torch.float32) / torch.tensor(s, dtype=torch.float32))
                    row.append(e4m3_nearest(qv) * s)
            xin.append(row)
        else:
            xin.append(list(x[t]))
    scale = f32(spec.route_scale) * f32(spec.global_scale)
    G = spec.n_groups
    ys = {}
    for e in range(G):
        gsc = None
        if arr.get("gs") is not None:
            g0, g1 = float(arr["gs"][e][0]), float(arr["gs"][e][1])
            gsc = [g0] * I + [g1] * I
        W13 = dense_weight(spec.fmt, arr["w13_q"][e],
                           None if arr["w13_s"] is None else arr["w13_s"][e], 2 * I, H, gsc)
        gsc2 = None
        if arr.get("gs2") is not None:
            gsc2 = [float(arr["gs2"][e])] * H
        W2 = dense_weight(spec.fmt, arr["w2_q"][e],
                          None if arr["w2_s"] is None else arr["w2_s"][e], H, I, gsc2)
        for t in range(T):
            gu = [sum(xin[t][kk] * W13[n][kk] for kk in range(H)) for n in range(2 * I)]
            a = 0 if adapter_ids is None else int(adapter_ids[t])
            pick = lambda name: arr[name][e] if spec.n_adapters == 1 else arr[name][a][e]
            has_lora = spec.lora_rank and e < spec.n_local and 0 <= a < spec.n_adapters
            if has_lora:
                A = pick("lora_A")
                B = pick("lora_B")
                r = spec.lora_rank
                z = [sum(x[t][kk] * bf16_bits_value(int(A[q][kk])) for kk in range(H))
                     for q in range(r)]
                for n in range(2 * I):
                    gu[n] += f32(spec.lora_scale) * sum(
                        z[q] * bf16_bits_value(int(B[n][q])) for q in range(r))
            h = []
            for n in range(I):
                g = min(gu[n], L)
                u = max(min(gu[I + n], L), -L)
                h.append(g * _sig(alpha * g) * (u + beta))
            dn = None
            if has_lora and spec.lora_down:
                # down LoRA on the true-units SwiGLU output, bf16-rounded
                A2 = pick("lora_A2")
                B2 = pick("lora_B2")
                hl = [bf16_nearest(v) for v in h]
                z2 = [sum(hl[n] * bf16_bits_value(int(A2[q][n])) for n in range(I))
                      for q in range(spec.lora_rank)]
                dn = [f32(spec.lora_scale) * sum(z2[q] * bf16_bits_value(int(B2[m][q]))
                                                 for q in range(spec.lora_rank))
                      for m in range(H)]
            if spec.fmt == "fp8":
                hq = []
                for c0 in range(0, I, 128):
                    grp = h[c0:c0 + 128]
                    amax = float(torch.tensor(max(abs(v) for v in grp), dtype=torch.float32))
                    s = float(torch.tensor(amax, dtype=torch.float32) / 448.0) if amax > 0 else 1.0
                    hq.extend(e4m3_nearest(v / s) * s for v in grp)
                h = hq
            else:
                h = [bf16_nearest(v) for v in h]
            ys[(e, t)] = [sum(h[n] * W2[m][n] for n in range(I)) for m in range(H)]
            if dn is not None:
                ys[(e, t)] = [a + b for a, b in zip(ys[(e, t)], dn)]
    out = []
    for t in range(T):
        ids, w, _ = route_row([float(v) for v in logits[t]], spec.n_routed,
                              spec.n_sink, k, scale)
        acc = [0.0] * H
        for j in range(k):
            e = ids[j] - spec.offset
            if 0 <= e < spec.n_local:
                acc = [a + w[j] * y for a, y in zip(acc, ys[(e, t)])]
        if spec.shared:
            acc = [a + f32(spec.shared_w) * y for a, y in zip(acc, ys[(spec.n_local, t)])]
        out.append(acc)
    return out
