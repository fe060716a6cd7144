"""Parity at the full layer sizes, in the launch configuration bench.py
times (MoeModule.forward -> moe_forward with a workspace sized for T):

- routing ids of every token bit-exactly and routing weights of every
  token to rtol = atol = 2e-3 against the oracle;
- the device error word stays clear;
- output rows against the oracle, element by element: every token when
  T <= 64, else 64 tokens (the first, the last and evenly spaced ones in
  between); max|err| <= tol * RMS and cosine >= 0.9999 (tol 1e-2 FP8/4-bit,
  5e-3 BF16); the error left beyond the boundary-rounding allowance is
  logged beside it;
- a token with no slot on this GPU's experts (expert-parallel share, no
  shared expert) gets an exactly zero row.
"""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from synth import CONFIGS, EXT_CONFIGS, FP4_CONFIGS, make_batch, make_layer, to_numpy_batch
from tests.gpu_helpers import LazyExperts, compare, module_for, tolerance

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")]

# every configured token count of the five layers, the EP share with the
# down LoRA as well, and the FP4 layers; cases of one layer stay together
FULL = [("fp8_clamp_288", 4096), ("fp8_clamp_288", 64), ("fp8_clamp_288", 1),
        ("fp8_oai_128_skew", 4096), ("fp8_oai_128_skew", 64), ("fp8_oai_128_skew", 1),
        ("int4_g32_64", 2048), ("int4_g32_64", 64), ("int4_g32_64", 1),
        ("ep_lora_258", 8192), ("ep_lora_258", 512), ("ep_lora_258", 37),
        ("ep_lora_258", 1),
        ("ep_lora_258_down", 8192), ("ep_lora_258_down", 37),
        ("nvfp4_lora_258", 8192), ("nvfp4_lora_258", 37), ("nvfp4_lora_258", 1),
        ("mxfp4_g32_64", 2048), ("mxfp4_g32_64", 1),
        ("mxfp4a8_g32_64", 2048), ("mxfp4a8_g32_64", 64), ("mxfp4a8_g32_64", 1)]
N_ROWS = 64           # compared output rows per case (all of them when T <= 64)
ORACLE_THREADS = 8    # per-expert FFNs of the oracle run side by side

_layers = {}


def _layer(name):
    if name not in _layers:
        _layers.clear()                 # one full-size layer resident at a time
        spec = {**CONFIGS, **EXT_CONFIGS, **FP4_CONFIGS}[name]
        layer = make_layer(spec, device="cuda")
        _layers[name] = (spec, layer, module_for(spec, layer))
    return _layers[name]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,T", FULL)
def test_full_size_forward(name, T):
    n_sample = min(T, N_ROWS)
    print(f"[case] full-size {name} T={T} compared rows={n_sample}", flush=True)
    spec, layer, mod = _layer(name)
    batch = make_batch(spec, layer, T, device="cuda")
    outs = mod.alloc_outputs(T)
    mod.workspace(T)
    mod.forward(batch.x, batch.logits, outs)
    torch.cuda.synchronize()
    assert int(outs["err_word"].cpu()[0]) == 0
    nb = to_numpy_batch(batch)
    routing = O.route(nb["logits"], spec.n_routed, spec.n_sink, spec.top_k,
                      spec.route_scale, spec.global_scale)
    ids, w, sw = routing
    assert np.array_equal(outs["topk_ids"].cpu().numpy(), ids)
    np.testing.assert_allclose(outs["topk_w"].cpu().numpy(), w, rtol=2e-3, atol=2e-3)

    tokens = np.unique(np.linspace(0, T - 1, n_sample).round().astype(int))
    ref, allow, _ = O.moe_layer(spec, LazyExperts(layer), nb["x_bits"], nb["logits"],
                                tokens=tokens, routing=routing, with_allowance=True,
                                workers=ORACLE_THREADS)
    got = outs["out"][torch.as_tensor(tokens, device="cuda")].double().cpu().numpy()
    tol, cmin = tolerance(spec.fmt)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    if rms == 0.0:          # no sampled token has a slot on this GPU's experts
        print(f"  rows={len(tokens)} reference rows all zero", flush=True)
        assert np.count_nonzero(got) == 0
        return
    rel_raw, cos = compare(got, ref)
    excess = float(np.max(np.abs(got - ref) - allow)) / rms
    print(f"  rows={len(tokens)} max|err|/rms={rel_raw:.3e} "
          f"beyond-allowance={excess:.3e} cos={cos:.8f}", flush=True)
    assert rel_raw <= tol, (rel_raw, tol)
    assert excess <= tol
    assert cos >= cmin

    if spec.n_local < spec.n_routed and not spec.shared:
        e_loc = ids - spec.offset
        none_local = ~np.any((e_loc >= 0) & (e_loc < spec.n_local), axis=1)
        idx = np.nonzero(none_local)[0]
        if len(idx):
            rows = outs["out"][torch.as_tensor(idx, device="cuda")]
            assert torch.count_nonzero(rows).item() == 0
