"""moe_forward captured in a HIP graph (torch.cuda.graph) and replayed.

The path allocates nothing and records no memset, so a captured forward
replays on its captured buffers. Each case runs the eager forward, captures
one forward into a graph, then replays it several times with eager work and
synchronisations in between (a different batch through the eager path),
checking every replay bit for bit against the eager result.
"""
import numpy as np
import pytest
import torch

from synth import CONFIGS, FP4_CONFIGS, make_batch, make_layer
from tests.gpu_helpers import module_for

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")]

CASES = [
    # decode: one-launch front end, split-K GEMM1 + its epilogue kernel
    ("fp8_clamp_288", dict(H=2048, I=1024, n_routed=64, cfg_id=61), 1),
    # EP share with both LoRAs and a batch of adapters, plain kernels
    ("ep_lora_258", dict(H=512, I=512, cfg_id=62, n_adapters=8, lora_down=True), 37),
    # NVFP4 decode
    ("nvfp4_lora_258", dict(H=2048, I=1024, cfg_id=63), 2),
]


@pytest.mark.parametrize("name,over,T", CASES)
def test_graph_replay_matches_eager(name, over, T):
    print(f"[case] graph {name} {over} T={T}", flush=True)
    spec = {**CONFIGS, **FP4_CONFIGS}[name].scaled(name=f"{name}_graph", **over)
    layer = make_layer(spec, device="cuda")
    mod = module_for(spec, layer)
    batch = make_batch(spec, layer, T, device="cuda")
    other = make_batch(spec, layer, T, device="cuda", seed_extra=5)
    ad = batch.adapter_ids
    mod.set_adapters(ad)
    outs = mod.alloc_outputs(T)
    mod.workspace(T)
    mod.forward(batch.x, batch.logits, outs, adapter_ids=ad)      # eager reference
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items() if v is not None}
    # capture on a side stream with the same inputs and outputs
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mod.forward(batch.x, batch.logits, outs, adapter_ids=ad)  # warm-up on the stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        mod.forward(batch.x, batch.logits, outs, adapter_ids=ad)
    torch.cuda.synchronize()
    for rep in range(4):
        for v in outs.values():
            if v is not None and v.dtype == torch.float32:
                v.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            if k == "err_word":
                continue
            assert torch.equal(outs[k], v), (rep, k)
        # eager work in between: another batch through its own outputs
        o2 = mod.forward(other.x, other.logits, adapter_ids=other.adapter_ids)
        torch.cuda.synchronize()
        assert torch.isfinite(o2["out"]).all()
        mod.set_adapters(ad)
    assert int(outs["err_word"].cpu()[0]) == 0
