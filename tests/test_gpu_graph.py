"""A layer call captured into a HIP graph (MoELayer.capture) and replayed:
every replay, on new inputs written into the captured x and with eager layer
calls and synchronisations in between, gives the eager call's outputs bit
for bit (the same kernels on the same inputs; every node is a libmoe
kernel, none a memset)."""

import pytest
import torch

import mixture_experts_layer_40_amd as moe
import synth
from gpu_parity import say

pytestmark = pytest.mark.gpu


def _cfg(base, **kw):
    name = base + "_graph_" + "_".join(f"{k}{v}" for k, v in sorted(kw.items()))
    return synth.scaled_config(base, name=name, **kw)


CASES = {
    # the fp32 layer: separate calls, shared expert on a second stream
    "tiny_f32": synth.get_config("tiny_f32"),
    # bf16, fused experts, split-K router
    "bf16_fused": _cfg("v3_prefill_bf16", T=300, d=256, E=64, K=6, I=128, Is=128),
    # fp8 row scales (decode-like)
    "fp8_decode": _cfg("v3_decode_fp8", T=64, d=512, E=64, K=8, I=256, Is=256),
    # fine-grained fp8: quantise + fp8 experts
    "fp8_block": _cfg("v3_prefill_fp8b", T=200, d=256, E=32, K=4, I=256, Is=256),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_equal_eager_calls(name):
    spec = CASES[name]
    say(f"[graph] {name}")
    inp = synth.make_inputs(spec, "cuda")
    layer = moe.MoELayer(spec, inp)
    bias = inp["bias"]
    x_cap = inp["x"].clone()
    graph = layer.capture(x_cap, bias)
    xs = [synth.make_x(spec, "cuda", batch=b) for b in range(1, 4)]
    for i, xb in enumerate(xs):
        x_cap.copy_(xb)
        graph.replay()
        torch.cuda.synchronize()
        got = {"y": layer.y[:spec.T].clone(), "idx": layer.topk_idx[:spec.T].clone(),
               "load": layer.load.clone(), "slots": layer.out_slots[:spec.T * spec.K].clone()}
        # an eager call on other data in between, then the eager reference
        layer.forward(xs[(i + 1) % len(xs)].clone(), bias)
        torch.cuda.synchronize()
        layer.forward(xb.clone(), bias)
        torch.cuda.synchronize()
        assert torch.equal(got["idx"], layer.topk_idx[:spec.T])
        assert torch.equal(got["load"], layer.load)
        assert torch.equal(got["slots"], layer.out_slots[:spec.T * spec.K])
        assert torch.equal(got["y"], layer.y[:spec.T]), f"replay {i} differs from the eager call"
