"""GPU: a step recorded as a HIP graph (LatentMoE.capture_step) replays exactly like eager steps.

Two layers share the weights; one runs eager steps (forward, then the QB update), the other replays
its captured step. After every step the outputs, the routing and the moved bias must be bit-identical
(the kernels are deterministic and the graph holds the same launches). Between replays the test does
eager work of its own and synchronises, and the input is overwritten in place with another batch, so
each replay must read the current input and carry the bias forward.
"""
import numpy as np
import pytest
import torch

from latent_space_routed_amd import LatentMoE, to_device
from workloads import CONFIGS
from workloads.inputs import token_rows

from .gpu_helpers import cached_inputs, device_layer, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,mx", [("mid_bf16", False), ("k3_decode", False), ("k3_prefill", False), ("mid_bf16", True)])
def test_graph_replays_match_eager(name, mx):
    cfg = CONFIGS[name]
    inp = cached_inputs(cfg)
    base, x = device_layer(cfg, inp)
    weights = base.w
    del base
    eager = LatentMoE(cfg, weights, mx=mx)
    graphed = LatentMoE(cfg, weights, mx=mx)
    xg = x.clone()
    eager.forward(x)  # set-up launches (function attributes) happen outside the capture
    eager.qb_update()
    eager.bias.copy_(graphed.bias)
    torch.cuda.synchronize()
    g, bg = graphed.capture_step(xg)
    torch.cuda.synchronize()
    for step in range(4):
        if step:
            xs = to_device(token_rows(cfg, 0, step), cfg.act_dtype)
            x.copy_(xs)
            xg.copy_(xs)
        say(f"[graph] {name} mx={mx} step {step}")
        be = eager.forward(x)
        eager.qb_update()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in ("idx", "thresh", "offsets", "slot_of_pair", "out"):
            a, b = be[key], bg[key]
            assert torch.equal(a, b), f"{name} step {step}: {key} differs between eager and replay"
        assert torch.equal(eager.bias, graphed.bias), f"{name} step {step}: bias differs"
        assert not graphed.hist.any()
        scratch = torch.randn(1 << 20, device="cuda").sum().item()  # eager work of the test's own
        assert np.isfinite(scratch)
