"""lmoe_grouped_situ_glu_noalloc (no workspace: the library's per-device scratch array) against
lmoe_grouped_situ_glu on the same inputs, through the C ABI: the routed experts of a mid-size layer
(ragged groups, rows gathered through sorted_token) on two calls in a row, the second with fewer
tokens, so the scratch array keeps the first call's tile list when the second starts. The two
calls share every kernel and the tile list is rewritten in full, so the outputs are bit-identical.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from latent_space_routed_amd import _lib as C
from workloads import CONFIGS

from .gpu_helpers import cached_inputs, device_layer, say

pytestmark = pytest.mark.gpu


def _routed_inputs(cfg):
    """x_lat, sorted_token and offsets of a forward of the layer (the grouped call's inputs)."""
    inp = cached_inputs(cfg)
    layer, x = device_layer(cfg, inp)
    b = layer.forward(x, accumulate_hist=False)
    torch.cuda.synchronize()
    return layer, b


def _grouped(fn, shape, G, rows, cfg, layer, b, ws=None):
    L, I = cfg.d_latent, cfg.inter
    h = torch.full((rows, I), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.full((rows, L), float("nan"), dtype=torch.bfloat16, device="cuda")
    offs = b["offsets"][: G + 1]
    if ws is None:
        fn(shape, G, rows, L, I, L, b["x_lat"], offs, layer.w["w1"], layer.w["w2"], h, y,
           a_row_index=b["sorted_token"])
    else:
        fn(shape, G, rows, L, I, L, b["x_lat"], offs, layer.w["w1"], layer.w["w2"], h, y, ws,
           a_row_index=b["sorted_token"])
    return h, y


def test_noalloc_matches_workspace_call_twice():
    """Two no-alloc calls in a row, the second smaller (fewer tokens and only the first 100 of the
    128 groups), each bit-identical to the workspace call on the same inputs."""
    runs = []
    for T, G in ((1000, 128), (300, 100)):
        cfg = replace(CONFIGS["mid_bf16"], T=T)
        layer, b = _routed_inputs(cfg)
        rows = int(b["offsets"][G].item())
        runs.append((cfg, layer, b, G, rows))
    got = []
    for cfg, layer, b, G, rows in runs:  # the no-alloc calls back to back
        got.append(_grouped(C.lmoe_grouped_situ_glu_noalloc, C.make_shape(cfg, cfg.T), G, rows, cfg, layer, b))
    torch.cuda.synchronize()
    for (cfg, layer, b, G, rows), (h1, y1) in zip(runs, got):
        shape = C.make_shape(cfg, cfg.T)
        ws = torch.empty(max(C.workspace_bytes(shape, C.LMOE_CALL_GROUPED_GLU), 256), dtype=torch.uint8,
                         device="cuda")
        h0, y0 = _grouped(C.lmoe_grouped_situ_glu, shape, G, rows, cfg, layer, b, ws)
        torch.cuda.synchronize()
        assert torch.equal(h1.view(torch.int16), h0.view(torch.int16)), f"h differs (T={cfg.T}, G={G})"
        assert torch.equal(y1.view(torch.int16), y0.view(torch.int16)), f"y differs (T={cfg.T}, G={G})"
        say(f"[noalloc] T={cfg.T}, {G} groups, {rows} rows: bit-identical to the workspace call")


def test_noalloc_dense_one_group_and_limits():
    """One dense group (the shared experts' shape): the same as the workspace call with no split-K
    partials; more groups than the scratch array holds is rejected before any launch."""
    cfg = replace(CONFIGS["mid_bf16"], T=256)
    inp = cached_inputs(cfg)
    layer, x = device_layer(cfg, inp)
    shape = C.make_shape(cfg, cfg.T)
    S, Is, D = cfg.n_shared, cfg.inter_shared, cfg.d_model
    h0 = torch.empty(cfg.T, S * Is, dtype=torch.bfloat16, device="cuda")
    h1 = torch.empty_like(h0)
    C.lmoe_grouped_situ_glu(shape, 1, cfg.T, D, S * Is, D, x, None, layer.w1s_packed, None, h0, None, None)
    C.lmoe_grouped_situ_glu_noalloc(shape, 1, cfg.T, D, S * Is, D, x, None, layer.w1s_packed, None, h1, None)
    torch.cuda.synchronize()
    assert torch.equal(h0.view(torch.int16), h1.view(torch.int16))
    offs = torch.zeros(4097, dtype=torch.int32, device="cuda")
    with pytest.raises(C.LmoeError) as e:
        C.lmoe_grouped_situ_glu_noalloc(shape, 4096, 16, 64, 64, 64, x, offs, layer.w1s_packed, None, h1, None)
    assert e.value.status == C.LMOE_ERR_UNSUPPORTED
