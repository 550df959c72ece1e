"""Host-side logic of the layer (no GPU): when the shared experts' GEMM1 goes to the side stream."""
from dataclasses import replace
from types import SimpleNamespace

import pytest

from latent_space_routed_amd.layer import LatentMoE
from workloads import CONFIGS


def overlapped(cfg, T=None, overlap=None, fused=True, mx=False):
    fake = SimpleNamespace(cfg=cfg, fused=fused, mx=mx, overlap_shared=overlap)
    return LatentMoE._overlapped(fake, cfg.T if T is None else T)


@pytest.mark.parametrize("name,want", [("tiny_f32", False), ("mid_bf16", True), ("k3_prefill", True),
                                       ("k3_decode", True), ("k3_stress", False)])
def test_side_stream_by_shared_gemm_size(name, want):
    # on when the shared GEMM1 of the batch, 2 T D (2 S Is) flops, is at least 1 GFLOP and the batch
    # holds at most 16384 tokens
    assert overlapped(CONFIGS[name]) is want


def test_side_stream_threshold_follows_the_batch():
    cfg = CONFIGS["k3_prefill"]  # 4 T D S Is = 1 GFLOP at T = 1e9 / (4 * 7168 * 2 * 2048) = 8.5 tokens
    assert not overlapped(cfg, T=8)
    assert overlapped(cfg, T=9)
    assert overlapped(cfg, T=16384) and not overlapped(cfg, T=16385)
    assert overlapped(cfg, T=32768, overlap=True)


def test_side_stream_explicit_setting_and_exclusions():
    cfg = CONFIGS["k3_prefill"]
    assert overlapped(cfg, overlap=True) and not overlapped(cfg, overlap=False)
    assert overlapped(CONFIGS["tiny_f32"], overlap=True)  # forced on below the threshold
    assert overlapped(cfg, mx=True) and not overlapped(cfg, mx=True, overlap=False)
    assert not overlapped(cfg, fused=False, overlap=True)  # the unfused path adds f32 y_sh on one stream
    assert not overlapped(replace(cfg, n_shared=0), overlap=True)
