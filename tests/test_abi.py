"""The C-ABI library loads and exports every symbol include/lmoe.h declares; host-side argument
validation answers before any GPU work (no compute calls here, so this runs without a GPU)."""
import ctypes
import os
import re

import pytest

from latent_space_routed_amd import _lib as C
from workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmoe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(C.LIB_PATH):
        from latent_space_routed_amd import build
        build.build()
    return C.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lmoe_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(C.EXPORTS) == names


def test_status_strings(lib):
    for code, name in enumerate(["LMOE_OK", "LMOE_ERR_INVALID_ARGUMENT", "LMOE_ERR_UNSUPPORTED",
                                 "LMOE_ERR_WORKSPACE", "LMOE_ERR_HIP"]):
        assert C.status_string(code) == name


def test_workspace_sizes(lib):
    k3 = C.make_shape(CONFIGS["k3_prefill"])
    # bf16 split of W_r, then two f32 partials of the router GEMM: its 128 256x256 tiles fill half
    # the chip, so the 3 x 7168 contraction is split in two halves on the DMA pipeline
    assert C.workspace_bytes(k3, C.LMOE_CALL_ROUTE) == 3 * 896 * 7168 * 2 + 2 * 8192 * 896 * 4
    assert C.workspace_bytes(k3, C.LMOE_CALL_PERMUTE) == 32 * 896 * 4             # per-chunk counts
    assert C.workspace_bytes(k3, C.LMOE_CALL_GROUPED_GLU) == 3840                # tile prefix, rounded
    # f32 router: no weight split; 64 tokens x 32 experts split K = 256 in two f32 partials
    assert C.workspace_bytes(C.make_shape(CONFIGS["tiny_f32"]), C.LMOE_CALL_ROUTE) == 2 * 64 * 32 * 4
    assert C.workspace_bytes(k3, C.LMOE_CALL_COMBINE_NORM_UP) == 0                # 8192 rows fill the chip
    bad = C.make_shape(CONFIGS["k3_prefill"])
    bad.top_k = bad.n_experts
    assert C.workspace_bytes(bad, C.LMOE_CALL_ROUTE) == 0


def test_split_k_workspace_for_small_batches(lib):
    """A 64-token batch splits the contraction of its dense GEMMs: the workspace grows by whole
    f32 partial products [splits, T, n_cols] beyond each call's own minimum."""
    dec = C.make_shape(CONFIGS["k3_decode"])
    T, D, L, E = 64, 7168, 3584, 896
    extra = C.workspace_bytes(dec, C.LMOE_CALL_ROUTE) - 3 * E * D * 2
    assert extra > 0 and extra % (T * E * 4) == 0 and 2 <= extra // (T * E * 4) <= 64
    # router: chunks divide d_model (the K-wrap of the bf16 split), about 256 workgroups over 7 tiles
    assert (3 * D) % (3 * D // (extra // (T * E * 4))) == 0 and 7 * (extra // (T * E * 4)) >= 256
    extra = C.workspace_bytes(dec, C.LMOE_CALL_PERMUTE) - 896 * 4                 # one chunk of E counts
    assert extra > 0 and extra % (T * L * 4) == 0
    assert C.workspace_bytes(dec, C.LMOE_CALL_COMBINE_NORM_UP) % (T * D * 4) == 0
    assert C.workspace_bytes(dec, C.LMOE_CALL_COMBINE_NORM_UP) >= 2 * T * D * 4


@pytest.mark.parametrize("field,value,status", [
    ("top_k", 896, C.LMOE_ERR_INVALID_ARGUMENT),     # (k+1)-th score must exist
    ("top_k", 0, C.LMOE_ERR_INVALID_ARGUMENT),
    ("T", -1, C.LMOE_ERR_INVALID_ARGUMENT),
    ("act_dtype", 7, C.LMOE_ERR_INVALID_ARGUMENT),
    ("d_latent", 3583, C.LMOE_ERR_UNSUPPORTED),      # not a multiple of 64
    ("n_bins", 1, C.LMOE_ERR_UNSUPPORTED),
    ("n_experts", 4096, C.LMOE_ERR_UNSUPPORTED),
])
def test_shape_validation_before_any_launch(lib, field, value, status):
    sh = C.make_shape(CONFIGS["k3_prefill"])
    setattr(sh, field, value)
    null = None
    assert lib.lmoe_route(ctypes.byref(sh), null, null, null, null, null, null, null, null, null, null, 0, null) == \
        status
    assert lib.lmoe_split_router(ctypes.byref(sh), null, null, null) == status
    assert lib.lmoe_qb_histogram(ctypes.byref(sh), null, null, null, null, null, null) == status
    assert lib.lmoe_qb_update(ctypes.byref(sh), null, 1, null, null) == status


def test_pointer_validation_before_any_launch(lib):
    sh = C.make_shape(CONFIGS["k3_prefill"])
    null = None
    fake = ctypes.c_void_p(0x1000)        # aligned, never dereferenced: validation fails first
    misaligned = ctypes.c_void_p(0x1002)
    assert lib.lmoe_qb_update(ctypes.byref(sh), null, 1, fake, null) == C.LMOE_ERR_INVALID_ARGUMENT
    assert lib.lmoe_qb_histogram(ctypes.byref(sh), misaligned, fake, fake, fake, fake, null) == \
        C.LMOE_ERR_INVALID_ARGUMENT
    # route with every pointer plausible but no workspace -> workspace error, still no launch
    assert lib.lmoe_route(ctypes.byref(sh), fake, fake, null, fake, null, fake, fake, fake, fake, null, 0, null) == \
        C.LMOE_ERR_WORKSPACE
    # with the router weights split beforehand the call needs no workspace at T = 8192 (its split-K
    # partials are optional): validation passes; the misaligned split is rejected first here
    assert lib.lmoe_route(ctypes.byref(sh), fake, null, misaligned, fake, null, fake, fake, fake, fake, null, 0,
                          null) == C.LMOE_ERR_INVALID_ARGUMENT
    # the split is a bf16-layer call; an f32 layer given a split is an error
    f32 = C.make_shape(CONFIGS["tiny_f32"])
    assert lib.lmoe_split_router(ctypes.byref(f32), fake, fake, null) == C.LMOE_ERR_UNSUPPORTED
    assert lib.lmoe_split_router(ctypes.byref(sh), fake, misaligned, null) == C.LMOE_ERR_INVALID_ARGUMENT
    assert lib.lmoe_route(ctypes.byref(f32), fake, fake, fake, fake, null, fake, fake, fake, fake, fake, 1 << 20,
                          null) == C.LMOE_ERR_INVALID_ARGUMENT
    # grouped GLU: a row gather needs a_rows consistent; K not a multiple of 64 is unsupported
    assert lib.lmoe_grouped_situ_glu(ctypes.byref(sh), 1, 16, 100, 64, 64, fake, 16, null, null, fake, fake, fake,
                                     fake, 0, null, 0, null) == C.LMOE_ERR_UNSUPPORTED
    assert lib.lmoe_grouped_situ_glu(ctypes.byref(sh), 1, 16, 128, 64, 64, fake, 8, null, null, fake, fake, fake,
                                     fake, 0, null, 0, null) == C.LMOE_ERR_INVALID_ARGUMENT
    # combine: y_shared and the folded shared pair are exclusive
    assert lib.lmoe_combine_norm_up(ctypes.byref(sh), fake, fake, fake, null, fake, fake, fake, fake, fake, fake, 0,
                                    null, 0, null) == C.LMOE_ERR_INVALID_ARGUMENT
    # the split calls check the same arguments
    assert lib.lmoe_up_project(ctypes.byref(sh), fake, fake, fake, fake, fake, fake, 0, null, 0, null) == \
        C.LMOE_ERR_INVALID_ARGUMENT
    assert lib.lmoe_up_project(ctypes.byref(sh), misaligned, fake, null, null, null, fake, 0, null, 0, null) == \
        C.LMOE_ERR_INVALID_ARGUMENT
    assert lib.lmoe_up_project(ctypes.byref(sh), fake, fake, null, null, null, fake, 7, null, 0, null) == \
        C.LMOE_ERR_INVALID_ARGUMENT
    assert lib.lmoe_combine_norm(ctypes.byref(sh), misaligned, fake, fake, null, fake, null) == \
        C.LMOE_ERR_INVALID_ARGUMENT


def test_empty_batch_is_a_no_op(lib):
    sh = C.make_shape(CONFIGS["k3_prefill"], T=0)
    null = None
    assert lib.lmoe_route(ctypes.byref(sh), null, null, null, null, null, null, null, null, null, null, 0, null) == \
        C.LMOE_OK
    assert lib.lmoe_qb_histogram(ctypes.byref(sh), null, null, null, null, null, null) == C.LMOE_OK
    assert lib.lmoe_combine_norm_up(ctypes.byref(sh), null, null, null, null, null, null, null, null, null, null, 0,
                                    null, 0, null) == C.LMOE_OK
    assert lib.lmoe_combine_norm(ctypes.byref(sh), null, null, null, null, null, null) == C.LMOE_OK
    assert lib.lmoe_up_project(ctypes.byref(sh), null, null, null, null, null, null, 0, null, 0, null) == C.LMOE_OK


def test_backward_workspace_and_validation(lib):
    """Backward calls: workspace sizes for every call id, argument checks before any launch."""
    k3 = C.make_shape(CONFIGS["k3_prefill"])
    for which in (C.LMOE_CALL_BWD_UP, C.LMOE_CALL_BWD_COMBINE_NORM, C.LMOE_CALL_BWD_EXPERTS, C.LMOE_CALL_BWD_DOWN,
                  C.LMOE_CALL_BWD_SHARED):
        assert C.workspace_bytes(k3, which) > 0
    # experts: three tile prefixes, then [L + I + 2I + L] x (T*k + 64 E) transposed activations
    kp = 8192 * 16 + 64 * 896
    assert C.workspace_bytes(k3, C.LMOE_CALL_BWD_EXPERTS) == 3 * 3840 + (3584 * 2 + 3 * 512) * kp * 2
    big = C.make_shape(CONFIGS["k3_prefill"])
    big.d_latent = 4096 + 64                                   # past the combine backward row limit (bf16)
    null = None
    fake = ctypes.c_void_p(0x1000)
    assert lib.lmoe_bwd_router(ctypes.byref(big), *([fake] * 9), null) == C.LMOE_ERR_UNSUPPORTED
    assert lib.lmoe_bwd_router(ctypes.byref(k3), fake, fake, fake, fake, fake, fake, fake, fake, null, null) == \
        C.LMOE_ERR_INVALID_ARGUMENT
    assert lib.lmoe_bwd_up(ctypes.byref(k3), *([fake] * 9), null, 0, null) == C.LMOE_ERR_WORKSPACE


def test_mx_workspace_and_validation(lib):
    """MX calls: the grouped call's workspace (tile list + FP8 h + its scales), argument checks
    before any launch."""
    k3 = C.make_shape(CONFIGS["k3_prefill"])
    rows, inter = 8192 * 16, 512
    want = 3840 + rows * inter + rows * inter // 32           # (896 + 1) * 4 rounded to 256
    assert C.workspace_bytes(k3, C.LMOE_CALL_GROUPED_GLU_MX) == want
    null = None
    fake = ctypes.c_void_p(0x1000)
    sh = ctypes.byref(k3)
    # quantise: unknown format, K not a multiple of 32, rows = 0 is a no-op, misaligned codes
    assert lib.lmoe_mx_quantize(sh, 5, 4, 64, fake, fake, fake, null) == C.LMOE_ERR_INVALID_ARGUMENT
    assert lib.lmoe_mx_quantize(sh, C.LMOE_MX_FP8, 4, 48, fake, fake, fake, null) == C.LMOE_ERR_UNSUPPORTED
    assert lib.lmoe_mx_quantize(sh, C.LMOE_MX_FP4, 0, 64, null, null, null, null) == C.LMOE_OK
    assert lib.lmoe_mx_quantize(sh, C.LMOE_MX_FP4, 4, 64, fake, ctypes.c_void_p(0x1004), fake, null) == \
        C.LMOE_ERR_INVALID_ARGUMENT
    args = [fake] * 2 + [16, null, null] + [fake] * 6
    # grouped MX: K or inter not a multiple of 128, f32 layers, missing workspace
    assert lib.lmoe_grouped_situ_glu_mx(sh, 1, 16, 192, 128, 256, *args, null, 0, null) == C.LMOE_ERR_UNSUPPORTED
    assert lib.lmoe_grouped_situ_glu_mx(sh, 1, 16, 256, 64, 256, *args, null, 0, null) == C.LMOE_ERR_UNSUPPORTED
    assert lib.lmoe_grouped_situ_glu_mx(sh, 1, 16, 256, 128, 256, *args, null, 0, null) == C.LMOE_ERR_WORKSPACE
    f32 = C.make_shape(CONFIGS["tiny_f32"])
    assert lib.lmoe_grouped_situ_glu_mx(ctypes.byref(f32), 1, 16, 256, 128, 256, *args, fake, 1 << 20, null) == \
        C.LMOE_ERR_UNSUPPORTED
    assert lib.lmoe_grouped_situ_glu_mx(sh, 2, 16, 256, 128, 256, *args, fake, 1 << 20, null) == \
        C.LMOE_ERR_INVALID_ARGUMENT                            # several groups need group offsets
