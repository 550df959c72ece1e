"""GPU parity of the biased top-k (lmoe_route) on rows built to stress the ordering rules.

The selection is integer output: indices and the k-th / (k+1)-th biased values are compared bit for
bit with the oracle's select_topk fed the GPU's own scores, the routing weights within f32
rounding. Cases: exact ties across experts (duplicated router rows and biases, so equal scores meet
at the selection boundary), the largest k the library takes (64), an expert count that is not a
multiple of the 64-lane wave, one expert count past 1024 (NPL = 32 registers per lane), and a row
count that leaves a partial workgroup. Rows whose winners are all among the keys at or above the
(k+1)-th largest lane maximum take the kernel's candidate pass, the others (k = 64 at E = 128, mass
ties) its exact pass; both are covered here.

The QB histogram of the same rows is compared bin for bin with the oracle's: expert counts that
give the kernel one, two or four experts per workgroup, with and without vector loads of a slice
(E odd), and bin counts from 2 to 32768 (the largest the library takes).
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from latent_space_routed_amd import _lib as C
from oracle import lmoe_oracle as O
from workloads import CONFIGS

from .gpu_helpers import say

pytestmark = pytest.mark.gpu

CASES = {
    # name: (T, D, E, k, duplicate group size of router rows)
    "ties_E128_k8": (301, 256, 128, 8, 4),
    "k64_E128": (130, 256, 128, 64, 1),
    "E100_k7_ties": (77, 128, 100, 7, 5),
    "E2048_k16": (64, 128, 2048, 16, 2),
    "E1001_k16": (200, 128, 1001, 16, 1),
    "E896_k16": (1030, 128, 896, 16, 1),
}
HIST_BINS = {"ties_E128_k8": 2, "k64_E128": 32768, "E100_k7_ties": 37, "E2048_k16": 4096, "E1001_k16": 1000,
             "E896_k16": 1000}


@pytest.mark.parametrize("name", list(CASES))
def test_route_topk_ordering(name):
    T, D, E, k, dup = CASES[name]
    cfg = replace(CONFIGS["mid_bf16"], T=T, d_model=D, n_experts=E, top_k=k, n_bins=HIST_BINS[name])
    rng = np.random.default_rng(31)
    base = (rng.standard_normal((-(-E // dup), D)) * D ** -0.5).astype(np.float32)
    w_router = np.repeat(base, dup, axis=0)[:E].copy()
    bias = np.repeat(rng.choice([0.0, 0.01, -0.02], -(-E // dup)).astype(np.float32), dup)[:E].copy()
    x = O.store(rng.standard_normal((T, D)), "bf16")
    dev = "cuda"
    xd = torch.as_tensor(x).to(torch.bfloat16).to(dev)
    shape = C.make_shape(cfg, T)
    scores = torch.empty(T, E, dtype=torch.float32, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=dev)
    thr = torch.empty(T, 2, dtype=torch.float32, device=dev)
    ws = torch.empty(max(C.workspace_bytes(shape, C.LMOE_CALL_ROUTE), 256), dtype=torch.uint8, device=dev)
    say(f"route {name}: T={T} E={E} k={k} duplicate rows x{dup}")
    C.lmoe_route(shape, xd, torch.as_tensor(w_router).to(dev), torch.as_tensor(bias).to(dev), None, scores, idx, wts,
                 thr, ws)
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    ref_idx, ref_w, ref_thr = O.select_topk(s, bias, k)
    if dup > 1:  # the case really has ties at the boundary
        sb = s + bias[None, :]
        ties = np.sum(sb == ref_thr[:, :1], axis=1) > 1
        say(f"rows with a tie at the k-th value: {int(ties.sum())} of {T}")
        assert ties.any()
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(thr.cpu().numpy(), ref_thr)
    np.testing.assert_allclose(wts.cpu().numpy(), ref_w, rtol=3e-7, atol=0)
    hist = torch.zeros(E, cfg.n_bins, dtype=torch.int32, device=dev)
    C.lmoe_qb_histogram(shape, scores, torch.as_tensor(bias).to(dev), idx, thr, hist)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(hist.cpu().numpy().view(np.uint32),
                                  O.qb_histogram(s, bias, ref_idx, ref_thr, cfg.n_bins))


@pytest.mark.parametrize("offset", [0, 1])
@pytest.mark.parametrize("nb", [2, 100, 1000, 1024, 1025, 4096, 32768])
def test_qb_update_bin_counts(nb, offset):
    """QB bias update on synthetic histograms whose rows each sum to N_acc (concentrated on a band of
    bins, one row all in one bin, one row spread evenly), bit-exact against the oracle for bin counts
    that give one to 512 bins per lane (the kernel keeps up to 16 per lane in registers). offset 1
    passes a histogram that starts 4 bytes into its allocation (not 16-byte aligned), which takes the
    kernel's one-bin accesses instead of its 16-byte ones."""
    E, k, n_acc = 37, 5, 5000
    rng = np.random.default_rng(nb)
    hist = np.zeros((E, nb), dtype=np.uint32)
    for e in range(E):
        if e == 0:
            hist[e, rng.integers(nb)] = n_acc
        elif e == 1:
            hist[e] = rng.multinomial(n_acc, np.full(nb, 1.0 / nb))
        else:
            c = rng.integers(nb)
            w = max(1, nb // 20)
            lo, hi = max(0, c - w), min(nb, c + w + 1)
            p = np.zeros(nb)
            p[lo:hi] = 1.0 / (hi - lo)
            hist[e] = rng.multinomial(n_acc, p)
    bias0 = (rng.standard_normal(E) * 0.01).astype(np.float32)
    cfg = replace(CONFIGS["mid_bf16"], T=64, d_model=128, n_experts=E, top_k=k, n_bins=nb)
    shape = C.make_shape(cfg, 64)
    flat = np.concatenate([np.zeros(offset, dtype=np.int32), hist.view(np.int32).ravel()])
    hd = torch.from_numpy(flat).cuda()[offset:].view(E, nb)
    bd = torch.from_numpy(bias0.copy()).cuda()
    say(f"qb_update E={E} k={k} nb={nb} n_acc={n_acc} offset={offset}")
    C.lmoe_qb_update(shape, hd, n_acc, bd)
    torch.cuda.synchronize()
    want, _ = O.qb_update(hist, n_acc, bias0, k)
    np.testing.assert_array_equal(bd.cpu().numpy(), want)
    assert not hd.cpu().numpy().any()


def test_topk_candidate_pass_boundary():
    """Rows built through an identity router (the logit of expert e is x[t, e]) so that the number of
    keys at or above the (k+1)-th largest lane maximum is exactly 64 (the candidate pass's limit,
    all tied), 65 (one more tie: the exact pass), 128 (every expert tied), 63 tied plus one more in
    a lane that already holds a tied expert, and distinct values. Selection must follow value
    descending, index ascending in every case."""
    T, D, E, k = 5, 128, 128, 8
    cfg = replace(CONFIGS["mid_bf16"], T=T, d_model=D, n_experts=E, top_k=k, n_bins=1000)
    x = np.full((T, D), -1.0, dtype=np.float32)
    x[0, :64] = 2.0                                   # lanes 0..63 each hold one tied key: 64 candidates
    x[1, :64] = 2.0
    x[1, 64] = 2.0                                    # lane 0's second expert ties too: 65 candidates
    x[2, :] = 0.0                                     # all 128 experts tied
    x[3, :63] = 2.0
    x[3, 100] = 2.0                                   # lane 36 holds experts 36 and 100, both tied
    x[4, :] = np.random.default_rng(5).standard_normal(D).astype(np.float32)  # distinct values
    x = O.store(x, "bf16").astype(np.float32)
    w_router = np.eye(E, D, dtype=np.float32)
    bias = np.zeros(E, dtype=np.float32)
    dev = "cuda"
    shape = C.make_shape(cfg, T)
    scores = torch.empty(T, E, dtype=torch.float32, device=dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=dev)
    thr = torch.empty(T, 2, dtype=torch.float32, device=dev)
    ws = torch.empty(max(C.workspace_bytes(shape, C.LMOE_CALL_ROUTE), 256), dtype=torch.uint8, device=dev)
    say("route: candidate-pass boundary rows (64, 65, 128 tied candidates)")
    C.lmoe_route(shape, torch.as_tensor(x).to(torch.bfloat16).to(dev), torch.as_tensor(w_router).to(dev),
                 torch.as_tensor(bias).to(dev), None, scores, idx, wts, thr, ws)
    torch.cuda.synchronize()
    s = scores.cpu().numpy()
    ref_idx, ref_w, ref_thr = O.select_topk(s, bias, k)
    assert (s[0, :64] == s[0, 0]).all() and (s[2] == s[2, 0]).all()  # the ties are exact
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(ref_idx[0], np.arange(k))
    np.testing.assert_array_equal(ref_idx[2], np.arange(k))
    np.testing.assert_array_equal(thr.cpu().numpy(), ref_thr)
    np.testing.assert_allclose(wts.cpu().numpy(), ref_w, rtol=3e-7, atol=0)


@pytest.mark.parametrize("E,k", [(2048, 16), (1001, 16), (2048, 64), (1001, 7)])
def test_permute_large_expert_counts(E, k):
    """The permutation at expert counts whose per-chunk masks and bases need more than the default
    64 KB of LDS (E = 2048, the largest the library takes; with k = 64, the largest k, the scatter's
    LDS also holds 64 KB of pair experts) and at an odd count and an odd k (a token's pairs spread
    unevenly over its four lanes), on random routing with some experts left empty: offsets, sorted
    tokens and slots bit-exact against the oracle."""
    T, D = 700, 128
    cfg = replace(CONFIGS["mid_bf16"], T=T, d_model=D, n_experts=E, top_k=k)
    rng = np.random.default_rng(E + k)
    # each token picks k distinct experts from the first 3/4 of the experts: the rest stay empty
    idx = np.stack([rng.choice(3 * E // 4, k, replace=False) for _ in range(T)]).astype(np.int32)
    dev = "cuda"
    L = cfg.d_latent
    shape = C.make_shape(cfg, T)
    x = torch.randn(T, D, device=dev).to(torch.bfloat16)
    w_down = (torch.randn(L, D, device=dev) * D ** -0.5).to(torch.bfloat16)
    x_lat = torch.empty(T, L, dtype=torch.bfloat16, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    st = torch.empty(T * k, dtype=torch.int32, device=dev)
    sp = torch.empty(T * k, dtype=torch.int32, device=dev)
    ws = torch.empty(max(C.workspace_bytes(shape, C.LMOE_CALL_PERMUTE), 256), dtype=torch.uint8, device=dev)
    say(f"permute: T={T} E={E} k={k}")
    C.lmoe_permute(shape, x, w_down, torch.as_tensor(idx).to(dev), x_lat, off, st, sp, None, ws)
    torch.cuda.synchronize()
    ref_off, ref_st, ref_sp = O.permute(idx, E)
    np.testing.assert_array_equal(off.cpu().numpy(), ref_off)
    np.testing.assert_array_equal(st.cpu().numpy(), ref_st)
    np.testing.assert_array_equal(sp.cpu().numpy(), ref_sp)


def test_permute_drops_repeated_and_out_of_range_ids():
    """Rows that list an expert twice, or ids outside [0, E): each such pair is dropped (slot -1,
    no sorted row), the first occurrence of an expert in a row is kept, and the kept pairs are
    sorted exactly as a stable sort by expert of the kept (token, slot) pairs."""
    T, D, k, E = 600, 128, 8, 40
    cfg = replace(CONFIGS["mid_bf16"], T=T, d_model=D, n_experts=E, top_k=k)
    rng = np.random.default_rng(5)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)       # many rows repeat an expert
    idx[::7, 3] = E + 5                                          # out of range
    idx[::11, 0] = -2
    idx[::13, 1:] = idx[::13, :1]                                # a row of one expert k times
    # expected: keep the first occurrence of each in-range expert in a row, stable sort by expert
    keep = np.zeros((T, k), bool)
    for t in range(T):
        seen = set()
        for j in range(k):
            e = int(idx[t, j])
            if 0 <= e < E and e not in seen:
                keep[t, j] = True
                seen.add(e)
    pairs = [(int(idx[t, j]), t, j) for t in range(T) for j in range(k) if keep[t, j]]
    pairs.sort(key=lambda p: (p[0], p[1]))                       # by expert, tokens ascending
    ref_sp = np.full(T * k, -1, np.int32)
    ref_st = np.empty(len(pairs), np.int32)
    for r, (e, t, j) in enumerate(pairs):
        ref_sp[t * k + j] = r
        ref_st[r] = t
    counts = np.bincount([p[0] for p in pairs], minlength=E)
    ref_off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    dev = "cuda"
    shape = C.make_shape(cfg, T)
    x = torch.randn(T, D, device=dev).to(torch.bfloat16)
    w_down = (torch.randn(cfg.d_latent, D, device=dev) * D ** -0.5).to(torch.bfloat16)
    x_lat = torch.empty(T, cfg.d_latent, dtype=torch.bfloat16, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    st = torch.full((T * k,), -7, dtype=torch.int32, device=dev)
    sp = torch.empty(T * k, dtype=torch.int32, device=dev)
    ws = torch.empty(max(C.workspace_bytes(shape, C.LMOE_CALL_PERMUTE), 256), dtype=torch.uint8, device=dev)
    C.lmoe_permute(shape, x, w_down, torch.as_tensor(idx).to(dev), x_lat, off, st, sp, None, ws)
    torch.cuda.synchronize()
    say(f"permute with dropped pairs: kept {len(pairs)} of {T * k}")
    np.testing.assert_array_equal(off.cpu().numpy(), ref_off)
    np.testing.assert_array_equal(sp.cpu().numpy(), ref_sp)
    np.testing.assert_array_equal(st.cpu().numpy()[: len(pairs)], ref_st)
    assert (st.cpu().numpy()[len(pairs):] == -7).all()           # no sorted row beyond the kept pairs
