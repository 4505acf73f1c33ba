"""GPU parity of the tracked-set scores and the top-k selection that follow
the fused step (jaehun.me review, "How It Works: A Concrete Example", Step 1:
Cache selection), through the C ABI, against the fp64 oracle.

Bar.  A score is a sum of exp(s - LSE) terms; the step's LSE meets 1e-3
absolute and its scores carry the fp32 error of q and the stored k rows, so
each term is within a factor exp(+-2e-3) of the oracle's: elementwise
|gpu - oracle| <= 3e-3 * oracle + 1e-6 * max(oracle).  The top-k of given
fp32 scores is an integer result and must match the oracle's ranking of the
same fp32 values exactly; against the oracle's own scores the selected set
must be a valid top-k up to that tolerance (near-equal scores may swap).
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_kv_amd.binding import FusedKVCache
from io_aware_kv_amd.workloads import (LayerShape, initial_cache, make_random_case, make_workload,
                                       selection_inputs)
from parity_util import log, run_oracle, shape_of

pytestmark = pytest.mark.gpu

RTOL, ATOL_REL = 3e-3, 1e-6


def masked_rows(wl):
    return selection_inputs(wl)[0].numpy()


def decoded_candidates(wl):
    return selection_inputs(wl)[1].numpy()


def run_gpu_selection(wl, sel, cand, k, repeat=1):
    ls = wl.shape
    dev = torch.device("cuda")
    K0, V0 = initial_cache(wl)
    Kc, Vc = K0.to(dev).contiguous(), V0.to(dev).contiguous()
    fk = FusedKVCache(ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, max(1, wl.nq), ls.dtype, ls.rope_base)
    X, W = wl.X.to(dev), wl.W.to(dev)
    Q, P = wl.Q_idx.to(dev), wl.pos_ids.to(dev)
    vis = wl.vis.to(dev) if wl.vis is not None else None
    O = torch.empty((ls.B, wl.nq, ls.H, ls.dh), dtype=ls.dtype, device=dev)
    LSE = torch.empty((ls.B, wl.nq, ls.H), dtype=torch.float32, device=dev)
    fk.step(X, Q, P, vis, W, Kc, Vc, O, LSE)
    sel_d = torch.from_numpy(sel).to(dev)
    cand_d = torch.from_numpy(cand).to(dev)
    runs = []
    for _ in range(repeat):
        scores = torch.full((ls.B, ls.N), float("nan"), dtype=torch.float32, device=dev)
        out = torch.full((ls.B, k), -7, dtype=torch.int32, device=dev)
        fk.tracked_scores(P, vis, sel_d, Kc, LSE, scores)
        fk.select_tracked(scores, cand_d, k, out)
        torch.cuda.synchronize()
        runs.append((scores.cpu(), out.cpu()))
    fk.close()
    return runs


def check_selection(wl, label, k=80):
    sel = masked_rows(wl)
    cand = decoded_candidates(wl)
    runs = run_gpu_selection(wl, sel, cand, k, repeat=2)
    sg, og = runs[-1]
    r = run_oracle(wl)
    ref = oracle.key_scores(shape_of(wl.shape), r["q"], r["Kc"], r["LSE"], wl.pos_ids, wl.vis, sel)
    g = sg.double().numpy()
    assert np.isfinite(g).all(), label + ": non-finite scores"
    err = np.abs(g - ref)
    bound = RTOL * ref + ATOL_REL * max(ref.max(), 1e-30)
    log("%s scores: max rel err %.2e (max score %.3g, %d rows selected)" %
        (label, float((err / np.maximum(ref, 1e-30)).max()), ref.max(), int(sel.sum())))
    assert (err <= bound).all(), "%s: scores off, worst %.3e" % (label, float((err - bound).max()))
    # same bits on a second call
    assert torch.equal(runs[0][0].view(torch.int32), sg.view(torch.int32))
    assert torch.equal(runs[0][1], og)
    # top-k of the GPU's own fp32 scores: exactly the oracle's ranking
    want = oracle.select_top(sg.numpy(), cand, k)
    assert np.array_equal(og.numpy(), want), label + ": top-k differs from the ranking of the same scores"
    # against the oracle's scores: a valid top-k up to the score tolerance
    for b in range(wl.shape.B):
        chosen = [p for p in og[b].tolist() if p >= 0]
        assert len(chosen) == min(k, int(cand[b].sum()))
        rest = np.setdiff1d(np.nonzero(cand[b])[0], chosen)
        if chosen and rest.size:
            lo = ref[b, chosen].min()
            hi = ref[b, rest].max()
            assert lo >= hi - 2 * (RTOL * hi + ATOL_REL * ref.max()), label + ": selection not a top-k"


@pytest.mark.parametrize("cid", [2, 3, 4, 6, 7, 1])
def test_tracked_scores_layer_workloads(cid):
    log("case: tracked scores, workload %d" % cid)
    check_selection(make_workload(cid), "workload%d" % cid, k=80 if cid != 1 else 5)


def test_tracked_scores_gqa_duplicates_mask():
    log("case: tracked scores, GQA with duplicates and a mask")
    ls = LayerShape(B=3, N=700, d_model=256, H=8, Hkv=2, dh=128)
    wl = make_random_case(ls, 40, seed=41, n_extra_rows=8, dup_frac=0.2, masked_vis=True, w_std=0.05)
    check_selection(wl, "gqa-dups-mask", k=33)


def test_tracked_scores_ring_form_gqa_splits():
    """At most 48 (row, head) pairs (20 rows x G = 2): the form that streams K
    through the LDS ring, here with GQA, duplicates, a mask and many key
    splits of 32 keys, so every 64-key tile ends past its split."""
    log("case: tracked scores, ring form, GQA with key splits")
    ls = LayerShape(B=3, N=700, d_model=256, H=4, Hkv=2, dh=128)
    wl = make_random_case(ls, 20, seed=47, n_extra_rows=4, dup_frac=0.2, masked_vis=True, w_std=0.05)
    check_selection(wl, "ring-gqa-splits", k=21)


def test_tracked_scores_many_rows_two_groups():
    """Up to 240 selected (row, head) pairs: the ring form with the pairs
    split across its consumer waves (several row blocks per wave)."""
    log("case: tracked scores, 100 selected rows x G=2")
    ls = LayerShape(B=2, N=300, d_model=128, H=4, Hkv=2, dh=128)
    wl = make_random_case(ls, 120, seed=42, masked_vis=True, w_std=0.05)
    check_selection(wl, "two-row-groups", k=50)


def test_tracked_scores_more_pairs_than_the_ring_forms_hold():
    """More than 256 possible (row, head) pairs (70 rows x G = 4): the direct
    form, which loads its key blocks straight into MFMA fragments."""
    log("case: tracked scores, 70 rows x G=4")
    ls = LayerShape(B=2, N=300, d_model=128, H=8, Hkv=2, dh=128)
    wl = make_random_case(ls, 70, seed=49, n_extra_rows=4, dup_frac=0.1, masked_vis=True, w_std=0.05)
    check_selection(wl, "direct-form", k=40)


def test_select_top_ties_and_short_candidate_lists():
    """Hand-made fp32 scores with many exact ties, N not a power of two,
    k larger than some sequences' candidate counts."""
    log("case: top-k ties")
    B, N, k = 3, 5000, 40
    rng = np.random.default_rng(43)
    sc = (rng.integers(0, 30, size=(B, N)) / 8.0).astype(np.float32)
    cand = (rng.random((B, N)) < 0.5).astype(np.uint8)
    cand[2] = 0
    cand[2, [5, 4999, 17]] = 1
    dev = torch.device("cuda")
    fk = FusedKVCache(B, N, 128, 2, 2, 128, 4, torch.bfloat16)
    out = torch.full((B, k), -7, dtype=torch.int32, device=dev)
    fk.select_tracked(torch.from_numpy(sc).to(dev), torch.from_numpy(cand).to(dev), k, out)
    torch.cuda.synchronize()
    fk.close()
    assert np.array_equal(out.cpu().numpy(), oracle.select_top(sc, cand, k))
    assert out[2, 3:].eq(-1).all()


TOPK_CASES = [
    # (label, B, N, k, pattern)
    ("k-above-N", 2, 37, 45, "ties"),
    ("max-N", 2, 16384, 80, "random"),
    ("max-N-ties", 1, 16384, 300, "ties"),
    ("ragged-N", 3, 1001, 17, "random"),
    ("one-candidate", 2, 64, 5, "one"),
    ("all-equal", 2, 3000, 50, "equal"),
    ("signs-and-zeros", 2, 777, 64, "signed"),
    ("k-one", 4, 2048, 1, "ties"),
    ("k-256", 2, 4096, 256, "ties"),           # the rank-count sort's largest slot count
    ("k-257", 1, 4096, 257, "ties"),           # one past it: the bitonic network
    ("first-digit-decides", 2, 3000, 5, "spikes"),  # each of the top 5 alone in its first-pass bin
    ("k-9000-of-max-N", 1, 16384, 9000, "random"),  # 16384 key slots: the most LDS the kernel takes
]


@pytest.mark.parametrize("label,B,N,k,pattern", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_select_top_edge_cases(label, B, N, k, pattern):
    """The top-k against the oracle's ranking of the same fp32 scores: k at
    or past the candidate count, the largest N, N not a multiple of 16, a
    single candidate, every score equal, negative scores and signed zeros,
    and a k-th score that the first radix digit already separates."""
    log("case: top-k %s" % label)
    rng = np.random.default_rng(44 + N + k)
    if pattern == "random":
        sc = rng.standard_normal((B, N)).astype(np.float32)
    elif pattern == "ties":
        sc = (rng.integers(0, 12, size=(B, N)) / 4.0).astype(np.float32)
    elif pattern == "equal":
        sc = np.full((B, N), 0.375, dtype=np.float32)
    elif pattern == "signed":
        sc = (rng.integers(-6, 7, size=(B, N)) / 2.0).astype(np.float32)
        sc[:, ::5] = -0.0
        sc[:, 1::7] = 0.0
    else:
        sc = rng.standard_normal((B, N)).astype(np.float32)
    cand = (rng.random((B, N)) < 0.6).astype(np.uint8)
    if pattern == "spikes":
        # scores 2^10, 2^14, ..., 2^26 fall in separate bins of the first
        # radix digit (sign and high exponent bits), so the select can stop
        # after one pass
        sc = (rng.standard_normal((B, N)) * 0.1).astype(np.float32)
        for j, p in enumerate((17, 2999, 1500, 4, 777)):
            sc[:, p] = np.float32(2.0 ** (10 + 4 * j))
            cand[:, p] = 1
    if pattern == "one":
        cand[:] = 0
        cand[:, N // 3] = 1
    dev = torch.device("cuda")
    fk = FusedKVCache(B, N, 128, 2, 2, 128, 4, torch.bfloat16)
    out = torch.full((B, k), -7, dtype=torch.int32, device=dev)
    fk.select_tracked(torch.from_numpy(sc).to(dev), torch.from_numpy(cand).to(dev), k, out)
    torch.cuda.synchronize()
    fk.close()
    assert np.array_equal(out.cpu().numpy(), oracle.select_top(sc, cand, k)), label


def test_tracked_scores_no_rows_selected():
    log("case: tracked scores, nothing selected")
    wl = make_workload(2)
    sel = np.zeros((wl.shape.B, wl.nq), dtype=np.uint8)
    cand = decoded_candidates(wl)
    (sg, og), = run_gpu_selection(wl, sel, cand, 10)
    assert torch.all(sg == 0)
    # all scores equal: the lowest candidate positions, in order
    assert og[0].tolist() == np.nonzero(cand[0])[0][:10].tolist()
