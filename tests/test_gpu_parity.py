"""GPU parity of the fused KV-cache step (HIP path through the C ABI) against
the fp64 oracle, on seeded inputs: the layer workloads at full size in the
launch configuration the bench times, on hidden states and weights with the
stated spreads and the full bf16 significand (and, for the bit-level checks of
the stored rows, on the same workloads snapped to a dyadic grid), small cases
that span several tiles with ragged tails, duplicates and masks, forced split counts, the
scalar kernel family, determinism, the views' mutual invisibility and the
chain-rule mask's dependencies, the largest verification window, edge
positions and empty key sets."""
import zlib

import numpy as np
import pytest
import torch

from io_aware_kv_amd.workloads import LayerShape, make_random_case, make_workload
from parity_util import compare, log, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 6, 7])
def test_layer_workload_full_size(cid):
    """X ~ N(0, 1), W ~ N(0, 0.02^2) drawn in fp32 and cast once to the
    layer's dtype: written k/v and O within 2e-2 (fp32 layer: 1e-4) of the
    oracle's max, every written k/v element within one bf16 unit of the exact
    value, LSE within 1e-3."""
    log("case: workload %d full size" % cid)
    wl = make_workload(cid)
    assert not wl.meta["grid"]
    g = run_gpu(wl)
    r = run_oracle(wl)
    compare(wl, g, r, "workload%d" % cid)


@pytest.mark.parametrize("cid", [2, 3, 6])
def test_layer_workload_grid_bits(cid):
    """The same workloads on the dyadic grid, where the fp32 projection is
    exact in any order: every written v element is the oracle's rounding bit
    for bit, every written k element too except at a rotation tie."""
    log("case: workload %d on the dyadic grid" % cid)
    wl = make_workload(cid, grid=True)
    g = run_gpu(wl)
    r = run_oracle(wl)
    errs = compare(wl, g, r, "workload%d-grid" % cid)
    assert "k_ties" in errs


def test_verification_window_all_exploratory():
    """The largest verification query set of the default window: no confident
    position, 64 exploratory positions in both views (nq = 208)."""
    log("case: workload 7, all exploratory")
    wl = make_workload(7, n_confident=0)
    assert wl.nq == 208
    g = run_gpu(wl)
    compare(wl, g, run_oracle(wl), "workload7-all-exploratory")


def test_chain_mask_dependencies_on_gpu():
    """Under the chain-rule mask the draft row of the last exploratory position
    is seen by no mask-view row, and the mask row of the first is seen by no
    other row: perturbing either leaves every other row's O and LSE
    bit-identical."""
    log("case: chain mask dependencies")
    wl = make_workload(7)
    groups = wl.meta["groups"]
    base = run_gpu(wl)
    for view, pick in (("draft", -1), ("mask", 0)):
        X2 = wl.X.clone()
        moved = []
        for b in range(wl.shape.B):
            rows = [i for i, t in enumerate(groups[b]) if t == view]
            i = rows[pick]
            moved.append(i)
            r = int(wl.Q_idx[b, i])
            X2[b, r] = (X2[b, r].float() + 2.0).to(X2.dtype)
        pert = run_gpu(wl, X=X2)
        for b in range(wl.shape.B):
            if view == "draft":
                same = [i for i, t in enumerate(groups[b]) if t == "mask"]
            else:
                same = [i for i in range(wl.nq) if i != moved[b]]
            assert torch.equal(pert["O"][b, same].view(torch.int16), base["O"][b, same].view(torch.int16))
            assert torch.equal(pert["LSE"][b, same].view(torch.int32), base["LSE"][b, same].view(torch.int32))
            assert not torch.equal(pert["O"][b, moved[b]], base["O"][b, moved[b]])


@pytest.mark.parametrize("layer", [0, 15, 31])
def test_large_batch_stack_layers(layer):
    log("case: workload 5 layer %d" % layer)
    wl = make_workload(5, layer=layer)
    g = run_gpu(wl)
    r = run_oracle(wl)
    compare(wl, g, r, "workload5-layer%d" % layer)


SMALL = [
    # (label, shape kwargs, nq, case kwargs)
    ("mha-ragged", dict(B=2, N=300, d_model=256, H=4, Hkv=4, dh=128), 13, dict()),
    ("gqa-dups-mask", dict(B=2, N=333, d_model=192, H=8, Hkv=2, dh=128), 21,
     dict(n_extra_rows=6, dup_frac=0.25, masked_vis=True)),
    ("gqa-dups-nomask", dict(B=3, N=129, d_model=128, H=6, Hkv=3, dh=128), 9,
     dict(n_extra_rows=4, dup_frac=0.4)),
    ("many-rows", dict(B=1, N=257, d_model=256, H=16, Hkv=2, dh=128), 20, dict(masked_vis=True)),
    ("single-row", dict(B=2, N=70, d_model=128, H=2, Hkv=1, dh=128), 1, dict()),
    ("large-mask-ragged", dict(B=2, N=700, d_model=256, H=4, Hkv=4, dh=128), 150,
     dict(n_extra_rows=10, dup_frac=0.05, masked_vis=True)),
    ("large-mask-aligned", dict(B=1, N=500, d_model=256, H=2, Hkv=2, dh=128), 208,
     dict(n_extra_rows=16, dup_frac=0.05, masked_vis=True)),
    # more (sequence, kv head) workgroups than CUs with up to 64 rows per kv
    # head: the 32-key, 64 KB-ring layout that puts two workgroups on a CU
    ("many-workgroups", dict(B=40, N=200, d_model=128, H=16, Hkv=8, dh=128), 13,
     dict(n_extra_rows=3, dup_frac=0.2, masked_vis=True)),
    # more than 288 query rows per kv head (48 rows x 8 heads): the MFMA
    # projection with the scalar attention kernel
    ("gqa8-rows-past-mfma-attention", dict(B=2, N=260, d_model=256, H=16, Hkv=2, dh=128), 48,
     dict(n_extra_rows=6, dup_frac=0.1, masked_vis=True)),
    ("fp32-generic", dict(B=2, N=50, d_model=64, H=4, Hkv=2, dh=32, dtype=torch.float32), 7,
     dict(n_extra_rows=2, dup_frac=0.3, masked_vis=True)),
    ("fp32-dh64", dict(B=1, N=90, d_model=96, H=2, Hkv=2, dh=64, dtype=torch.float32), 5, dict()),
    # a 64-wide head in bf16: the scalar kernels (the MFMA ones take 128)
    ("bf16-dh64", dict(B=2, N=120, d_model=128, H=4, Hkv=2, dh=64), 9,
     dict(n_extra_rows=3, dup_frac=0.2, masked_vis=True)),
    # head widths that are not a multiple of 16 or reach the scalar kernels'
    # limit: lanes past dh run on a clamped dim and are never stored
    ("fp32-dh24", dict(B=1, N=70, d_model=64, H=2, Hkv=1, dh=24, dtype=torch.float32), 6,
     dict(n_extra_rows=2, dup_frac=0.2, masked_vis=True)),
    ("bf16-dh8", dict(B=1, N=40, d_model=32, H=2, Hkv=2, dh=8), 4, dict()),
    ("bf16-dh48", dict(B=2, N=100, d_model=96, H=4, Hkv=2, dh=48), 8,
     dict(n_extra_rows=2, dup_frac=0.2, masked_vis=True)),
    ("bf16-dh256", dict(B=1, N=80, d_model=256, H=2, Hkv=1, dh=256), 5, dict(n_extra_rows=1)),
]


@pytest.mark.parametrize("label,shape,nq,kw", SMALL, ids=[s[0] for s in SMALL])
def test_small_cases(label, shape, nq, kw):
    log("case: small %s" % label)
    ls = LayerShape(**shape)
    wl = make_random_case(ls, nq, seed=zlib.crc32(label.encode()) % 10000, w_std=0.05, **kw)
    g = run_gpu(wl)
    if label.startswith("gqa8-rows-past"):
        assert g["plan"]["kernel_family"] == 1     # the projection stays on MFMA
    if label == "bf16-dh64":
        assert g["plan"]["kernel_family"] == 2
    r = run_oracle(wl)
    compare(wl, g, r, label)


@pytest.mark.parametrize("splits", [1, 2, 3, 8])
@pytest.mark.parametrize("nq", [11, 40])
def test_forced_splits(splits, nq):
    log("case: splits %d nq %d" % (splits, nq))
    ls = LayerShape(B=2, N=1000, d_model=384, H=4, Hkv=2, dh=128)
    wl = make_random_case(ls, nq, seed=77, n_extra_rows=3, dup_frac=0.2, masked_vis=True, w_std=0.05)
    g = run_gpu(wl, tuning={"attn_splits": splits})
    assert g["plan"]["attn_splits"] == splits and g["plan"]["gemm_splitk"] == 1
    r = run_oracle(wl)
    compare(wl, g, r, "splits%d-nq%d" % (splits, nq))


@pytest.mark.parametrize("choice", list(range(1, 12)))
def test_forced_projection_tiles(choice):
    """Every projection tile configuration (tuning proj_tile) on a case with
    ragged row tiles, GQA, duplicates and a mask."""
    log("case: projection tile %d" % choice)
    ls = LayerShape(B=3, N=400, d_model=512, H=4, Hkv=2, dh=128)
    wl = make_random_case(ls, 70, seed=31, n_extra_rows=8, dup_frac=0.1, masked_vis=True, w_std=0.05)
    g = run_gpu(wl, tuning={"proj_tile": choice})
    compare(wl, g, run_oracle(wl), "proj-tile%d" % choice)


def test_generic_family_on_bf16():
    log("case: generic family bf16")
    ls = LayerShape(B=2, N=200, d_model=256, H=4, Hkv=2, dh=128)
    wl = make_random_case(ls, 10, seed=5, n_extra_rows=3, dup_frac=0.3, masked_vis=True, w_std=0.05)
    g = run_gpu(wl, tuning={"kernel_family": 2})
    assert g["plan"]["kernel_family"] == 2
    r = run_oracle(wl)
    compare(wl, g, r, "generic-bf16")


def test_q_max_larger_than_nq_and_edge_positions():
    log("case: edge positions")
    ls = LayerShape(B=2, N=160, d_model=128, H=2, Hkv=2, dh=128)
    wl = make_random_case(ls, 4, seed=6, positions=[[0, 159, 1, 158], [159, 0, 80, 81]], w_std=0.05)
    g = run_gpu(wl, q_max=40)
    r = run_oracle(wl)
    compare(wl, g, r, "edges")


def test_determinism_bit_identical_reruns():
    log("case: determinism")
    wl = make_workload(3)
    g = run_gpu(wl, repeat=3)
    (O1, L1, K1, V1), (O2, L2, K2, V2) = g["runs"][1], g["runs"][2]
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))
    assert torch.equal(L1.view(torch.int32), L2.view(torch.int32))
    assert torch.equal(K1.view(torch.int16), K2.view(torch.int16))
    assert torch.equal(V1.view(torch.int16), V2.view(torch.int16))


def test_views_mutually_invisible_on_gpu():
    """Perturbing the draft view's hidden states leaves the [MASK] view's O
    and LSE bit-identical (and the other way round)."""
    log("case: view invisibility")
    wl = make_workload(3)
    groups = wl.meta["groups"]
    base = run_gpu(wl)
    for view, other, delta in (("draft", "mask", 3.0), ("mask", "draft", -2.0)):
        X2 = wl.X.clone()
        for b in range(wl.shape.B):
            rows = [int(wl.Q_idx[b, i]) for i, t in enumerate(groups[b]) if t == view]
            X2[b, rows] = (X2[b, rows].float() + delta).to(X2.dtype)
        pert = run_gpu(wl, X=X2)
        for b in range(wl.shape.B):
            idx = [i for i, t in enumerate(groups[b]) if t == other]
            assert torch.equal(pert["O"][b, idx].view(torch.int16), base["O"][b, idx].view(torch.int16))
            assert torch.equal(pert["LSE"][b, idx].view(torch.int32), base["LSE"][b, idx].view(torch.int32))
            moved = [i for i, t in enumerate(groups[b]) if t == view]
            assert not torch.equal(pert["O"][b, moved], base["O"][b, moved])


def test_empty_key_set_gives_zero_and_minus_inf():
    log("case: empty key set")
    ls = LayerShape(B=1, N=3, d_model=128, H=2, Hkv=1, dh=128)
    wl = make_random_case(ls, 3, seed=8, positions=[[2, 0, 1]], w_std=0.05)
    wl.vis = torch.zeros((1, 3, 3), dtype=torch.uint8)
    wl.vis[0, 1, 1] = 1
    g = run_gpu(wl)
    r = run_oracle(wl)
    assert torch.all(g["O"][0, [0, 2]].float() == 0)
    assert torch.all(torch.isneginf(g["LSE"][0, [0, 2]]))
    compare(wl, g, r, "empty-keys")


def test_prefill_matches_oracle():
    """Cache build from the full sequence: within 2e-2 (fp32: 1e-4) of the
    oracle's max, and on bf16 layers every element within one bf16 unit of
    the exact value (full-significand inputs, d_model 4096 included)."""
    import oracle
    from parity_util import check_faithful, rel_err, run_prefill, shape_of, round_mode, store_error_floor
    log("case: prefill")
    for ls in (LayerShape(B=1, N=64, d_model=128, H=4, Hkv=4, dh=32, dtype=torch.float32),
               LayerShape(B=2, N=200, d_model=256, H=4, Hkv=2, dh=128),
               LayerShape(B=1, N=300, d_model=4096, H=8, Hkv=2, dh=128)):
        wl = make_random_case(ls, 1, seed=9, w_std=0.05 if ls.d_model < 4096 else 0.02)
        assert not wl.meta["grid"]
        Kg, Vg = run_prefill(wl)
        Kr, Vr = oracle.prefill(shape_of(ls), wl.X_pre, wl.W, round_mode(ls.dtype))
        tol = 1e-4 if ls.dtype == torch.float32 else 2e-2
        assert rel_err(Kg.double().numpy(), Kr) <= tol
        assert rel_err(Vg.double().numpy(), Vr) <= tol
        if ls.dtype == torch.bfloat16:
            Kx, Vx = oracle.prefill(shape_of(ls), wl.X_pre, wl.W, oracle.ROUND_EXACT)
            # [B, Hkv, N, dh] -> [B, N, Hkv, dh] to match the row-wise bounds
            fk, fv = store_error_floor(ls, wl.W, wl.X_pre.double().numpy(), Kx.transpose(0, 2, 1, 3))
            n_k, o_k = check_faithful(Kg.double().numpy().transpose(0, 2, 1, 3), Kx.transpose(0, 2, 1, 3),
                                      Kr.transpose(0, 2, 1, 3), fk, ls.dtype, "prefill", "k")
            n_v, o_v = check_faithful(Vg.double().numpy().transpose(0, 2, 1, 3), Vx.transpose(0, 2, 1, 3),
                                      Vr.transpose(0, 2, 1, 3), fv, ls.dtype, "prefill", "v")
            log("prefill %s: %d of %d elements not the nearest-even rounding" % (ls, o_k + o_v, n_k + n_v))
            assert o_k + o_v <= 0.01 * (n_k + n_v)


def test_status_codes_on_gpu():
    from io_aware_kv_amd.binding import FdllmError, FusedKVCache
    log("case: status codes")
    import os
    ls = LayerShape(B=1, N=64, d_model=128, H=2, Hkv=2, dh=128)
    wl = make_random_case(ls, 4, seed=10)
    dev = "cuda"
    W = wl.W.to(dev)
    X = wl.X.to(dev)
    Kc = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device=dev)
    Vc = torch.zeros_like(Kc)
    fk = FusedKVCache(1, 64, 128, 2, 2, 128, 4)
    O = torch.empty((1, 5, 2, 128), dtype=torch.bfloat16, device=dev)
    LSE = torch.empty((1, 5, 2), dtype=torch.float32, device=dev)
    Q5 = torch.zeros((1, 5), dtype=torch.int32, device=dev)
    with pytest.raises(FdllmError) as e:
        fk.step(X, Q5, Q5, None, W, Kc, Vc, O, LSE)
    assert e.value.status == -2
    fk.close()
    bad = torch.tensor([[0, 1, 2, 64]], dtype=torch.int32, device=dev)
    O4 = torch.empty((1, 4, 2, 128), dtype=torch.bfloat16, device=dev)
    L4 = torch.empty((1, 4, 2), dtype=torch.float32, device=dev)
    # range checks belong to handles created while FDLLM_VALIDATE=1 is set
    os.environ["FDLLM_VALIDATE"] = "1"
    try:
        fkv = FusedKVCache(1, 64, 128, 2, 2, 128, 4)
    finally:
        del os.environ["FDLLM_VALIDATE"]
    with pytest.raises(FdllmError) as e:
        fkv.step(X, bad - 1, bad, None, W, Kc, Vc, O4, L4)
    assert e.value.status == -4
    fkv.close()
