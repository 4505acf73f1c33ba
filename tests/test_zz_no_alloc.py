"""The allocation-free fused step (fdllm_fused_step_noalloc, for callers that
cannot allocate device memory) against the handle's fused step on the same
inputs, through the C ABI: two calls in a row on one layer, the second with
fewer query rows, each within the parity bar of the handle's outputs
(untouched cache rows bit-exact, written k/v and O within 2e-2 of the max,
LSE within 1e-3), including a layer whose attention splits the cache (split
partials in the scratch array)."""
import dataclasses

import numpy as np
import pytest
import torch

from io_aware_kv_amd import binding
from io_aware_kv_amd.binding import FusedKVCache
from io_aware_kv_amd.workloads import LayerShape, initial_cache, make_random_case, make_workload
from parity_util import log, rel_err

pytestmark = pytest.mark.gpu


def _subset(wl, n):
    """The workload's first n query rows (same layer, same hidden states)."""
    return dataclasses.replace(wl, nq=n, Q_idx=wl.Q_idx[:, :n].contiguous(), pos_ids=wl.pos_ids[:, :n].contiguous(),
                               vis=None if wl.vis is None else wl.vis[:, :n, :n].contiguous())


def _run(wl, q_max, noalloc):
    ls = wl.shape
    dev = torch.device("cuda")
    K0, V0 = initial_cache(wl)
    Kc, Vc = K0.to(dev).contiguous(), V0.to(dev).contiguous()
    X, W = wl.X.to(dev), wl.W.to(dev)
    Q, P = wl.Q_idx.to(dev), wl.pos_ids.to(dev)
    vis = wl.vis.to(dev) if wl.vis is not None else None
    O = torch.full((ls.B, wl.nq, ls.H, ls.dh), float("nan"), dtype=ls.dtype, device=dev)
    LSE = torch.full((ls.B, wl.nq, ls.H), float("nan"), dtype=torch.float32, device=dev)
    if noalloc:
        binding.fused_step_noalloc(X, Q, P, vis, W, Kc, Vc, O, LSE, ls.H, ls.Hkv, ls.rope_base, q_max=q_max)
        plan = None
    else:
        fk = FusedKVCache(ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, q_max, ls.dtype, ls.rope_base)
        fk.step(X, Q, P, vis, W, Kc, Vc, O, LSE)
        plan = fk.plan(wl.nq)
        fk.close()
    torch.cuda.synchronize()
    return {"O": O.cpu(), "LSE": LSE.cpu(), "K": Kc.cpu(), "V": Vc.cpu(), "K0": K0, "V0": V0, "plan": plan}


def _compare(wl, a, b, label):
    ls = wl.shape
    P = wl.pos_ids.numpy()
    written = np.zeros((ls.B, ls.N), dtype=bool)
    for s in range(ls.B):
        written[s, P[s]] = True
    keep = torch.from_numpy(~written)[:, None, :].expand(ls.B, ls.Hkv, ls.N)
    ib = torch.int16 if ls.dtype == torch.bfloat16 else torch.int32
    for t in ("K", "V"):
        assert torch.equal(b[t].view(ib)[keep], b[t + "0"].view(ib)[keep]), label + ": untouched rows changed"
    wm = torch.from_numpy(written)[:, None, :].expand(ls.B, ls.Hkv, ls.N)
    errs = {"k": rel_err(b["K"].double()[wm].numpy(), a["K"].double()[wm].numpy()),
            "v": rel_err(b["V"].double()[wm].numpy(), a["V"].double()[wm].numpy()),
            "O": rel_err(b["O"].double().numpy(), a["O"].double().numpy())}
    la, lb = a["LSE"].double().numpy(), b["LSE"].double().numpy()
    assert np.array_equal(np.isneginf(la), np.isneginf(lb))
    fin = np.isfinite(la)
    errs["LSE"] = float(np.abs(la[fin] - lb[fin]).max()) if fin.any() else 0.0
    same = all(torch.equal(a[t].view(ib if t != "LSE" else torch.int32), b[t].view(ib if t != "LSE" else torch.int32))
               for t in ("O", "K", "V", "LSE"))
    log("%s: plan %s errors %s bit-identical %s" % (label, a["plan"], errs, same))
    tol = 2e-2 if ls.dtype == torch.bfloat16 else 1e-4
    assert errs["k"] <= tol and errs["v"] <= tol and errs["O"] <= tol and errs["LSE"] <= 1e-3, errs


def test_noalloc_matches_the_handle_step_on_two_calls():
    # the draft-pass layer (its attention splits the cache 8 ways), then the
    # same layer with its first 17 query rows
    wl = make_workload(2)
    for label, w in (("draft-pass nq=33", wl), ("draft-pass nq=17", _subset(wl, 17))):
        log("case: noalloc %s" % label)
        a = _run(w, wl.nq, noalloc=False)
        b = _run(w, wl.nq, noalloc=True)
        assert a["plan"]["attn_splits"] > 1
        _compare(w, a, b, label)


def test_noalloc_gqa_duplicates_mask_then_smaller():
    ls = LayerShape(B=3, N=700, d_model=512, H=8, Hkv=2, dh=128)
    big = make_random_case(ls, 40, seed=71, n_extra_rows=6, dup_frac=0.15, masked_vis=True, w_std=0.05)
    small = make_random_case(ls, 9, seed=72, n_extra_rows=2, dup_frac=0.2, masked_vis=True, w_std=0.05)
    for label, w in (("gqa nq=40", big), ("gqa nq=9", small)):
        log("case: noalloc %s" % label)
        a = _run(w, 40, noalloc=False)
        b = _run(w, 40, noalloc=True)
        _compare(w, a, b, label)


def test_noalloc_fp32_layer():
    wl = make_workload(1)
    log("case: noalloc tiny fp32 layer")
    a = _run(wl, wl.nq, noalloc=False)
    b = _run(wl, wl.nq, noalloc=True)
    _compare(wl, a, b, "fp32")


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    ls = LayerShape(B=64, N=4096, d_model=256, H=32, Hkv=32, dh=128)
    dev = torch.device("cuda")
    nq = 64
    X = torch.zeros((ls.B, ls.N, ls.d_model), dtype=ls.dtype, device=dev)
    W = torch.zeros((ls.cols, ls.d_model), dtype=ls.dtype, device=dev)
    Kc = torch.zeros((ls.B, ls.Hkv, ls.N, ls.dh), dtype=ls.dtype, device=dev)
    Q = torch.zeros((ls.B, nq), dtype=torch.int32, device=dev)
    O = torch.zeros((ls.B, nq, ls.H, ls.dh), dtype=ls.dtype, device=dev)
    LSE = torch.zeros((ls.B, nq, ls.H), dtype=torch.float32, device=dev)
    with pytest.raises(binding.FdllmError) as e:
        binding.fused_step_noalloc(X, Q, Q, None, W, Kc, Kc.clone(), O, LSE, ls.H, ls.Hkv)
    assert e.value.status == -8
