"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare.

Pass criteria (relative to the oracle's output magnitude):
  - cache rows at positions the step does not write: bit-exact;
  - written k/v rows and O: max|gpu - oracle| / max|oracle| <= 2e-2 (bf16) or
    1e-4 (fp32);
  - LSE: <= 1e-3 absolute (finite entries; -inf must match exactly).
"""
import sys

import numpy as np
import torch

import oracle
from io_aware_kv_amd.binding import FusedKVCache

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
LSE_TOL = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def shape_of(ls):
    return oracle.Shape(ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, ls.rope_base)


def round_mode(dtype):
    return oracle.ROUND_BF16 if dtype == torch.bfloat16 else oracle.ROUND_FP32


def run_gpu(wl, tuning=None, q_max=None, repeat=1, X=None):
    """Prefill the cache from X_pre on the GPU, run the fused step.  Returns a
    dict of host tensors: pre-step caches, post-step caches, O, LSE."""
    ls = wl.shape
    dev = torch.device("cuda")
    Xp = wl.X_pre.to(dev)
    Xs = (wl.X if X is None else X).to(dev)
    W = wl.W.to(dev)
    Kc = torch.empty((ls.B, ls.Hkv, ls.N, ls.dh), dtype=ls.dtype, device=dev)
    Vc = torch.empty_like(Kc)
    fk = FusedKVCache(ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, q_max or max(1, wl.nq), ls.dtype,
                      ls.rope_base, X_full=Xp, W=W, Kc=Kc, Vc=Vc)
    if tuning:
        fk.set_tuning(**tuning)
    torch.cuda.synchronize()
    K0, V0 = Kc.cpu(), Vc.cpu()
    Q = wl.Q_idx.to(dev)
    P = wl.pos_ids.to(dev)
    vis = wl.vis.to(dev) if wl.vis is not None else None
    outs = []
    for _ in range(repeat):
        O = torch.full((ls.B, wl.nq, ls.H, ls.dh), float("nan"), dtype=ls.dtype, device=dev)
        LSE = torch.full((ls.B, wl.nq, ls.H), float("nan"), dtype=torch.float32, device=dev)
        fk.step(Xs, Q, P, vis, W, Kc, Vc, O, LSE)
        torch.cuda.synchronize()
        outs.append((O.cpu(), LSE.cpu(), Kc.cpu(), Vc.cpu()))
    plan = fk.plan(wl.nq)
    fk.close()
    O, LSE, K1, V1 = outs[-1]
    return {"K0": K0, "V0": V0, "K1": K1, "V1": V1, "O": O, "LSE": LSE, "runs": outs, "plan": plan}


def run_oracle(wl, K0, V0, X=None):
    ls = wl.shape
    return oracle.step(shape_of(ls), wl.X if X is None else X, wl.Q_idx, wl.pos_ids, wl.vis, wl.W,
                       K0, V0, round_mode(ls.dtype))


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.abs(ref).max()
    if denom == 0:
        return float(np.abs(got - ref).max()) if got.size else 0.0
    return float(np.abs(got - ref).max() / denom)


def compare(wl, g, r, label=""):
    """Assert the pass criteria; return a dict of the measured errors."""
    ls = wl.shape
    tol = TOL[ls.dtype]
    P = wl.pos_ids.numpy()
    written = np.zeros((ls.B, ls.N), dtype=bool)
    for b in range(ls.B):
        written[b, P[b]] = True
    K0, V0 = g["K0"], g["V0"]
    K1, V1 = g["K1"], g["V1"]
    # untouched rows: bit-exact (compare raw bits through an integer view)
    keep = torch.from_numpy(~written)[:, None, :].expand(ls.B, ls.Hkv, ls.N)
    ib = torch.int16 if ls.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(K1.view(ib)[keep], K0.view(ib)[keep]), label + ": untouched K rows changed"
    assert torch.equal(V1.view(ib)[keep], V0.view(ib)[keep]), label + ": untouched V rows changed"
    # written rows vs the oracle's rows (first occurrence owns the position)
    wmask = torch.from_numpy(written)[:, None, :].expand(ls.B, ls.Hkv, ls.N).numpy()
    k_err = rel_err(K1.double().numpy()[wmask], r["Kc"][wmask])
    v_err = rel_err(V1.double().numpy()[wmask], r["Vc"][wmask])
    o_err = rel_err(g["O"].double().numpy(), r["O"])
    lg, lr = g["LSE"].double().numpy(), r["LSE"]
    assert np.array_equal(np.isneginf(lg), np.isneginf(lr)), label + ": empty key sets differ"
    fin = np.isfinite(lr)
    lse_err = float(np.abs(lg[fin] - lr[fin]).max()) if fin.any() else 0.0
    errs = {"k": k_err, "v": v_err, "O": o_err, "LSE": lse_err}
    log("%s errors %s plan %s" % (label, {k: "%.2e" % v for k, v in errs.items()}, g.get("plan")))
    assert np.isfinite(g["O"].double().numpy()).all(), label + ": non-finite O"
    assert k_err <= tol and v_err <= tol, label + ": written k/v off %s" % errs
    assert o_err <= tol, label + ": O off %s" % errs
    assert lse_err <= LSE_TOL, label + ": LSE off %s" % errs
    return errs
