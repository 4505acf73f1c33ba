"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the fp64 oracle on the same seeded inputs, and compare.

Pass criteria:
  - cache rows at positions the step does not write: bit-exact;
  - written k/v rows and O: max|gpu - oracle| / max|oracle| <= 2e-2 (bf16) or
    1e-4 (fp32);
  - LSE: <= 1e-3 absolute (finite entries; -inf must match exactly);
  - bf16 storage, element by element:
      * inputs with the full bf16 significand (the default): every written
        k and v element lies within one storage unit of the oracle's exact
        (unrounded, fp64) value, i.e. it is one of the two bf16 values that
        bracket it, and at most STORE_MISMATCH_MAX of them differ from the
        oracle's nearest-even rounding (the fp32 accumulation error, ~1e-5
        of a value, moves a rounding only where the exact value lies that
        close to a midpoint between two bf16 values: a fraction of a per
        cent);
      * inputs on the dyadic grid (grid=True; the projection is exact in
        fp32 in any order): every written v element is the oracle's rounding
        bit for bit, and so is every written k element except at a rounding
        tie of the rotation (rounding_ties), where it may be the other
        neighbour.  The LSE shift those ties could cause
        (lse_rounding_slack) is logged as a diagnostic only.

Both sides start from the same seeded cache (initial_cache), generated on the
host; no input of the oracle comes from the GPU.
"""
import sys

import numpy as np
import torch

import oracle
from io_aware_kv_amd.binding import FusedKVCache
from io_aware_kv_amd.workloads import initial_cache

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
    """Load the seeded initial cache onto the GPU and run the fused step.
    Returns a dict of host tensors: pre-step caches, post-step caches, O, LSE."""
    ls = wl.shape
    dev = torch.device("cuda")
    Xs = (wl.X if X is None else X).to(dev)
    W = wl.W.to(dev)
    K0, V0 = initial_cache(wl)
    Kc = K0.to(dev).contiguous()
    Vc = V0.to(dev).contiguous()
    fk = FusedKVCache(ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, q_max or max(1, wl.nq), ls.dtype,
                      ls.rope_base)
    if tuning:
        fk.set_tuning(**tuning)
    Q = wl.Q_idx.to(dev)
    P = wl.pos_ids.to(dev)
    vis = wl.vis.to(dev) if wl.vis is not None else None
    outs = []
    for _ in range(repeat):
        O = torch.full((ls.B, wl.nq, ls.H, ls.dh), float("nan"), dtype=ls.dtype, device=dev)
        LSE = torch.full((ls.B, wl.nq, ls.H), float("nan"), dtype=torch.float32, device=dev)
        if repeat > 1:
            Kc.copy_(K0)
            Vc.copy_(V0)
        fk.step(Xs, Q, P, vis, W, Kc, Vc, O, LSE)
        torch.cuda.synchronize()
        outs.append((O.cpu(), LSE.cpu(), Kc.cpu(), Vc.cpu()))
    plan = fk.plan(wl.nq)
    fk.close()
    O, LSE, K1, V1 = outs[-1]
    return {"K0": K0, "V0": V0, "K1": K1, "V1": V1, "O": O, "LSE": LSE, "runs": outs, "plan": plan}


def run_prefill(wl):
    """Build the cache from X_pre with the library's prefill (fdllm_cache_init
    with the full sequence).  Returns host Kc, Vc."""
    ls = wl.shape
    dev = torch.device("cuda")
    Xp = wl.X_pre.to(dev)
    W = wl.W.to(dev)
    Kc = torch.empty((ls.B, ls.Hkv, ls.N, ls.dh), dtype=ls.dtype, device=dev)
    Vc = torch.empty_like(Kc)
    fk = FusedKVCache(ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, 1, ls.dtype, ls.rope_base,
                      X_full=Xp, W=W, Kc=Kc, Vc=Vc)
    torch.cuda.synchronize()
    fk.close()
    return Kc.cpu(), Vc.cpu()


def run_oracle(wl, X=None):
    """The oracle's step on the workload's own inputs (seeded initial cache),
    plus the unrounded k and v rows of the query set (element-wise checks of
    the stored rows)."""
    ls = wl.shape
    K0, V0 = initial_cache(wl)
    Xs = wl.X if X is None else X
    r = oracle.step(shape_of(ls), Xs, wl.Q_idx, wl.pos_ids, wl.vis, wl.W, K0, V0, round_mode(ls.dtype))
    _, r["k_exact"], r["v_exact"] = oracle.project(shape_of(ls), Xs, wl.Q_idx, wl.pos_ids, wl.W,
                                                    oracle.ROUND_EXACT)
    return r


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    denom = np.abs(ref).max()
    if denom == 0:
        return float(np.abs(got - ref).max()) if got.size else 0.0
    return float(np.abs(got - ref).max() / denom)


MANTISSA_BITS = {torch.bfloat16: 7, torch.float32: 23}
U32 = 2.0 ** -24     # unit roundoff of fp32


def storage_unit(x, dtype):
    """Spacing of the storage type's values in the binade of |x| (0 at 0)."""
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - MANTISSA_BITS[dtype]), 0.0)


def k_rounding_range(k_exact, dtype):
    """(lo, hi): the storage-type values an fp32 evaluation of the stored k
    elements can round to.  With the seeded inputs on their dyadic grid the
    projection is exact in fp32, so the only fp32 error in a stored k element
    is the rotation's: c and s are fp32 roundings of the cosine and sine, and
    a*c - b*s takes at most three more roundings, so |k_fp32 - k| <=
    4u(|a| + |b|) <= 4 sqrt(2) u |(a, b)| = 4 sqrt(2) u |(k_i, k_{i+dh/2})|
    (the rotation keeps the pair's norm).  Every value in [k - bound,
    k + bound] rounds into [round(k - bound), round(k + bound)]."""
    kx = np.asarray(k_exact, dtype=np.float64)
    half = kx.shape[-1] // 2
    pn = np.sqrt(kx[..., :half] ** 2 + kx[..., half:] ** 2)
    bound = 4.0 * np.sqrt(2.0) * U32 * np.concatenate([pn, pn], axis=-1) * (1 + 1e-6)
    mode = round_mode(dtype)
    return oracle.round_store(kx - bound, mode), oracle.round_store(kx + bound, mode)


def rounding_ties(k_exact, dtype):
    """Boolean mask of exact k elements whose rounding to the storage type the
    fp32 arithmetic does not decide (k_rounding_range holds two values)."""
    lo, hi = k_rounding_range(k_exact, dtype)
    return lo != hi


def lse_rounding_slack(wl, r):
    """[B, nq, H] bound on how far LSE can move when the stored k elements of
    the step's rows whose rounding is a tie take another value of their
    range: sum over visible step rows j of p_ij * scale * sum_e |q_e| *
    (hi - lo)_je, from the oracle's own values (10% added for the
    second-order term)."""
    ls = wl.shape
    B, nq, H, Hkv, dh = ls.B, wl.nq, ls.H, ls.Hkv, ls.dh
    if nq == 0:
        return np.zeros((B, 0, H))
    lo, hi = k_rounding_range(r["k_exact"], ls.dtype)
    du = hi - lo                                                  # [B, nq, Hkv, dh]
    if not du.any():
        return np.zeros((B, nq, H))
    grp = (np.arange(H) * Hkv) // H
    q = np.asarray(r["q"], dtype=np.float64)                      # [B, nq, H, dh]
    k = np.asarray(r["k"], dtype=np.float64)                      # [B, nq, Hkv, dh]
    scale = 1.0 / np.sqrt(dh)
    qh = np.ascontiguousarray(q.transpose(0, 2, 1, 3))            # [B, H, nq, dh]
    kh = np.ascontiguousarray(k[:, :, grp, :].transpose(0, 2, 3, 1))    # [B, H, dh, nq]
    duh = np.ascontiguousarray(du[:, :, grp, :].transpose(0, 2, 3, 1))
    s = (qh @ kh) * scale                                          # [B, H, i, j]
    shift = (np.abs(qh) @ duh) * scale
    lse = np.asarray(r["LSE"], dtype=np.float64).transpose(0, 2, 1)[..., None]
    with np.errstate(invalid="ignore", over="ignore"):
        p = np.where(np.isfinite(lse), np.exp(s - lse), 0.0)
    if wl.vis is not None:
        p = p * wl.vis.numpy()[:, None, :, :]
    return 1.1 * (p * shift).sum(axis=-1).transpose(0, 2, 1)       # [B, nq, H]


def owner_rows(wl):
    """(b, j, position) of the rows that own a cache write (first occurrence)."""
    P = wl.pos_ids.numpy()
    bb, jj, pp = [], [], []
    for b in range(wl.shape.B):
        seen = set()
        for j in range(wl.nq):
            p = int(P[b, j])
            if p not in seen:
                seen.add(p)
                bb.append(b); jj.append(j); pp.append(p)
    return np.array(bb, dtype=np.int64), np.array(jj, dtype=np.int64), np.array(pp, dtype=np.int64)


def check_written_rows_bits(wl, g, r, label):
    """bf16 storage: every written v element equals the oracle's rounding and
    every written k element lies in its k_rounding_range (a single value, the
    oracle's rounding, except at ties).  Returns the count of tie elements
    and of those where the GPU's value is not the oracle's."""
    bb, jj, pp = owner_rows(wl)
    if bb.size == 0:
        return 0, 0
    tb, tp = torch.from_numpy(bb), torch.from_numpy(pp)
    gk = g["K1"][tb, :, tp, :].double().numpy()                   # [n, Hkv, dh]
    gv = g["V1"][tb, :, tp, :].double().numpy()
    ok = np.asarray(r["k"])[bb, jj]
    ov = np.asarray(r["v"])[bb, jj]
    nv = int((gv != ov).sum())
    assert nv == 0, "%s: %d written v elements differ from the oracle's rounding" % (label, nv)
    lo, hi = k_rounding_range(np.asarray(r["k_exact"])[bb, jj], wl.shape.dtype)
    assert np.all((lo <= ok) & (ok <= hi))
    out = (gk < lo) | (gk > hi)
    assert not out.any(), "%s: %d written k elements outside their rounding range" % (label, int(out.sum()))
    return int((lo != hi).sum()), int((gk != ok).sum())


STORE_MISMATCH_MAX = 0.01
LAMBDA = 7.0         # probabilistic rounding-error bound: exceeded with probability < 2 exp(-LAMBDA^2 / 2)


def store_error_floor(ls, W, Xrows, k_exact):
    """Absolute bounds [B, n, Hkv, dh] on the fp32 evaluation error of the
    stored k and v elements (before their rounding to the storage type) of
    the rows Xrows [B, n, d_model], for full-significand inputs.  An inner
    product of n terms summed in fp32 in any order is off by at most
    LAMBDA * sqrt(n) * u * sum |x_i w_i| except with probability below
    2 exp(-LAMBDA^2 / 2) (the probabilistic bound of Higham and Mary, 2019);
    bf16 x bf16 products are exact in fp32.  The rotation of a pair (a, b) by
    fp32 (c, s) scales those errors by at most |c| + |s| <= sqrt(2) and adds
    at most 4 sqrt(2) u |(a, b)| (see k_rounding_range).
    Returns (floor_k, floor_v)."""
    H, Hkv, dh, d = ls.H, ls.Hkv, ls.dh, ls.d_model
    Wa = W.double().abs().numpy()
    Wk = Wa[H * dh:(H + Hkv) * dh]
    Wv = Wa[(H + Hkv) * dh:(H + 2 * Hkv) * dh]
    Xa = np.abs(np.asarray(Xrows, dtype=np.float64))
    B, n = Xa.shape[0], Xa.shape[1]
    c = LAMBDA * np.sqrt(d) * U32
    half = dh // 2
    fk = np.empty((B, n, Hkv, dh))
    fv = np.empty((B, n, Hkv, dh))
    for b in range(B):
        sk = (Xa[b] @ Wk.T).reshape(n, Hkv, dh)
        sv = (Xa[b] @ Wv.T).reshape(n, Hkv, dh)
        pair_max = np.maximum(sk[..., :half], sk[..., half:])
        fk[b] = np.sqrt(2.0) * c * np.concatenate([pair_max, pair_max], axis=-1)
        fv[b] = c * sv
    kx = np.asarray(k_exact, dtype=np.float64)
    pn = np.sqrt(kx[..., :half] ** 2 + kx[..., half:] ** 2)
    fk += 4.0 * np.sqrt(2.0) * U32 * np.concatenate([pn, pn], axis=-1)
    return fk, fv


def check_faithful(got, exact, rounded, floor, dtype, label, name):
    """Element-wise: |got - exact| <= storage unit of exact + floor.  Returns
    the number of elements and how many differ from the nearest-even
    rounding `rounded`."""
    got = np.asarray(got, dtype=np.float64)
    ex = np.asarray(exact, dtype=np.float64)
    far = np.abs(got - ex) > storage_unit(ex, dtype) + floor
    assert not far.any(), "%s: %d %s elements more than one storage unit from the exact value" % (
        label, int(far.sum()), name)
    return got.size, int((got != np.asarray(rounded)).sum())


def check_written_rows_faithful(wl, g, r, label):
    """bf16 storage on full-significand inputs: every written k and v element
    lies within one storage unit (the bf16 spacing in the binade of the exact
    value) plus the fp32 evaluation bound (store_error_floor, which matters
    only for elements near zero) of the oracle's unrounded fp64 value; and at
    most STORE_MISMATCH_MAX of them differ from the oracle's nearest-even
    rounding.  A dropped or truncated low operand bit, a lower-precision
    operand path or a wrong rounding mode moves elements by a unit or more,
    or moves far more than a per cent of them off the nearest-even rounding.
    Returns (elements checked, elements that differ from the oracle's
    nearest-even rounding)."""
    bb, jj, pp = owner_rows(wl)
    if bb.size == 0:
        return 0, 0
    tb, tp = torch.from_numpy(bb), torch.from_numpy(pp)
    Xrows = torch.stack([wl.X[b, wl.Q_idx[b].long()] for b in range(wl.shape.B)]).double().numpy()
    floor_k, floor_v = store_error_floor(wl.shape, wl.W, Xrows, r["k_exact"])
    n_el, n_other = 0, 0
    for name, cache, exact, rounded, floor in (("k", "K1", "k_exact", "k", floor_k),
                                               ("v", "V1", "v_exact", "v", floor_v)):
        got = g[cache][tb, :, tp, :].double().numpy()                 # [n, Hkv, dh]
        ne, no = check_faithful(got, np.asarray(r[exact])[bb, jj], np.asarray(r[rounded])[bb, jj],
                                floor[bb, jj], wl.shape.dtype, label, "written " + name)
        n_el += ne
        n_other += no
    assert n_other <= STORE_MISMATCH_MAX * n_el, "%s: %d of %d written elements are not the nearest-even " \
        "rounding of the exact value" % (label, n_other, n_el)
    return n_el, n_other


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
    if ls.dtype == torch.bfloat16:
        if wl.meta.get("grid", False):
            n_ties, n_other = check_written_rows_bits(wl, g, r, label)
            errs["k_ties"], errs["k_other_neighbour"] = n_ties, n_other
            slack = lse_rounding_slack(wl, r)
            errs["LSE_tie_slack"] = float(slack[fin].max()) if fin.any() else 0.0
        else:
            n_el, n_other = check_written_rows_faithful(wl, g, r, label)
            errs["kv_elements"], errs["kv_not_nearest"] = n_el, n_other
    log("%s errors %s plan %s" % (label, {k: ("%.2e" % v if isinstance(v, float) else v)
                                          for k, v in errs.items()}, g.get("plan")))
    assert np.isfinite(g["O"].double().numpy()).all(), label + ": non-finite O"
    assert k_err <= tol and v_err <= tol, label + ": written k/v off %s" % errs
    assert o_err <= tol, label + ": O off %s" % errs
    assert lse_err <= LSE_TOL, label + ": LSE off %s" % errs
    return errs
