"""GPU parity of the fused step over a paged cache with per-sequence valid
lengths and query counts (fdllm_fused_step_paged), against the oracle's
definition (oracle.step_paged) and against the flat step.

Bar: as for the flat step (written k/v and O within 2e-2 / 1e-4 relative of
the oracle's magnitude, LSE within 1e-3 absolute); padding rows exactly
0 / -inf; pool rows the step does not write bit-exact.  With full lengths and row counts the
paged step must reproduce the flat step bit for bit (the kernels visit the
same keys in the same order; only the addresses differ).
"""
import numpy as np
import pytest
import torch

import oracle
from io_aware_kv_amd.binding import FusedKVCache
from io_aware_kv_amd.workloads import LayerShape, initial_cache, make_random_case, make_workload, paged_layout
from parity_util import TOL, log, rel_err, round_mode, run_gpu, shape_of

pytestmark = pytest.mark.gpu


def run_paged(wl, table, Kpool, Vpool, seq_len, nq_seq, block_size, paged=True):
    ls = wl.shape
    dev = torch.device("cuda")
    fk = FusedKVCache(ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, max(1, wl.nq), ls.dtype, ls.rope_base)
    Kp, Vp = Kpool.to(dev).contiguous(), Vpool.to(dev).contiguous()
    O = torch.full((ls.B, wl.nq, ls.H, ls.dh), float("nan"), dtype=ls.dtype, device=dev)
    LSE = torch.full((ls.B, wl.nq, ls.H), float("nan"), dtype=torch.float32, device=dev)
    vis = wl.vis.to(dev) if wl.vis is not None else None
    fk.step_paged(wl.X.to(dev), wl.Q_idx.to(dev), wl.pos_ids.to(dev), vis, wl.W.to(dev), Kp, Vp, O, LSE,
                  block_table=table.to(dev) if paged else None, block_size=block_size,
                  num_blocks=Kpool.shape[0] if paged else 0,
                  seq_len=seq_len.to(dev) if seq_len is not None else None,
                  nq_seq=nq_seq.to(dev) if nq_seq is not None else None)
    torch.cuda.synchronize()
    fk.close()
    return O.cpu(), LSE.cpu(), Kp.cpu(), Vp.cpu()


def check_against_oracle(wl, table, Kpool, Vpool, seq_len, nq_seq, bs, label):
    ls = wl.shape
    O, LSE, Kp1, Vp1 = run_paged(wl, table, Kpool, Vpool, seq_len, nq_seq, bs)
    r = oracle.step_paged(shape_of(ls), wl.X, wl.Q_idx, wl.pos_ids, nq_seq, wl.vis, wl.W, Kpool, Vpool, table, bs,
                          seq_len, round_mode(ls.dtype))
    tol = TOL[ls.dtype]
    nb = nq_seq.numpy()
    live = np.zeros((ls.B, wl.nq), dtype=bool)
    for b in range(ls.B):
        live[b, :nb[b]] = True
    o, lse = O.double().numpy(), LSE.double().numpy()
    assert np.all(o[~live] == 0.0) and np.all(np.isneginf(lse[~live])), label + ": padding rows"
    o_err = rel_err(o[live], r["O"][live])
    fin = np.isfinite(r["LSE"]) & live[:, :, None]
    lse_err = float(np.abs(lse[fin] - r["LSE"][fin]).max()) if fin.any() else 0.0
    k_err = rel_err(Kp1.double().numpy(), r["Kpool"])
    v_err = rel_err(Vp1.double().numpy(), r["Vpool"])
    log("%s errors O %.2e LSE %.2e k %.2e v %.2e" % (label, o_err, lse_err, k_err, v_err))
    assert o_err <= tol and k_err <= tol and v_err <= tol
    assert lse_err <= 1e-3
    # pool rows nobody writes: bit-exact
    written = np.zeros(Kpool.shape[0] * Kpool.shape[2], dtype=bool).reshape(Kpool.shape[0], Kpool.shape[2])
    P = wl.pos_ids.numpy()
    for b in range(ls.B):
        for j in range(nb[b]):
            p = int(P[b, j])
            written[int(table[b, p // bs]), p % bs] = True
    ib = torch.int16 if ls.dtype == torch.bfloat16 else torch.int32
    keep = torch.from_numpy(~written)[:, None, :].expand(Kpool.shape[0], ls.Hkv, Kpool.shape[2])
    assert torch.equal(Kp1.view(ib)[keep], Kpool.view(ib)[keep])
    assert torch.equal(Vp1.view(ib)[keep], Vpool.view(ib)[keep])


@pytest.mark.parametrize("cid,bs", [(3, 16), (4, 64), (7, 32)])
def test_paged_full_lengths_equal_flat_step_bit_for_bit(cid, bs):
    log("case: paged = flat, workload %d block %d" % (cid, bs))
    wl = make_workload(cid)
    table, Kpool, Vpool, L, nb = paged_layout(wl, bs, ragged=False)
    O, LSE, Kp1, Vp1 = run_paged(wl, table, Kpool, Vpool, L, nb, bs)
    g = run_gpu(wl)
    assert torch.equal(O.view(torch.int16), g["O"].view(torch.int16))
    assert torch.equal(LSE.view(torch.int32), g["LSE"].view(torch.int32))
    ls = wl.shape
    for b in range(ls.B):
        for k in range(table.shape[1]):
            p0, p1 = k * bs, min(ls.N, (k + 1) * bs)
            blk = int(table[b, k])
            assert torch.equal(Kp1[blk, :, :p1 - p0].view(torch.int16), g["K1"][b, :, p0:p1].view(torch.int16))
            assert torch.equal(Vp1[blk, :, :p1 - p0].view(torch.int16), g["V1"][b, :, p0:p1].view(torch.int16))


@pytest.mark.parametrize("cid,bs", [(3, 16), (6, 128), (5, 16), (2, 256)])
def test_paged_ragged_layer_workloads(cid, bs):
    log("case: paged ragged, workload %d block %d" % (cid, bs))
    wl = make_workload(cid)
    table, Kpool, Vpool, L, nb = paged_layout(wl, bs, ragged=True)
    check_against_oracle(wl, table, Kpool, Vpool, L, nb, bs, "paged-w%d" % cid)


SMALL = [
    ("gqa-dups-mask", dict(B=3, N=333, d_model=192, H=8, Hkv=2, dh=128), 21,
     dict(n_extra_rows=6, dup_frac=0.25, masked_vis=True), 16),
    ("fp32-generic", dict(B=2, N=50, d_model=64, H=4, Hkv=2, dh=32, dtype=torch.float32), 7,
     dict(n_extra_rows=2, dup_frac=0.3, masked_vis=True), 16),
    ("many-splits", dict(B=1, N=1500, d_model=128, H=4, Hkv=1, dh=128), 9, dict(masked_vis=True), 32),
]


@pytest.mark.parametrize("label,shape,nq,kw,bs", SMALL, ids=[s[0] for s in SMALL])
def test_paged_ragged_small_cases(label, shape, nq, kw, bs):
    log("case: paged ragged small %s" % label)
    ls = LayerShape(**shape)
    wl = make_random_case(ls, nq, seed=61, w_std=0.05, **kw)
    table, Kpool, Vpool, L, nb = paged_layout(wl, bs, ragged=True)
    check_against_oracle(wl, table, Kpool, Vpool, L, nb, bs, label)


def test_ragged_flat_layout():
    """No block table: the flat layout with per-sequence lengths and rows."""
    log("case: ragged flat")
    wl = make_workload(3)
    ls = wl.shape
    K0, V0 = initial_cache(wl)
    g = torch.Generator().manual_seed(5)
    nb = torch.randint(1, wl.nq + 1, (ls.B,), generator=g).to(torch.int32)
    L = torch.tensor([max(int(wl.pos_ids[b, :int(nb[b])].max()) + 1, 700 + 100 * b) for b in range(ls.B)],
                     dtype=torch.int32)
    L = torch.clamp(L, max=ls.N)
    O, LSE, K1, V1 = run_paged(wl, None, K0, V0, L, nb, 0, paged=False)
    # the oracle's definition with a trivial table over the flat cache
    bs = 16
    nblk = ls.N // bs
    table = torch.arange(ls.B * nblk, dtype=torch.int32).reshape(ls.B, nblk)
    Kp = K0.reshape(ls.B, ls.Hkv, nblk, bs, ls.dh).permute(0, 2, 1, 3, 4).reshape(ls.B * nblk, ls.Hkv, bs, ls.dh)
    Vp = V0.reshape(ls.B, ls.Hkv, nblk, bs, ls.dh).permute(0, 2, 1, 3, 4).reshape(ls.B * nblk, ls.Hkv, bs, ls.dh)
    r = oracle.step_paged(shape_of(ls), wl.X, wl.Q_idx, wl.pos_ids, nb, wl.vis, wl.W, Kp.contiguous(),
                          Vp.contiguous(), table, bs, L, round_mode(ls.dtype))
    live = np.zeros((ls.B, wl.nq), dtype=bool)
    for b in range(ls.B):
        live[b, :int(nb[b])] = True
    o = O.double().numpy()
    assert np.all(o[~live] == 0.0) and np.all(np.isneginf(LSE.numpy()[~live]))
    assert rel_err(o[live], r["O"][live]) <= TOL[ls.dtype]
    fin = np.isfinite(r["LSE"]) & live[:, :, None]
    assert float(np.abs(LSE.double().numpy()[fin] - r["LSE"][fin]).max()) <= 1e-3
