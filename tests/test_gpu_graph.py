"""The fused step captured into a HIP graph (torch's graph capture on the
launch stream) replays to the eager result bit for bit: three replays, with
eager work and synchronisations between them, for the handle's step and for
the allocation-free step (whose workspace is a static device array, so the
captured step allocates nothing).  The library issues no memset, so the graph
holds kernel nodes only."""
import pytest
import torch

from io_aware_kv_amd import binding
from io_aware_kv_amd.binding import FusedKVCache
from io_aware_kv_amd.workloads import LayerShape, initial_cache, make_random_case
from parity_util import log

pytestmark = pytest.mark.gpu


def _inputs(wl, dev):
    ls = wl.shape
    K0, V0 = initial_cache(wl)
    return dict(X=wl.X.to(dev), W=wl.W.to(dev), Q=wl.Q_idx.to(dev), P=wl.pos_ids.to(dev),
                vis=wl.vis.to(dev) if wl.vis is not None else None,
                K=K0.to(dev).contiguous(), V=V0.to(dev).contiguous(),
                O=torch.empty((ls.B, wl.nq, ls.H, ls.dh), dtype=ls.dtype, device=dev),
                L=torch.empty((ls.B, wl.nq, ls.H), dtype=torch.float32, device=dev))


@pytest.mark.parametrize("noalloc", [False, True])
def test_step_replays_from_a_graph(noalloc):
    log("case: graph replay, %s step" % ("allocation-free" if noalloc else "handle"))
    dev = torch.device("cuda")
    ls = LayerShape(B=2, N=512, d_model=512, H=8, Hkv=2, dh=128)
    wl = make_random_case(ls, 24, seed=77, n_extra_rows=4, dup_frac=0.1, masked_vis=True, w_std=0.05)
    fk = None if noalloc else FusedKVCache(ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, wl.nq, ls.dtype,
                                           ls.rope_base)

    def step(t, stream=None):
        if noalloc:
            binding.fused_step_noalloc(t["X"], t["Q"], t["P"], t["vis"], t["W"], t["K"], t["V"], t["O"], t["L"],
                                       ls.H, ls.Hkv, ls.rope_base, q_max=wl.nq, stream=stream)
        else:
            fk.step(t["X"], t["Q"], t["P"], t["vis"], t["W"], t["K"], t["V"], t["O"], t["L"], stream=stream)

    # eager reference (the step is idempotent: it rewrites the same rows)
    ref = _inputs(wl, dev)
    step(ref)
    step(ref)
    torch.cuda.synchronize()
    other = _inputs(wl, dev)                  # eager work between the replays

    t = _inputs(wl, dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(t, stream=s)                     # first calls outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(t, stream=s)
    torch.cuda.synchronize()
    for rep in range(3):
        t["O"].fill_(float("nan"))
        t["L"].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ("O", "L", "K", "V"):
            assert torch.equal(t[k].view(torch.int16 if t[k].dtype == torch.bfloat16 else torch.int32),
                               ref[k].view(torch.int16 if ref[k].dtype == torch.bfloat16 else torch.int32)), \
                "replay %d: %s differs from the eager step" % (rep, k)
        step(other)
        other["O"].add_(1.0)
        torch.cuda.synchronize()
    if fk is not None:
        fk.close()
