"""Seeded synthetic inputs for the fused KV-cache step.

This module draws random tensors and index sets only; it holds none of the
step's arithmetic (no projection, rotary, scatter or attention), so both the
HIP path and the CPU oracle can be fed from it.

The shapes follow the workloads the Flash-dLLM pages describe: a draft pass
whose query set is the tracked rows plus the front masked positions (jaehun.me
review, "Flash-Verify" and "How It Works: A Concrete Example"), and a
verification pass laid out as [tracked | confident | draft view | mask view]
where the two views share positions (same sections, Fig. 2).  The pages
measure LLaDA-1.5 on public benchmarks; no weights or data are used here, the
seeded tensors below stand in for them.

All tensors are created on the CPU with a seeded ``torch.Generator`` in fp32
and cast once (round to nearest even) to the layer's storage dtype: hidden
states X ~ N(0, 1) and weights W ~ N(0, w_std^2) with every bit of the storage
type's significand in use.  ``grid=True`` instead snaps them to a coarse dyadic
grid (see X_GRID) for the checks that need an fp32 projection exact in any
summation order.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import torch


@dataclass(frozen=True)
class LayerShape:
    B: int
    N: int
    d_model: int
    H: int
    Hkv: int
    dh: int
    rope_base: float = 10000.0
    dtype: torch.dtype = torch.bfloat16

    @property
    def cols(self) -> int:
        return (self.H + 2 * self.Hkv) * self.dh


@dataclass
class Workload:
    name: str
    shape: LayerShape
    nq: int
    x_rows: int
    seed: int
    X_pre: torch.Tensor          # [B, N, d]: hidden states the cache is built from
    X: torch.Tensor              # [B, x_rows, d]: hidden states of this step
    W: torch.Tensor              # [(H + 2 Hkv) dh, d]
    Q_idx: torch.Tensor          # [B, nq] int32: X row of each query
    pos_ids: torch.Tensor        # [B, nq] int32: position of each query
    vis: Optional[torch.Tensor]  # [B, nq, nq] uint8 or None (all visible)
    meta: dict = field(default_factory=dict)


SHAPES = {
    1: LayerShape(B=1, N=64, d_model=128, H=4, Hkv=4, dh=32, dtype=torch.float32),
    2: LayerShape(B=1, N=1024, d_model=4096, H=32, Hkv=32, dh=128),
    3: LayerShape(B=8, N=2048, d_model=4096, H=32, Hkv=32, dh=128),
    4: LayerShape(B=4, N=8192, d_model=3584, H=28, Hkv=4, dh=128),
    5: LayerShape(B=64, N=2048, d_model=4096, H=32, Hkv=8, dh=128),
    6: LayerShape(B=8, N=1024, d_model=4096, H=32, Hkv=32, dh=128),
    7: LayerShape(B=8, N=1024, d_model=4096, H=32, Hkv=32, dh=128),
}

NAMES = {
    1: "tiny fp32 layer B=1 N=64 d=128 H=Hkv=4 dh=32 |Q|=4",
    2: "8B-class layer draft pass B=1 N=1024 d=4096 H=Hkv=32 dh=128 |Q|=33",
    3: "8B-class layer Flash-Verify pass B=8 N=2048 d=4096 H=Hkv=32 dh=128 |Q|=44",
    4: "long-context GQA layer B=4 N=8192 d=3584 H=28 Hkv=4 dh=128 |Q|=32",
    5: "large-batch GQA layer B=64 N=2048 d=4096 H=32 Hkv=8 dh=128 |Q|=16",
    6: "default-window draft pass B=8 N=1024 d=4096 H=Hkv=32 dh=128 |Q|=144 (beta_t=80, beta_m=64)",
    7: "default-window verification pass, chain mask, B=8 N=1024 d=4096 H=Hkv=32 dh=128 |Q|=176",
}

BASE_SEED = 20260


# The optional dyadic grid (grid=True): X rounded to multiples of 1/8 (std 1),
# W to multiples of 1/512 (std w_std).  Every product x*w is then a multiple of
# 2^-12 and every partial sum of a row's projection (d_model <= 4096 terms,
# magnitude far below 2^11) fits in fp32's 24-bit significand, so the
# projection is exact in fp32 in any summation order and the stored k/v
# rounding depends on the rotary step alone.  Such values carry at most six
# significant bits, so these inputs serve bit-level checks of the stored rows
# only; the default inputs use the full bf16 significand.
X_GRID = 2.0 ** -3
W_GRID = 2.0 ** -9


def _randn(g, shape, std, dtype, grid=None):
    t = torch.randn(shape, generator=g, dtype=torch.float32) * std
    if grid is not None:
        t = torch.round(t / grid) * grid
    return t.to(dtype)


def _randint(g, lo, hi_incl):
    return int(torch.randint(lo, hi_incl + 1, (1,), generator=g).item())


def _perm(g, n):
    return torch.randperm(n, generator=g).tolist()


def hidden_and_weights(shape: LayerShape, x_rows: int, g: torch.Generator, w_std: float = 0.02,
                       grid: bool = False):
    X_pre = _randn(g, (shape.B, shape.N, shape.d_model), 1.0, shape.dtype, X_GRID if grid else None)
    W = _randn(g, (shape.cols, shape.d_model), w_std, shape.dtype, W_GRID if grid else None)
    return X_pre, W


def step_hidden(shape: LayerShape, X_pre, Q_idx, x_rows, g, grid: bool = False):
    """Hidden states of the step: the prefill states with the query rows (and
    any rows past N) redrawn, so that the step's cache writes are observable."""
    B, N, d = X_pre.shape
    xg = X_GRID if grid else None
    X = torch.empty((B, x_rows, d), dtype=shape.dtype)
    X[:, :N] = X_pre
    if x_rows > N:
        X[:, N:] = _randn(g, (B, x_rows - N, d), 1.0, shape.dtype, xg)
    for b in range(B):
        rows = sorted(set(int(r) for r in Q_idx[b].tolist() if r < N))
        if rows:
            X[b, rows] = _randn(g, (len(rows), d), 1.0, shape.dtype, xg)
    return X


def view_block_mask(groups: List[List[str]]) -> torch.Tensor:
    """[B, nq, nq] uint8: zero exactly on the draft-view x mask-view pairs."""
    B, nq = len(groups), len(groups[0])
    vis = torch.ones((B, nq, nq), dtype=torch.uint8)
    for b in range(B):
        gr = groups[b]
        d_rows = [i for i, t in enumerate(gr) if t == "draft"]
        m_rows = [i for i, t in enumerate(gr) if t == "mask"]
        for i in d_rows:
            for j in m_rows:
                vis[b, i, j] = 0
                vis[b, j, i] = 0
    return vis


def view_chain_mask(groups: List[List[str]]) -> torch.Tensor:
    """[B, nq, nq] uint8 chain-rule verification mask.  The k-th mask-view row
    (views in ascending position order) sees the draft view of the earlier
    exploratory positions and the mask view of its own and the later ones;
    draft-view rows and the context rows (tracked, confident) see the context
    and the whole draft view, never the mask view."""
    B, nq = len(groups), len(groups[0])
    vis = torch.zeros((B, nq, nq), dtype=torch.uint8)
    for b in range(B):
        gr = groups[b]
        ctx = [i for i, t in enumerate(gr) if t in ("track", "confident")]
        d_rows = [i for i, t in enumerate(gr) if t == "draft"]
        m_rows = [i for i, t in enumerate(gr) if t == "mask"]
        for i in ctx + d_rows:
            for j in ctx + d_rows:
                vis[b, i, j] = 1
        for k, i in enumerate(m_rows):
            for j in ctx + d_rows[:k] + m_rows[k:]:
                vis[b, i, j] = 1
    return vis


def make_workload(cid: int, layer: int = 0, w_std: float = 0.02, n_confident: int = 32,
                  grid: bool = False) -> Workload:
    """The layer configurations, seeded with 20260 + id (+1000 per layer).
    n_confident sets how many of the 64 window positions the verification
    pass (7) takes as confident; the rest are exploratory.  grid=True snaps
    X and W to the dyadic grid (same seeds, same index sets)."""
    shape = SHAPES[cid]
    seed = BASE_SEED + cid + 1000 * layer
    g = torch.Generator().manual_seed(seed)
    B, N = shape.B, shape.N
    meta = {}
    vis = None
    if cid == 1:
        nq, x_rows = 4, N
        Q = torch.tensor([[33, 34, 35, 36]], dtype=torch.int32)
        P = Q.clone()
    elif cid == 2:
        nq, x_rows = 33, N
        L = _randint(g, 512, 992)
        t = _randint(g, 0, L - 1)
        Q = torch.tensor([[t] + list(range(L, L + 32))], dtype=torch.int32)
        P = Q.clone()
        meta["decoded_prefix"] = [L]
    elif cid == 3:
        n_t, n_d, n_s = 4, 8, 16
        nq = n_t + n_d + 2 * n_s
        x_rows = N + n_s
        prompt, gen = N // 2, N - N // 2
        Qs, Ps, groups = [], [], []
        for b in range(B):
            r = float(torch.empty(1).uniform_(0.2, 0.8, generator=g).item())
            n_mask = max(n_d + n_s, int(round(r * gen)))
            first_mask = N - n_mask
            tv = sorted(_perm(g, first_mask)[:n_t])
            front = list(range(first_mask, first_mask + n_d + n_s))
            order = _perm(g, n_d + n_s)
            Dset = sorted(front[i] for i in order[:n_d])
            Sset = sorted(front[i] for i in order[n_d:])
            q_idx = tv + Dset + Sset + [N + k for k in range(n_s)]
            pos = tv + Dset + Sset + Sset
            Qs.append(q_idx)
            Ps.append(pos)
            groups.append(["track"] * n_t + ["confident"] * n_d + ["draft"] * n_s + ["mask"] * n_s)
            meta.setdefault("masked_from", []).append(first_mask)
        Q = torch.tensor(Qs, dtype=torch.int32)
        P = torch.tensor(Ps, dtype=torch.int32)
        vis = view_block_mask(groups)
        meta["groups"] = groups
    elif cid == 4:
        nq, x_rows = 32, N
        Ls = [_randint(g, 2048, 7000) for _ in range(B)]
        Q = torch.tensor([list(range(L, L + nq)) for L in Ls], dtype=torch.int32)
        P = Q.clone()
        meta["decoded_prefix"] = Ls
    elif cid == 5:
        nq, x_rows = 16, N
        # the query sets are shared by every layer of the stack
        gq = torch.Generator().manual_seed(BASE_SEED + cid)
        Ls = [_randint(gq, 512, 2000) for _ in range(B)]
        Q = torch.tensor([list(range(L, L + nq)) for L in Ls], dtype=torch.int32)
        P = Q.clone()
        meta["decoded_prefix"] = Ls
    elif cid in (6, 7):
        # the pages' default window: beta_t = 80 tracked decoded positions and
        # the first beta_m = 64 masked positions after a decoded prefix
        n_t, n_m = 80, 64
        Qs, Ps, groups = [], [], []
        if not 0 <= n_confident <= n_m:
            raise ValueError("n_confident must be in [0, %d]" % n_m)
        n_d = n_confident if cid == 7 else 0
        n_s = n_m - n_d
        for b in range(B):
            L = _randint(g, N // 2 + n_t, N - n_m)
            tv = sorted(_perm(g, L)[:n_t])
            front = list(range(L, L + n_m))
            if cid == 6:
                Qs.append(tv + front)
                Ps.append(tv + front)
                groups.append(["track"] * n_t + ["mask"] * n_m)
            else:
                order = _perm(g, n_m)
                Dset = sorted(front[i] for i in order[:n_d])
                Sset = sorted(front[i] for i in order[n_d:])
                Qs.append(tv + Dset + Sset + [N + k for k in range(n_s)])
                Ps.append(tv + Dset + Sset + Sset)
                groups.append(["track"] * n_t + ["confident"] * n_d + ["draft"] * n_s + ["mask"] * n_s)
            meta.setdefault("decoded_prefix", []).append(L)
        nq = len(Qs[0])
        x_rows = N + (n_s if cid == 7 else 0)
        Q = torch.tensor(Qs, dtype=torch.int32)
        P = torch.tensor(Ps, dtype=torch.int32)
        if cid == 7:
            vis = view_chain_mask(groups)
        meta["groups"] = groups
    else:
        raise ValueError("unknown configuration %r" % cid)
    X_pre, W = hidden_and_weights(shape, x_rows, g, w_std, grid)
    X = step_hidden(shape, X_pre, Q, x_rows, g, grid)
    meta["w_std"] = w_std
    meta["grid"] = grid
    name = NAMES[cid] if cid != 7 else NAMES[cid].replace("|Q|=176", "|Q|=%d" % nq)
    return Workload(name, shape, nq, x_rows, seed, X_pre, X, W, Q.contiguous(),
                    P.contiguous(), vis, meta)


def make_random_case(shape: LayerShape, nq: int, seed: int, *, n_extra_rows: int = 0,
                     dup_frac: float = 0.0, masked_vis: bool = False, w_std: float = 0.02,
                     positions: Optional[List[List[int]]] = None, grid: bool = False) -> Workload:
    """Small generic case for parity tests: random distinct positions per
    sequence, optionally some rows duplicated at an earlier row's position
    (reading from X rows past N, like a second view), and an optional random
    visibility mask."""
    g = torch.Generator().manual_seed(seed)
    B, N = shape.B, shape.N
    x_rows = N + n_extra_rows
    Qs, Ps = [], []
    for b in range(B):
        if positions is not None:
            pos = list(positions[b])
        else:
            n_dup = int(round(dup_frac * nq)) if nq > 1 else 0
            n_dup = min(n_dup, n_extra_rows, nq - 1) if nq > 1 else 0
            base = _perm(g, N)[: nq - n_dup]
            pos = list(base)
            for k in range(n_dup):
                pos.append(base[_randint(g, 0, len(base) - 1)])
        q_idx = []
        seen = set()
        extra = 0
        for p in pos:
            if p in seen and extra < n_extra_rows:
                q_idx.append(N + extra)
                extra += 1
            else:
                q_idx.append(p)
            seen.add(p)
        Qs.append(q_idx)
        Ps.append(pos)
    Q = torch.tensor(Qs, dtype=torch.int32).reshape(B, nq)
    P = torch.tensor(Ps, dtype=torch.int32).reshape(B, nq)
    vis = None
    if masked_vis and nq > 0:
        vis = (torch.rand((B, nq, nq), generator=g) < 0.7).to(torch.uint8)
    X_pre, W = hidden_and_weights(shape, x_rows, g, w_std, grid)
    X = step_hidden(shape, X_pre, Q, x_rows, g, grid)
    return Workload("random", shape, nq, x_rows, seed, X_pre, X, W, Q.contiguous(),
                    P.contiguous(), vis, {"w_std": w_std, "grid": grid})


CACHE_SEED_OFFSET = 7_000_003


def initial_cache(wl: Workload):
    """Seeded cache content before the step: Kc, Vc [B, Hkv, N, dh] in the
    storage dtype, drawn i.i.d. normal with the spread of a projected k/v
    element (w_std * sqrt(d_model) for unit-variance hidden states).  The step
    only reads the rows it does not overwrite, so any seeded content serves;
    both the GPU run and the oracle start from these tensors."""
    key = "_initial_cache"
    if key not in wl.meta:
        ls = wl.shape
        g = torch.Generator().manual_seed(wl.seed + CACHE_SEED_OFFSET)
        std = wl.meta.get("w_std", 0.02) * float(ls.d_model) ** 0.5
        shape = (ls.B, ls.Hkv, ls.N, ls.dh)
        wl.meta[key] = (_randn(g, shape, std, ls.dtype), _randn(g, shape, std, ls.dtype))
    return wl.meta[key]


def selection_inputs(wl: Workload):
    """Inputs of the tracked-set selection that follows the step: sel [B, nq]
    uint8 marks the masked query rows (the [MASK] group where the workload
    names groups, else the rows at or past the decoded prefix, else every
    other row); cand [B, N] uint8 marks the decoded positions (before the
    prefix end where there is one, else every position no query row writes)."""
    B, nq, N = wl.shape.B, wl.nq, wl.shape.N
    sel = torch.zeros((B, nq), dtype=torch.uint8)
    cand = torch.ones((B, N), dtype=torch.uint8)
    Ls = wl.meta.get("decoded_prefix")
    for b in range(B):
        if "groups" in wl.meta:
            sel[b] = torch.tensor([1 if t == "mask" else 0 for t in wl.meta["groups"][b]], dtype=torch.uint8)
        elif Ls is not None:
            sel[b] = (wl.pos_ids[b] >= Ls[b]).to(torch.uint8)
        else:
            sel[b, ::2] = 1
        if Ls is not None:
            cand[b, Ls[b]:] = 0
        else:
            cand[b, wl.pos_ids[b].long()] = 0
    return sel, cand


SYNTH_VOCAB = 131072   # synthetic vocabulary size (the pages name none)


def decision_logits(rows: int, V: int = SYNTH_VOCAB, seed: int = 7, dtype: torch.dtype = torch.bfloat16):
    """Seeded logits [rows, V] for the decision kernels: N(0, 2^2) noise with
    one raised id per row (raise drawn from U[0, 24]), so the confidences of
    the rows spread from near zero to near one."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((rows, V), generator=g, dtype=torch.float32) * 2.0
    top = torch.randint(0, V, (rows,), generator=g)
    lift = torch.rand((rows,), generator=g) * 24.0
    x[torch.arange(rows), top] += lift
    return x.to(dtype)


def paged_layout(wl: Workload, block_size: int, seed: int = 99, ragged: bool = True, spare_blocks: int = 7):
    """Seeded block table and per-sequence lengths for serving the workload's
    cache from a pool of blocks: each sequence gets its own blocks in a
    random order (plus spare blocks nobody uses), a valid length covering
    every position its rows write (when ragged: drawn up to N, else N), and a
    query count (when ragged: at least one row, else nq).  The pools start
    from the workload's initial cache placed through the table; spare
    blocks hold seeded values.  Returns table [B, max_blocks], Kpool, Vpool
    [blocks, Hkv, block_size, dh], seq_len [B], nq_seq [B] (int32 tensors)."""
    ls = wl.shape
    B, N, Hkv, dh = ls.B, ls.N, ls.Hkv, ls.dh
    g = torch.Generator().manual_seed(wl.seed * 31 + seed)
    max_blocks = (N + block_size - 1) // block_size
    nblocks = B * max_blocks + spare_blocks
    order = torch.randperm(nblocks, generator=g)
    table = order[:B * max_blocks].reshape(B, max_blocks).to(torch.int32)
    K0, V0 = initial_cache(wl)
    std = wl.meta.get("w_std", 0.02) * float(ls.d_model) ** 0.5
    Kpool = _randn(g, (nblocks, Hkv, block_size, dh), std, ls.dtype)
    Vpool = _randn(g, (nblocks, Hkv, block_size, dh), std, ls.dtype)
    for b in range(B):
        for k in range(max_blocks):
            p0, p1 = k * block_size, min(N, (k + 1) * block_size)
            blk = int(table[b, k])
            Kpool[blk, :, :p1 - p0] = K0[b, :, p0:p1]
            Vpool[blk, :, :p1 - p0] = V0[b, :, p0:p1]
    nq = wl.nq
    if ragged:
        nq_seq = torch.tensor([_randint(g, 1, nq) if nq > 0 else 0 for _ in range(B)], dtype=torch.int32)
        lens = []
        for b in range(B):
            live = wl.pos_ids[b, :int(nq_seq[b])]
            lo = int(live.max()) + 1 if live.numel() else 1
            lens.append(_randint(g, lo, N))
        seq_len = torch.tensor(lens, dtype=torch.int32)
    else:
        nq_seq = torch.full((B,), nq, dtype=torch.int32)
        seq_len = torch.full((B,), N, dtype=torch.int32)
    return table, Kpool, Vpool, seq_len, nq_seq
