"""Plain fp64 CPU oracle of the fused KV-cache step, and its ctypes loader.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` are the only callers.  The HIP product path never
imports this package, and this package imports nothing from the product.

The arithmetic lives in ``fdllm_oracle.c`` (plain loops in fp64, OpenMP over
independent rows); this module only converts arrays to fp64 and back.  The
decision helpers of the verification pass live in ``oracle.decode``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fdllm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ROUND_EXACT, ROUND_FP32, ROUND_BF16 = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (-O3 -fopenmp).  Returns the path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-march=x86-64-v2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c11", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("dh", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("round_mode", ctypes.c_int32)]


_lib = None


def bind(path: str):
    """Open a compiled oracle library and declare its entry points."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.fdllm_oracle_round.argtypes = [P, P, ctypes.c_int64, i32]
    lib.fdllm_oracle_round.restype = None
    lib.fdllm_oracle_project.argtypes = [P, P, i32, P, P, i32, P, P, P, P]
    lib.fdllm_oracle_project.restype = ctypes.c_int
    lib.fdllm_oracle_step.argtypes = [P, P, i32, P, P, i32, P, P, P, P, P, P, P, P, P]
    lib.fdllm_oracle_step.restype = ctypes.c_int
    lib.fdllm_oracle_prefill.argtypes = [P, P, i32, P, P, P]
    lib.fdllm_oracle_prefill.restype = ctypes.c_int
    lib.fdllm_oracle_key_scores.argtypes = [P, P, P, P, P, i32, P, P, P]
    lib.fdllm_oracle_key_scores.restype = ctypes.c_int
    lib.fdllm_oracle_threads.argtypes = []
    lib.fdllm_oracle_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        # FDLLM_ORACLE_LIB lets the mutation tests swap in a deliberately broken copy
        alt = os.environ.get("FDLLM_ORACLE_LIB")
        _lib = bind(alt if alt else build())
    return _lib


@dataclass
class Shape:
    B: int
    N: int
    d_model: int
    H: int
    Hkv: int
    dh: int
    rope_base: float = 10000.0


def _f64(a):
    """Exact upcast to a C-contiguous fp64 numpy array (bf16/fp32 -> fp64 is exact)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return np.ascontiguousarray(a.detach().to("cpu", torch.float64).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a):
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return np.ascontiguousarray(a.detach().to("cpu", torch.int32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _cfg(shape: Shape, round_mode: int) -> _Cfg:
    return _Cfg(shape.B, shape.N, shape.d_model, shape.H, shape.Hkv, shape.dh,
                float(shape.rope_base), int(round_mode))


def threads() -> int:
    """OpenMP threads the oracle's loops run on."""
    return int(_load().fdllm_oracle_threads())


def round_store(x, mode: int) -> np.ndarray:
    """Round fp64 values to the storage type (1 = fp32, 2 = bf16, nearest-even)."""
    a = _f64(x)
    out = np.empty_like(a)
    _load().fdllm_oracle_round(_ptr(a), _ptr(out), a.size, int(mode))
    return out


def project(shape: Shape, X, Q_idx, pos_ids, W, round_mode: int):
    """Gather + projection + rotary; k and v rounded to the storage type (q is
    an on-chip value and stays unrounded).  Returns q [B,nq,H,dh], k, v [B,nq,Hkv,dh]."""
    X = _f64(X)
    Qi, Pi, W = _i32(Q_idx), _i32(pos_ids), _f64(W)
    B, x_rows = X.shape[0], X.shape[1]
    nq = Qi.shape[1]
    q = np.empty((B, nq, shape.H, shape.dh))
    k = np.empty((B, nq, shape.Hkv, shape.dh))
    v = np.empty_like(k)
    c = _cfg(shape, round_mode)
    rc = _load().fdllm_oracle_project(ctypes.byref(c), _ptr(X), x_rows, _ptr(Qi), _ptr(Pi), nq,
                                      _ptr(W), _ptr(q), _ptr(k), _ptr(v))
    if rc != 0:
        raise ValueError("oracle project failed: %d" % rc)
    return q, k, v


def step(shape: Shape, X, Q_idx, pos_ids, vis, W, Kc, Vc, round_mode: int):
    """One fused step.  Kc/Vc are copied (the caller's arrays are not touched).

    Returns dict with O [B,nq,H,dh], LSE [B,nq,H], Kc, Vc (updated copies) and
    the query rows' q (unrounded) and k, v (rounded to the storage type).
    """
    X = _f64(X)
    Qi, Pi, W = _i32(Q_idx), _i32(pos_ids), _f64(W)
    Kc = _f64(Kc).copy()
    Vc = _f64(Vc).copy()
    B, x_rows = X.shape[0], X.shape[1]
    nq = Qi.shape[1]
    vis_a = None
    if vis is not None:
        try:
            import torch
            if isinstance(vis, torch.Tensor):
                vis = vis.detach().cpu().numpy()
        except ImportError:  # pragma: no cover
            pass
        vis_a = np.ascontiguousarray(np.asarray(vis, dtype=np.uint8))
        assert vis_a.shape == (B, nq, nq)
    O = np.empty((B, nq, shape.H, shape.dh))
    LSE = np.empty((B, nq, shape.H))
    q = np.empty((B, nq, shape.H, shape.dh))
    k = np.empty((B, nq, shape.Hkv, shape.dh))
    v = np.empty_like(k)
    c = _cfg(shape, round_mode)
    rc = _load().fdllm_oracle_step(ctypes.byref(c), _ptr(X), x_rows, _ptr(Qi), _ptr(Pi), nq,
                                   _ptr(vis_a), _ptr(W), _ptr(Kc), _ptr(Vc), _ptr(O), _ptr(LSE),
                                   _ptr(q), _ptr(k), _ptr(v))
    if rc != 0:
        raise ValueError("oracle step failed: %d" % rc)
    return {"O": O, "LSE": LSE, "Kc": Kc, "Vc": Vc, "q": q, "k": k, "v": v}


def prefill(shape: Shape, X, W, round_mode: int):
    """Build the cache from a full sequence (X row p at position p).  Returns Kc, Vc."""
    X = _f64(X)
    W = _f64(W)
    B, x_rows = X.shape[0], X.shape[1]
    Kc = np.empty((B, shape.Hkv, shape.N, shape.dh))
    Vc = np.empty_like(Kc)
    c = _cfg(shape, round_mode)
    rc = _load().fdllm_oracle_prefill(ctypes.byref(c), _ptr(X), x_rows, _ptr(W), _ptr(Kc), _ptr(Vc))
    if rc != 0:
        raise ValueError("oracle prefill failed: %d" % rc)
    return Kc, Vc


def _u8(a):
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return np.ascontiguousarray(a.detach().to("cpu", torch.uint8).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint8))


def key_scores(shape: Shape, q, Kc, LSE, pos_ids, vis, sel):
    """Tracked-set scores a_p [B, N]: attention mass of the selected query rows
    on each cache position (see fdllm_oracle.c).  q is the step's unrounded q,
    Kc the cache after the step, LSE the step's."""
    q, Kc, LSE = _f64(q), _f64(Kc), _f64(LSE)
    Pi = _i32(pos_ids)
    B, nq = Pi.shape
    sel_a = _u8(sel)
    vis_a = None if vis is None else _u8(vis)
    out = np.empty((B, shape.N))
    c = _cfg(shape, ROUND_EXACT)
    rc = _load().fdllm_oracle_key_scores(ctypes.byref(c), _ptr(q), _ptr(Kc), _ptr(LSE), _ptr(Pi), nq,
                                         _ptr(vis_a), _ptr(sel_a), _ptr(out))
    if rc != 0:
        raise ValueError("oracle key scores failed: %d" % rc)
    return out


def select_top(scores, cand, k: int):
    """Top-k candidate positions per sequence by score, highest first; equal
    scores go to the lower position; -1 fills the rows with fewer than k
    candidates.  The comparison is made on the scores as given (the caller
    passes the precision the ranking is decided in)."""
    sc = np.asarray(scores)
    cd = np.asarray(cand).astype(bool)
    B, N = sc.shape
    out = np.full((B, k), -1, dtype=np.int32)
    for b in range(B):
        idx = [p for p in range(N) if cd[b, p]]
        idx.sort(key=lambda p: (-sc[b, p], p))
        for t, p in enumerate(idx[:k]):
            out[b, t] = p
    return out


def step_paged(shape: Shape, X, Q_idx, pos_ids, nq_seq, vis, W, Kpool, Vpool, table, block_size: int, seq_len,
               round_mode: int):
    """The step over a paged cache with per-sequence lengths and query counts,
    by its definition: sequence b's cache is the rows p < seq_len[b] gathered
    from its blocks (position p in block table[b, p // block_size], row
    p % block_size of pools [blocks, Hkv, block_size, dh]); its live query
    rows are j < nq_seq[b]; ``step`` runs on that flat cache alone and the
    written rows go back to their blocks.  Padding rows get O = 0, LSE = -inf.
    Returns dict with O, LSE and the updated pools (copies)."""
    X = _f64(X)
    Qi, Pi = _i32(Q_idx), _i32(pos_ids)
    B, nq = Qi.shape
    Kp = _f64(Kpool).copy()
    Vp = _f64(Vpool).copy()
    tab = _i32(table)
    L = _i32(seq_len) if seq_len is not None else np.full(B, shape.N, dtype=np.int32)
    nb = _i32(nq_seq) if nq_seq is not None else np.full(B, nq, dtype=np.int32)
    vis_a = None
    if vis is not None:
        try:
            import torch
            if isinstance(vis, torch.Tensor):
                vis = vis.detach().cpu().numpy()
        except ImportError:  # pragma: no cover
            pass
        vis_a = np.asarray(vis, dtype=np.uint8)
    O = np.zeros((B, nq, shape.H, shape.dh))
    LSE = np.full((B, nq, shape.H), -np.inf)
    for b in range(B):
        Lb, n = int(L[b]), int(nb[b])
        blk = np.array([tab[b, p // block_size] for p in range(Lb)], dtype=np.int64)
        row = np.arange(Lb) % block_size
        Kb = Kp[blk, :, row, :].transpose(1, 0, 2)[None]        # [1, Hkv, Lb, dh]
        Vb = Vp[blk, :, row, :].transpose(1, 0, 2)[None]
        if n > 0:
            sh = Shape(1, Lb, shape.d_model, shape.H, shape.Hkv, shape.dh, shape.rope_base)
            vb = None if vis_a is None else vis_a[b:b + 1, :n, :n]
            r = step(sh, X[b:b + 1], Qi[b:b + 1, :n], Pi[b:b + 1, :n], vb, W, Kb, Vb, round_mode)
            O[b, :n], LSE[b, :n] = r["O"][0], r["LSE"][0]
            Kb, Vb = r["Kc"], r["Vc"]
        Kp[blk, :, row, :] = Kb[0].transpose(1, 0, 2)
        Vp[blk, :, row, :] = Vb[0].transpose(1, 0, 2)
    return {"O": O, "LSE": LSE, "Kpool": Kp, "Vpool": Vp}
