"""ctypes binding of libfdllm (include/fdllm.h): argument marshalling only.

Every step of the fused KV-cache step runs in the library's HIP kernels; this
module checks tensor devices, dtypes and shapes, passes raw device pointers
and the current HIP stream, and turns status codes into exceptions.  It
raises if the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfdllm.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "fdllm.h")
HEADERS = [os.path.join(os.path.dirname(_PKG), "include", h) for h in ("fdllm.h", "fdllm_probe.h")]

FDLLM_F32, FDLLM_BF16 = 0, 1
STATUS = {0: "FDLLM_OK", -1: "FDLLM_ERR_ARG", -2: "FDLLM_ERR_SHAPE", -3: "FDLLM_ERR_ALIGN",
          -4: "FDLLM_ERR_INDEX", -5: "FDLLM_ERR_ALLOC", -6: "FDLLM_ERR_HIP", -7: "FDLLM_ERR_UNSUPPORTED",
          -8: "FDLLM_ERR_SCRATCH"}


class FdllmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (what, STATUS.get(status, "?"), status))


class Config(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("H", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("dh", ctypes.c_int32),
                ("q_max", ctypes.c_int32), ("rope_base", ctypes.c_double), ("dtype", ctypes.c_int32)]


class Tuning(ctypes.Structure):
    _fields_ = [("attn_splits", ctypes.c_int32), ("gemm_splitk", ctypes.c_int32),
                ("kernel_family", ctypes.c_int32), ("proj_tile", ctypes.c_int32)]


_lib = None


def declared_symbols():
    """Function names declared in the library's headers (include/fdllm*.h)."""
    names = set()
    for path in HEADERS:
        with open(path) as f:
            names |= set(re.findall(r"^\s*(?:int|const char\*)\s+(fdllm_\w+)\s*\(", f.read(), re.M))
    return sorted(names)


def load():
    """Load libfdllm.so (built by io_aware_kv_amd.build); raises if missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libfdllm.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.fdllm_validate_config.argtypes = [ctypes.POINTER(Config)]
    lib.fdllm_cache_init.argtypes = [ctypes.POINTER(P), ctypes.POINTER(Config), P, P, P, P, P]
    lib.fdllm_prefill.argtypes = [P, P, i32, P, P, P, P]
    lib.fdllm_fused_step.argtypes = [P, P, i32, P, P, i32, P, P, P, P, P, P, P]
    lib.fdllm_step_project.argtypes = [P, P, i32, P, P, i32, P, P, P, P]
    lib.fdllm_step_attend.argtypes = [P, P, i32, P, P, P, P, P, P]
    lib.fdllm_fused_step_paged.argtypes = [P, P, i32, P, P, i32, P, P, P, P, P, P, i32, i32, i32, P, P, P, P]
    lib.fdllm_tracked_scores.argtypes = [P, P, i32, P, P, P, P, P, P]
    lib.fdllm_select_tracked.argtypes = [P, P, P, i32, P, P]
    lib.fdllm_confidence.argtypes = [P, i32, ctypes.c_int64, i32, i32, ctypes.c_float, P, P, P, P]
    lib.fdllm_accept.argtypes = [P, P, P, i32, i32, ctypes.c_float, P, P]
    lib.fdllm_set_tuning.argtypes = [P, ctypes.POINTER(Tuning)]
    lib.fdllm_get_plan.argtypes = [P, i32, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.fdllm_cache_destroy.argtypes = [P]
    lib.fdllm_probe_read.argtypes = [P, ctypes.c_int64, i32, P, P]
    lib.fdllm_probe_mfma.argtypes = [i32, i32, i32, P, P]
    lib.fdllm_probe_lds_dma.argtypes = [P, ctypes.c_int64, i32, i32, i32, P, P]
    lib.fdllm_fused_step_noalloc.argtypes = [ctypes.POINTER(Config), P, i32, P, P, i32, P, P, P, P, P, P, P]
    lib.fdllm_status_str.argtypes = [ctypes.c_int]
    lib.fdllm_status_str.restype = ctypes.c_char_p
    for name in ("fdllm_validate_config", "fdllm_cache_init", "fdllm_prefill", "fdllm_fused_step",
                 "fdllm_step_project", "fdllm_step_attend", "fdllm_tracked_scores", "fdllm_select_tracked",
                 "fdllm_confidence", "fdllm_accept", "fdllm_fused_step_paged",
                 "fdllm_set_tuning", "fdllm_get_plan", "fdllm_cache_destroy", "fdllm_probe_read",
                 "fdllm_fused_step_noalloc"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        raise FdllmError(rc, what)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return FDLLM_BF16
    if dtype == torch.float32:
        return FDLLM_F32
    raise ValueError("dtype must be bfloat16 or float32")


def confidence(logits: torch.Tensor, mask_id: int, thr: float, pred: torch.Tensor, conf: torch.Tensor,
               over: Optional[torch.Tensor] = None, stream=None):
    """Per-row prediction and confidence of logits [..., V] (see fdllm.h);
    pred int32, conf fp32 and over uint8 hold one value per row."""
    V = logits.shape[-1]
    rows = logits.numel() // V
    for name, t, dt in (("pred", pred, torch.int32), ("conf", conf, torch.float32)):
        if t.dtype != dt or t.numel() != rows:
            raise ValueError("%s must be %s with one value per row" % (name, dt))
    if over is not None and (over.dtype != torch.uint8 or over.numel() != rows):
        raise ValueError("over must be uint8 with one value per row")
    _check(load().fdllm_confidence(_ptr(logits), _dtype_code(logits.dtype), rows, V, mask_id, float(thr),
                                   _ptr(pred), _ptr(conf), _ptr(over), _stream(stream)), "fdllm_confidence")


def accept(x_hat: torch.Tensor, x_tilde: torch.Tensor, c_tilde: torch.Tensor, gamma: float,
           n_accept: torch.Tensor, stream=None):
    """Sequential acceptance over [B, S] rows in decoding order into n_accept [B] int32."""
    B, S = x_hat.shape
    if x_hat.dtype != torch.int32 or x_tilde.dtype != torch.int32 or c_tilde.dtype != torch.float32:
        raise ValueError("x_hat, x_tilde int32 and c_tilde fp32 [B, S]")
    if tuple(x_tilde.shape) != (B, S) or tuple(c_tilde.shape) != (B, S):
        raise ValueError("x_tilde and c_tilde must be [B, S]")
    if n_accept.dtype != torch.int32 or n_accept.numel() != B:
        raise ValueError("n_accept must be int32 [B]")
    _check(load().fdllm_accept(_ptr(x_hat), _ptr(x_tilde), _ptr(c_tilde), B, S, float(gamma), _ptr(n_accept),
                               _stream(stream)), "fdllm_accept")


def probe_read(buf: torch.Tensor, sink: torch.Tensor, workgroups: int = 0, stream=None):
    """One streaming read of buf (fdllm_probe.h); sink is a 16-byte device buffer."""
    if sink.numel() * sink.element_size() < 16:
        raise ValueError("sink must hold 16 bytes")
    _check(load().fdllm_probe_read(_ptr(buf), buf.numel() * buf.element_size(), workgroups, _ptr(sink),
                                   _stream(stream)), "fdllm_probe_read")


def probe_mfma(sink: torch.Tensor, workgroups: int = 0, waves: int = 4, iters: int = 4096, stream=None):
    """Issue-rate probe of the bf16 MFMA (fdllm_probe.h); executed flops are
    workgroups * waves * iters * 8 * 16384 (workgroups 0 means 256)."""
    _check(load().fdllm_probe_mfma(workgroups, waves, iters, _ptr(sink), _stream(stream)), "fdllm_probe_mfma")


def probe_lds_dma(buf: torch.Tensor, sink: torch.Tensor, workgroups: int = 0, waves: int = 4, iters: int = 4096,
                  stream=None):
    """LDS-DMA rate probe over buf (fdllm_probe.h); bytes moved are
    workgroups * waves * iters * 1024 (workgroups 0 means 256)."""
    _check(load().fdllm_probe_lds_dma(_ptr(buf), buf.numel() * buf.element_size(), workgroups, waves, iters,
                                      _ptr(sink), _stream(stream)), "fdllm_probe_lds_dma")


def fused_step_noalloc(X, Q_idx, pos_ids, vis, W, Kc, Vc, O, LSE, H, Hkv, rope_base=10000.0, q_max=None,
                       stream=None):
    """The fused step without a handle (fdllm_fused_step_noalloc): the layer
    shape comes from the tensors (X [B, x_rows, d], Kc [B, Hkv, N, dh]) and
    H, Hkv; the workspace is the library's static per-device scratch."""
    B, x_rows, d = X.shape
    N, dh = Kc.shape[2], Kc.shape[3]
    nq = Q_idx.shape[1]
    cfg = make_config(B, N, d, H, Hkv, dh, q_max or max(1, nq), X.dtype, rope_base)
    for name, t, shape in (("Q_idx", Q_idx, (B, nq)), ("pos_ids", pos_ids, (B, nq))):
        if t.dtype != torch.int32 or tuple(t.shape) != shape:
            raise ValueError("%s must be int32 [B, nq]" % name)
    if vis is not None and (vis.dtype != torch.uint8 or tuple(vis.shape) != (B, nq, nq)):
        raise ValueError("vis must be uint8 [B, nq, nq]")
    if tuple(W.shape) != ((H + 2 * Hkv) * dh, d) or tuple(Vc.shape) != tuple(Kc.shape) or Kc.shape[:2] != (B, Hkv):
        raise ValueError("W must be [(H + 2 Hkv) dh, d], Kc/Vc [B, Hkv, N, dh]")
    if tuple(O.shape) != (B, nq, H, dh) or tuple(LSE.shape) != (B, nq, H) or LSE.dtype != torch.float32:
        raise ValueError("O must be [B, nq, H, dh], LSE fp32 [B, nq, H]")
    for t in (W, Kc, Vc, O):
        if t.dtype != X.dtype:
            raise ValueError("X, W, Kc, Vc and O share the layer dtype")
    _check(load().fdllm_fused_step_noalloc(ctypes.byref(cfg), _ptr(X), x_rows, _ptr(Q_idx), _ptr(pos_ids), nq,
                                           _ptr(vis), _ptr(W), _ptr(Kc), _ptr(Vc), _ptr(O), _ptr(LSE),
                                           _stream(stream)), "fdllm_fused_step_noalloc")


def make_config(B, N, d_model, H, Hkv, dh, q_max, dtype=torch.bfloat16, rope_base=10000.0) -> Config:
    return Config(B, N, d_model, H, Hkv, dh, q_max, float(rope_base), _dtype_code(dtype))


def validate_config(cfg: Config) -> int:
    """Host-only configuration check; returns the status code."""
    return load().fdllm_validate_config(ctypes.byref(cfg))


class FusedKVCache:
    """A library handle for one layer shape: workspace plus the fused step."""

    def __init__(self, B, N, d_model, H, Hkv, dh, q_max, dtype=torch.bfloat16, rope_base=10000.0,
                 X_full=None, W=None, Kc=None, Vc=None, stream=None):
        lib = load()
        self.cfg = make_config(B, N, d_model, H, Hkv, dh, q_max, dtype, rope_base)
        self.dtype = dtype
        h = ctypes.c_void_p()
        if X_full is not None:
            self._check_layer(X_full, W, Kc, Vc)
        rc = lib.fdllm_cache_init(ctypes.byref(h), ctypes.byref(self.cfg), _ptr(X_full), _ptr(W),
                                  _ptr(Kc), _ptr(Vc), _stream(stream))
        _check(rc, "fdllm_cache_init")
        self._h = h

    def _check_layer(self, X, W, Kc, Vc):
        c = self.cfg
        for name, t in (("X", X), ("W", W), ("Kc", Kc), ("Vc", Vc)):
            if t is None or t.dtype != self.dtype:
                raise ValueError("%s must be a %s tensor" % (name, self.dtype))
        if X.dim() != 3 or X.shape[0] != c.B or X.shape[2] != c.d_model:
            raise ValueError("X must be [B, x_rows, d_model]")
        if tuple(W.shape) != ((c.H + 2 * c.Hkv) * c.dh, c.d_model):
            raise ValueError("W must be [(H + 2 Hkv) dh, d_model]")
        for t in (Kc, Vc):
            if tuple(t.shape) != (c.B, c.Hkv, c.N, c.dh):
                raise ValueError("Kc/Vc must be [B, Hkv, N, dh]")

    @property
    def handle(self):
        return self._h

    def prefill(self, X, W, Kc, Vc, stream=None):
        self._check_layer(X, W, Kc, Vc)
        rc = load().fdllm_prefill(self._h, _ptr(X), X.shape[1], _ptr(W), _ptr(Kc), _ptr(Vc), _stream(stream))
        _check(rc, "fdllm_prefill")

    def step(self, X, Q_idx, pos_ids, vis, W, Kc, Vc, O, LSE, stream=None):
        """One fused step.  O [B,nq,H,dh] and LSE [B,nq,H] (fp32) are written."""
        c = self.cfg
        self._check_layer(X, W, Kc, Vc)
        nq = Q_idx.shape[1]
        if Q_idx.dtype != torch.int32 or pos_ids.dtype != torch.int32:
            raise ValueError("Q_idx and pos_ids must be int32")
        if tuple(Q_idx.shape) != (c.B, nq) or tuple(pos_ids.shape) != (c.B, nq):
            raise ValueError("Q_idx and pos_ids must be [B, nq]")
        if vis is not None and (vis.dtype != torch.uint8 or tuple(vis.shape) != (c.B, nq, nq)):
            raise ValueError("vis must be uint8 [B, nq, nq]")
        if O.dtype != self.dtype or tuple(O.shape) != (c.B, nq, c.H, c.dh):
            raise ValueError("O must be [B, nq, H, dh] of the layer dtype")
        if LSE.dtype != torch.float32 or tuple(LSE.shape) != (c.B, nq, c.H):
            raise ValueError("LSE must be fp32 [B, nq, H]")
        rc = load().fdllm_fused_step(self._h, _ptr(X), X.shape[1], _ptr(Q_idx), _ptr(pos_ids), nq,
                                     _ptr(vis), _ptr(W), _ptr(Kc), _ptr(Vc), _ptr(O), _ptr(LSE),
                                     _stream(stream))
        _check(rc, "fdllm_fused_step")

    def step_paged(self, X, Q_idx, pos_ids, vis, W, Kpool, Vpool, O, LSE, block_table=None, block_size=0,
                   num_blocks=0, seq_len=None, nq_seq=None, stream=None):
        """The fused step over a paged cache (block_table [B, max_blocks]
        int32, pools [num_blocks, Hkv, block_size, dh]) or the flat layout
        (block_table None), with optional seq_len [B] and nq_seq [B] int32."""
        c = self.cfg
        nq = Q_idx.shape[1]
        for name, t in (("seq_len", seq_len), ("nq_seq", nq_seq)):
            if t is not None and (t.dtype != torch.int32 or tuple(t.shape) != (c.B,)):
                raise ValueError("%s must be int32 [B]" % name)
        max_blocks = 0
        if block_table is not None:
            if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != c.B:
                raise ValueError("block_table must be int32 [B, max_blocks]")
            max_blocks = block_table.shape[1]
            for t in (Kpool, Vpool):
                if tuple(t.shape) != (num_blocks, c.Hkv, block_size, c.dh) or t.dtype != self.dtype:
                    raise ValueError("pools must be [num_blocks, Hkv, block_size, dh] of the layer dtype")
        rc = load().fdllm_fused_step_paged(self._h, _ptr(X), X.shape[1], _ptr(Q_idx), _ptr(pos_ids), nq,
                                           _ptr(nq_seq), _ptr(vis), _ptr(W), _ptr(Kpool), _ptr(Vpool),
                                           _ptr(block_table), block_size, max_blocks, num_blocks, _ptr(seq_len),
                                           _ptr(O), _ptr(LSE), _stream(stream))
        _check(rc, "fdllm_fused_step_paged")

    def project(self, X, Q_idx, pos_ids, W, Kc, Vc, stream=None):
        """First launch of the step (gather, projection, rotary, k/v write)."""
        self._check_layer(X, W, Kc, Vc)
        nq = Q_idx.shape[1]
        rc = load().fdllm_step_project(self._h, _ptr(X), X.shape[1], _ptr(Q_idx), _ptr(pos_ids), nq,
                                       _ptr(W), _ptr(Kc), _ptr(Vc), _stream(stream))
        _check(rc, "fdllm_step_project")

    def attend(self, pos_ids, vis, Kc, Vc, O, LSE, stream=None):
        """Second launch of the step (attention over the cache, split combine)."""
        nq = pos_ids.shape[1]
        rc = load().fdllm_step_attend(self._h, _ptr(pos_ids), nq, _ptr(vis), _ptr(Kc), _ptr(Vc), _ptr(O),
                                      _ptr(LSE), _stream(stream))
        _check(rc, "fdllm_step_attend")

    def tracked_scores(self, pos_ids, vis, sel, Kc, LSE, scores, stream=None):
        """Attention mass of the selected rows (sel [B, nq] uint8) on every
        cache position, after the step of the same nq: scores [B, N] fp32."""
        c = self.cfg
        nq = pos_ids.shape[1]
        if sel.dtype != torch.uint8 or tuple(sel.shape) != (c.B, nq):
            raise ValueError("sel must be uint8 [B, nq]")
        if scores.dtype != torch.float32 or tuple(scores.shape) != (c.B, c.N):
            raise ValueError("scores must be fp32 [B, N]")
        rc = load().fdllm_tracked_scores(self._h, _ptr(pos_ids), nq, _ptr(vis), _ptr(sel), _ptr(Kc), _ptr(LSE),
                                         _ptr(scores), _stream(stream))
        _check(rc, "fdllm_tracked_scores")

    def select_tracked(self, scores, cand, k, out, stream=None):
        """Top-k candidate positions by score per sequence into out [B, k] int32."""
        c = self.cfg
        if cand.dtype != torch.uint8 or tuple(cand.shape) != (c.B, c.N):
            raise ValueError("cand must be uint8 [B, N]")
        if out.dtype != torch.int32 or tuple(out.shape) != (c.B, k):
            raise ValueError("out must be int32 [B, k]")
        rc = load().fdllm_select_tracked(self._h, _ptr(scores), _ptr(cand), k, _ptr(out), _stream(stream))
        _check(rc, "fdllm_select_tracked")

    def set_tuning(self, attn_splits=0, gemm_splitk=0, kernel_family=0, proj_tile=0):
        t = Tuning(attn_splits, gemm_splitk, kernel_family, proj_tile)
        _check(load().fdllm_set_tuning(self._h, ctypes.byref(t)), "fdllm_set_tuning")

    def plan(self, nq):
        a, g, f = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(load().fdllm_get_plan(self._h, nq, ctypes.byref(a), ctypes.byref(g), ctypes.byref(f)),
               "fdllm_get_plan")
        return {"attn_splits": a.value, "gemm_splitk": g.value, "kernel_family": f.value}

    def close(self):
        if getattr(self, "_h", None):
            _check(load().fdllm_cache_destroy(self._h), "fdllm_cache_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
