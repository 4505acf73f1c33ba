"""The C-ABI library loads, exports what include/fdllm.h declares, and rejects
bad arguments on the host before touching the GPU (no compute calls here)."""
import ctypes
import os

import pytest
import torch

from io_aware_kv_amd import binding


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from io_aware_kv_amd import build
        build.build(verbose=False)
    return binding.load()


def test_every_declared_symbol_is_exported(lib):
    names = binding.declared_symbols()
    assert {"fdllm_cache_init", "fdllm_fused_step", "fdllm_cache_destroy", "fdllm_status_str",
            "fdllm_prefill", "fdllm_validate_config", "fdllm_set_tuning", "fdllm_get_plan"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in binding.STATUS.items():
        assert lib.fdllm_status_str(code).decode().startswith(name)
    assert b"unknown" in lib.fdllm_status_str(-99)


def _cfg(**kw):
    base = dict(B=2, N=64, d_model=256, H=4, Hkv=2, dh=128, q_max=8, dtype=torch.bfloat16)
    base.update(kw)
    return binding.make_config(**base)


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    ({"dtype": torch.float32, "dh": 32, "d_model": 128}, 0),
    ({"B": 0}, -1), ({"N": 0}, -1), ({"H": 3}, -1), ({"dh": 7}, -1), ({"q_max": 0}, -1),
    ({"rope_base": 0.0}, -1), ({"rope_base": -1.0}, -1),
    ({"dh": 4}, -7),            # a bf16 head of 4 is not a whole 16-byte row
    ({"d_model": 12}, -7),
    ({"dh": 512}, -7),
])
def test_validate_config(lib, kw, status):
    assert binding.validate_config(_cfg(**kw)) == status


def test_bad_dtype_code_rejected(lib):
    c = _cfg()
    c.dtype = 7
    assert binding.validate_config(c) == -1


def test_null_handle_and_shape_errors_are_host_side(lib):
    P = ctypes.c_void_p
    assert lib.fdllm_fused_step(None, None, 1, None, None, 1, None, None, None, None, None, None, None) == -1
    assert lib.fdllm_prefill(None, None, 1, None, None, None, None) == -1
    assert lib.fdllm_get_plan(None, 1, None, None, None) == -1
    assert lib.fdllm_set_tuning(None, None) == -1
    assert lib.fdllm_cache_destroy(None) == 0
    out = P()
    assert lib.fdllm_cache_init(None, ctypes.byref(_cfg()), None, None, None, None, None) == -1
    bad = _cfg(H=5)
    assert lib.fdllm_cache_init(ctypes.byref(out), ctypes.byref(bad), None, None, None, None, None) == -1
    assert not out.value
    # X_full without the weight or caches is an argument error, caught before any HIP call
    assert lib.fdllm_cache_init(ctypes.byref(out), ctypes.byref(_cfg()), P(16), None, None, None, None) == -1


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU error path")
def test_init_without_gpu_reports_hip_error(lib):
    out = ctypes.c_void_p()
    rc = lib.fdllm_cache_init(ctypes.byref(out), ctypes.byref(_cfg()), None, None, None, None, None)
    assert rc in (-6, -5) and not out.value


def test_read_probe_argument_errors_are_host_side(lib):
    P = ctypes.c_void_p
    assert lib.fdllm_probe_read(None, 1024, 0, P(16), None) == -1
    assert lib.fdllm_probe_read(P(16), 1024, 0, None, None) == -1
    assert lib.fdllm_probe_read(P(16), 8, 0, P(16), None) == -1       # fewer than 16 bytes
    assert lib.fdllm_probe_read(P(16), 1000, 0, P(16), None) == -1    # not whole 16-byte chunks
    assert lib.fdllm_probe_read(P(16), 1024, -1, P(16), None) == -1
    assert lib.fdllm_probe_read(P(24), 1024, 0, P(16), None) == -3    # misaligned buffer


def test_rate_probe_argument_errors_are_host_side(lib):
    P = ctypes.c_void_p
    assert lib.fdllm_probe_mfma(0, 4, 16, None, None) == -1
    assert lib.fdllm_probe_mfma(-1, 4, 16, P(16), None) == -1
    assert lib.fdllm_probe_mfma(0, 0, 16, P(16), None) == -1         # no wave
    assert lib.fdllm_probe_mfma(0, 9, 16, P(16), None) == -1         # more than eight waves
    assert lib.fdllm_probe_mfma(0, 4, 0, P(16), None) == -1
    assert lib.fdllm_probe_mfma(0, 4, 16, P(24), None) == -3         # misaligned sink
    assert lib.fdllm_probe_lds_dma(None, 1024, 0, 4, 16, P(16), None) == -1
    assert lib.fdllm_probe_lds_dma(P(16), 1000, 0, 4, 16, P(16), None) == -1   # not whole 1 KB blocks
    assert lib.fdllm_probe_lds_dma(P(16), 512, 0, 4, 16, P(16), None) == -1
    assert lib.fdllm_probe_lds_dma(P(16), 1024, 0, 9, 16, P(16), None) == -1
    assert lib.fdllm_probe_lds_dma(P(16), 1024, 0, 4, 0, P(16), None) == -1
    assert lib.fdllm_probe_lds_dma(P(24), 1024, 0, 4, 16, P(16), None) == -3


def test_noalloc_step_host_side_errors(lib):
    """The allocation-free step validates its arguments and sizes its
    workspace against the static scratch before any HIP call."""
    P = ctypes.c_void_p
    a = [P(16)] * 2
    def call(cfg, nq, x_rows=64):
        return lib.fdllm_fused_step_noalloc(ctypes.byref(cfg) if cfg is not None else None, P(16), x_rows, P(16),
                                            P(16), nq, None, P(16), P(16), P(16), P(16), P(16), None)
    assert call(None, 1) == -1
    assert call(_cfg(H=3), 1) == -1
    assert call(_cfg(), 9) == -2                 # nq > q_max
    assert call(_cfg(), 1, x_rows=0) == -2
    assert call(_cfg(), 0) == 0                  # nothing to do
    # a workspace larger than the 64 MiB scratch: q staging alone is
    # B*Hkv*nq*G*dh*4 = 64*32*64*128*4 bytes = 64 MiB, plus the rest
    big = _cfg(B=64, N=4096, d_model=256, H=32, Hkv=32, dh=128, q_max=64)
    assert call(big, 64) == -8
    assert lib.fdllm_status_str(-8).decode().startswith("FDLLM_ERR_SCRATCH")


def test_binding_refuses_cpu_tensors():
    with pytest.raises(ValueError):
        binding._ptr(torch.zeros(4))
