"""The element-wise check of the stored k/v rows on full-significand inputs
(parity_util.check_written_rows_faithful) accepts an honest fp32 evaluation
of the projection and rotation and rejects the mistakes it is there to catch:
an operand with its low significand bits dropped, and a store that truncates
instead of rounding to nearest even.  The fp32 evaluation here is an
independent emulation on the CPU (a torch fp32 matmul, an fp32 rotation),
not the HIP path and not the oracle."""
import math

import numpy as np
import pytest
import torch

from io_aware_kv_amd.workloads import LayerShape, initial_cache, make_random_case
from parity_util import check_written_rows_faithful, run_oracle


def _truncate_bits(t, bits):
    """bf16 tensor with the lowest `bits` significand bits cleared."""
    i = t.contiguous().view(torch.int16)
    return (i & ~((1 << bits) - 1)).to(torch.int16).view(torch.bfloat16)


def _fp32_step_rows(wl, X, store):
    """Emulated device cache after the step: k/v of the owner rows from an fp32
    projection and rotation, stored by `store` (fp32 -> bf16)."""
    ls = wl.shape
    H, Hkv, dh = ls.H, ls.Hkv, ls.dh
    half = dh // 2
    K0, V0 = initial_cache(wl)
    K1, V1 = K0.clone(), V0.clone()
    W = wl.W.float()
    e = torch.arange(half, dtype=torch.float64)
    theta = ls.rope_base ** (-2.0 * e / dh)
    for b in range(ls.B):
        seen = set()
        for j in range(wl.nq):
            p = int(wl.pos_ids[b, j])
            if p in seen:
                continue
            seen.add(p)
            x = X[b, int(wl.Q_idx[b, j])].float()
            y = W @ x
            k = y[H * dh:(H + Hkv) * dh].reshape(Hkv, dh)
            v = y[(H + Hkv) * dh:].reshape(Hkv, dh)
            c = torch.cos(p * theta).float()
            s = torch.sin(p * theta).float()
            a, bb = k[:, :half], k[:, half:]
            kr = torch.cat([a * c - bb * s, bb * c + a * s], dim=-1)
            K1[b, :, p] = store(kr)
            V1[b, :, p] = store(v)
    return {"K0": K0, "V0": V0, "K1": K1, "V1": V1}


def _rne(x):
    return x.to(torch.bfloat16)


def _rtz(x):
    """fp32 -> bf16 by dropping the low 16 bits (round toward zero)."""
    i = x.contiguous().view(torch.int32) & ~0xFFFF
    return (i >> 16).to(torch.int16).view(torch.bfloat16)


@pytest.fixture(scope="module")
def case():
    ls = LayerShape(B=2, N=96, d_model=1024, H=4, Hkv=2, dh=128)
    wl = make_random_case(ls, 24, seed=123, n_extra_rows=4, dup_frac=0.15)
    assert not wl.meta["grid"]
    return wl, run_oracle(wl)


def test_inputs_use_the_full_bf16_significand(case):
    wl, _ = case
    low = (wl.X.view(torch.int16) & 1).double().mean().item()
    assert 0.4 < low < 0.6          # about half the elements have the last bit set


def test_honest_fp32_evaluation_passes(case):
    wl, r = case
    g = _fp32_step_rows(wl, wl.X, _rne)
    n_el, n_other = check_written_rows_faithful(wl, g, r, "fp32-emulation")
    assert n_el > 0 and n_other <= 0.01 * n_el


@pytest.mark.parametrize("bits", [1, 2])
def test_dropped_operand_bits_fail(case, bits):
    wl, r = case
    g = _fp32_step_rows(wl, _truncate_bits(wl.X, bits), _rne)
    with pytest.raises(AssertionError):
        check_written_rows_faithful(wl, g, r, "dropped-%d-bits" % bits)


def test_truncating_store_fails(case):
    wl, r = case
    g = _fp32_step_rows(wl, wl.X, _rtz)
    with pytest.raises(AssertionError):
        check_written_rows_faithful(wl, g, r, "truncating-store")
