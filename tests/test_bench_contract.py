"""The measurement harness's host-side contract, on the CPU: the algorithmic
bytes and flops that the roofline figures divide by, written out here from
the layer shapes (weights once, the gathered X rows, one new k/v row per
distinct position, one full K and V read, O and LSE, mask and indices), and
the refusal of a multi-GPU run."""
import os
import subprocess
import sys

import pytest

import bench
from io_aware_kv_amd.workloads import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("cid", [2, 3, 4])
def test_algorithmic_bytes_from_the_shapes(cid):
    wl = make_workload(cid)
    ls = wl.shape
    B, N, d, H, Hkv, dh, nq = ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, wl.nq
    e = 2                                                  # bf16 layers
    distinct = sum(len(set(wl.pos_ids[b].tolist())) for b in range(B))
    weights = (H + 2 * Hkv) * dh * d * e
    xrows = B * nq * d * e
    kv_new = distinct * Hkv * dh * 2 * e
    kv_all = B * Hkv * N * dh * 2 * e
    o_lse = B * nq * H * (dh * e + 4)
    mask = B * nq * nq if wl.vis is not None else 0
    ab = bench.algorithmic_bytes(wl)
    assert ab["total"] == weights + xrows + kv_new + kv_all + o_lse + mask + 2 * B * nq * 4
    # the attention phase: K/V once, O and LSE, the mask and the positions
    assert ab["attn"] == kv_all + o_lse + mask + B * nq * 4
    assert ab["qkv_flops"] == 2 * B * nq * d * (H + 2 * Hkv) * dh
    # scores, then P V: 2 flops per multiply-add over every key and head dim
    assert ab["attn_flops"] == 2 * 2 * B * nq * H * N * dh


def test_step_sizes_of_the_verification_layer():
    """The verification layer's figures in MB as stated beside its shapes
    (B=8, N=2048, d=4096, H=Hkv=32, |Q|=44 with 28 distinct positions)."""
    ab = bench.algorithmic_bytes(make_workload(3))
    assert ab["total"] == pytest.approx(378.6e6, rel=2e-3)
    assert ab["attn"] == pytest.approx(271.4e6, rel=2e-3)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.gpu
def test_bench_json_line_on_the_gpu():
    """A short run of the default workload prints one JSON line with the
    contract's fields, a roofline object for the dominant kernel and the
    CPU oracle's baseline."""
    import json
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5", "--warmup", "2",
                        "--no-select", "--cpu-budget", "1"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["dtype"] == "bf16"
    assert "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma") and rf["unit"] in ("GB/s", "TFLOP/s")
    assert 0 < rf["frac"] <= 1 and rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-3)
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert d["device_read_GBps"] > 0 and d["device_copy_GBps"] > 0
    assert d["host_submit_us_per_step"] > 0
    assert d["graph_step_us"] > 0
    # the other workloads of the target set: step and phase figures of each
    assert set(d["configs"]) == {"workload1", "workload2", "workload4"}
    for c in d["configs"].values():
        for key in ("workload", "step_us", "graph_step_us", "proj_us", "attn_us", "attn_hbm_frac", "proj_roofline",
                    "plan"):
            assert key in c, key
        assert c["step_us"] > 0 and 0 < c["attn_hbm_frac"] < 1
