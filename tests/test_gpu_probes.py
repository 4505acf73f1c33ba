"""The library's measurement probes run on the device and give rates in a
plausible range (positive, below the chip's published peaks by no more than a
margin for clock variation)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def _time(fn, reps=3):
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e-3


def test_rate_probes_run():
    from io_aware_kv_amd import binding
    dev = torch.device("cuda")
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    print("case: probes read, mfma, lds-dma", flush=True)
    buf = torch.ones(64 << 20, dtype=torch.uint8, device=dev)
    s = _time(lambda: binding.probe_read(buf, sink))
    read = buf.numel() / s / 1e9
    s = _time(lambda: binding.probe_mfma(sink, 256, 4, 1024))
    tflops = 256 * 4 * 1024 * 8 * 16384 / s / 1e12
    small = torch.ones(2 << 20, dtype=torch.uint8, device=dev)
    s = _time(lambda: binding.probe_lds_dma(small, sink, 256, 4, 1024))
    dma = 256 * 4 * 1024 * 1024 / s / 1e9
    print("read %.0f GB/s, mfma %.0f TFLOP/s, lds-dma %.0f GB/s" % (read, tflops, dma))
    assert 100 < read < 9000
    assert 100 < tflops < 2800
    assert 100 < dma
    assert int(sink.abs().sum()) == 0          # the sinks are never written on ordinary data
