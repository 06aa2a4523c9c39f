"""The achievable-rate probes on the GPU: they run through the C ABI, leave their sink
word untouched, report the launch's flops exactly, and give rates within physical
bounds of an MI355X (a read sweep below the 8 TB/s HBM peak once the buffer is far
larger than the caches, MFMA work below the 2.5 PFLOP/s bf16 peak at 2.4 GHz)."""
import pytest
import torch

import mtp_draft_verification_amd as mv

pytestmark = pytest.mark.gpu


def _median_s(fn, reps=3):
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / 1e3)
    return sorted(ts)[len(ts) // 2]


def test_read_probe_rate_and_sink():
    dev = torch.device("cuda:0")
    nbytes = 2 << 30  # 2 GiB: eight times the Infinity Cache
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.full((4,), 7, dtype=torch.int32, device=dev)
    mv.read_bytes(buf, nbytes, sink)
    t = _median_s(lambda: mv.read_bytes(buf, nbytes, sink))
    gbs = nbytes / t / 1e9
    print(f"read probe: {gbs:.1f} GB/s over {nbytes} bytes", flush=True)
    assert 1000.0 < gbs < 8000.0
    mv.read_bytes(buf, 16, sink)  # a single 16-byte chunk
    torch.cuda.synchronize()
    assert sink.tolist() == [7, 7, 7, 7]


def test_mfma_probe_flops_rate_and_sink():
    dev = torch.device("cuda:0")
    sink = torch.full((4,), 7, dtype=torch.int32, device=dev)
    iters = 256
    flops = mv.mfma_rate(iters, sink)
    assert flops == 256 * 4 * iters * 16 * 16 * 16 * 32 * 2
    t = _median_s(lambda: mv.mfma_rate(iters, sink))
    tflops = flops / t / 1e12
    print(f"mfma probe: {tflops:.1f} TFLOP/s", flush=True)
    assert 200.0 < tflops < 2520.0
    torch.cuda.synchronize()
    assert sink.tolist() == [7, 7, 7, 7]
