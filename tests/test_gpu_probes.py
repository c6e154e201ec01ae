"""The two rate probes of the device (include/spa_probe.h), through the C ABI: each runs, leaves its
sink untouched, and reports a rate that is positive and no higher than the vendor peak allows
(1 GiB read from HBM at most 8 TB/s, bf16 MFMAs at most 2.5 PFLOP/s, each with 10 % slack for
clock and timer granularity).  The measured rates themselves are reported by bench.py."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def S():
    import block_sparse_long_int8_amd as mod
    mod.lib()
    return mod


def _time(fn):
    fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    fn()
    b.record()
    b.synchronize()
    return a.elapsed_time(b) * 1e-3


def test_probe_read_rate(S):
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = 1 << 30
    buf = torch.full((nbytes,), 7, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    t = _time(lambda: S.spa_probe_read(buf, 8 * n_cu, sink))
    gbs = nbytes / t / 1e9
    print(f"[probe] read {gbs:.0f} GB/s")
    assert 100.0 < gbs < 8800.0
    assert int(sink.item()) == 0
    # a size that is not a whole number of grid strides, on a small grid
    tail = buf[: (1 << 20) + 48]
    S.spa_probe_read(tail, 3, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_probe_mfma_rate(S):
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    flops = []
    t = _time(lambda: flops.append(S.spa_probe_mfma_bf16(2 * n_cu, 1024, sink)))
    tflops = flops[-1] / t / 1e12
    print(f"[probe] bf16 MFMA {tflops:.0f} TFLOP/s")
    assert flops[-1] == 2 * n_cu * 4 * 1024 * 131072
    assert 10.0 < tflops < 2750.0
    assert float(sink.item()) == 0.0


def test_probe_binding_rejects(S):
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        S.spa_probe_read(torch.zeros(16, dtype=torch.uint8), 1, sink)  # host buffer
    with pytest.raises(ValueError):
        S.spa_probe_mfma_bf16(1, 1, sink)  # int32 sink where a float is written
    with pytest.raises(S.SpaError):
        S.spa_probe_read(torch.zeros(24, dtype=torch.uint8, device="cuda"), 1, sink)  # not a multiple of 16
