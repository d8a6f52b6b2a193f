"""The ceiling kernels run and report rates that a real read and a real MFMA
loop can give: above a floor that only a broken launch misses, and not above
MI355X's published peaks (8 TB/s HBM3E, 2.5 PFLOP/s dense bf16), which a
kernel that skipped its work would exceed."""
import pytest

from block_sparse_gqa_amd import msa

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def timed(fn, reps):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    e0.record()
    work = sum(fn() for _ in range(reps))
    e1.record()
    torch.cuda.synchronize()
    return work / (e0.elapsed_time(e1) * 1e-3)


@pytest.mark.timeout(120)
def test_stream_read_rate():
    buf = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    nbytes = msa.msa_ceiling_stream_read(buf, sink)
    assert 0.9 * buf.numel() < nbytes <= buf.numel()
    rate = timed(lambda: msa.msa_ceiling_stream_read(buf, sink), 5) / 1e9
    print(f"stream read {rate:.0f} GB/s", flush=True)
    assert 1000 < rate < 8200
    assert int(sink.item()) == 0   # all-ones data never matches the sink pattern


@pytest.mark.timeout(120)
def test_mfma_loop_rate():
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    rate = timed(lambda: msa.msa_ceiling_mfma_bf16(8192, sink), 3) / 1e12
    print(f"mfma bf16 {rate:.0f} TFLOP/s", flush=True)
    assert 300 < rate < 2600
