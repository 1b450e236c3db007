"""qkr_read_probe and qkr_mfma_probe (measurement helpers outside the attention
path) through the C ABI: they run and leave the output alone."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_read_probe_reads_and_writes_nothing():
    import qk_norm_rope_amd as Q
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    buf = torch.ones(3 * 1024 * 1024 + 4, dtype=torch.float32, device="cuda")   # not a multiple of the grid's step
    out = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    Q.read_probe(buf, out)
    torch.cuda.synchronize()
    assert float(out) == 7.0
    with pytest.raises(Q.QknrError):
        Q.read_probe(buf[1:], out)   # 4-byte offset: misaligned


def test_mfma_probe_counts_its_flops_and_writes_nothing():
    import qk_norm_rope_amd as Q
    out = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    flops = Q.mfma_probe(3, out)
    torch.cuda.synchronize()
    assert flops == cus * 8 * 3 * 8 * 32 * 32 * 16 * 2
    assert float(out) == 7.0
